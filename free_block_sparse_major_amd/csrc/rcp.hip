// Response-coupled partitioning: the query and key/value groups of one
// attention call, built from its own activations.
//
// SparsePR paper §4.1 (key-response coordinates for paired K/V groups,
// query-response coordinates from K/V groups), App. B.1 (key response
// metric), App. B.2 (query response metric, RMS normalisation with floor
// 1e-6) and App. C.1 (clustering on the GPU, initial centres sampled from
// the feature rows; metric construction, centroid statistics and the
// factorisation in FP32).  Per head:
//   1. M_K = Q_s^T Q_s / M_s over M_s evenly spaced query rows (fp32).
//   2. F_K: the leading r_K eigenvectors of M_K (fp64: Householder reduction
//      to tridiagonal form, bisection, twisted factorisations; the pages do
//      this step in FP32), each scaled by the square root of its eigenvalue
//      over the mean of the r_K retained (eigenvalues clamped at 0).
//   3. phi_K = k F_K, held as a bf16 pair (hi = bf16(phi), lo = bf16(phi - hi)).
//   4. Lloyd's k-means with C_k centres started at the rows init_k: the
//      assignment is an MFMA product |c|^2 - 2 x.c with x.c taken as
//      hi.hi + hi.lo + lo.hi (fp32 accumulation), ties to the smaller centre;
//      the update is each cluster's mean in row order after a stable counting
//      sort of the labels (an empty cluster keeps its centre).  The labels
//      are those of the last assignment.
//   5. K/V group centroids in the original key space (fp32, row order), their
//      mean over the non-empty groups subtracted: M_Q = K~^T K~ / C_nonempty.
//   6. F_Q from M_Q as in 2 (r_Q); phi_Q = u / max(RMS(u), 1e-6), u = q F_Q.
//   7. k-means on phi_Q with C_q centres from init_q -> query labels.
//
// Later calls of the same layer (App. C.1) start from the state an earlier
// call left: the factors come from two subspace iterations started at the
// previous orthonormal bases (fp64, Cholesky orthonormalisation, directions
// weighted by their Rayleigh quotients), and k-means starts from the previous
// group centroids in the original space mapped by the current coordinates.
// The state written back is the bases and each group's mean in the original
// space (an empty group keeps its previous centroid; on a first call, its
// initial row).

#include <utility>

#include "common.h"
#include "f64_lanes.h"

namespace spr {

size_t group_sort_ws_bytes(int heads, int n, int c);
int32_t group_sort(const int32_t* labels, int heads, int n, int c, int32_t* perm,
                   int32_t* offsets, void* ws, hipStream_t stream);

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kMaxR = 64;          // padded coordinate rank (multiple of 16)
constexpr int kMetricRows = 32;    // rows staged per metric step

SPR_DEV float load_elem(const void* x, int dtype, long long off) {
  return dtype == SPARSEPR_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(x)[off])
                                : static_cast<const float*>(x)[off];
}

// ---------------------------------------------------------------------------
// metrics
// ---------------------------------------------------------------------------
// Thread t owns entries (a, b) with b = t % D and a = t / D + (256 / D) i; the
// sum over rows runs in row order.
template <int D>
SPR_DEV void metric_accumulate(float (&xs)[kMetricRows][D + 1], int rows, float* acc) {
  constexpr int NE = D * D / 256, AS = 256 / D;
  const int b = threadIdx.x % D, a0 = threadIdx.x / D;
  for (int rr = 0; rr < rows; ++rr) {
    const float xb = xs[rr][b];
#pragma unroll
    for (int i = 0; i < NE; ++i) acc[i] = fmaf(xs[rr][a0 + AS * i], xb, acc[i]);
  }
}

template <int D>
SPR_DEV void metric_store(const float* acc, float scale, float* m) {
  constexpr int NE = D * D / 256, AS = 256 / D;
  const int b = threadIdx.x % D, a0 = threadIdx.x / D;
#pragma unroll
  for (int i = 0; i < NE; ++i) m[(a0 + AS * i) * D + b] = acc[i] * scale;
}

// M_K of head blockIdx.x from rows floor(i * n / m_s) of q (every row if n <= m_s).
template <int D>
__global__ __launch_bounds__(256) void key_metric_kernel(const void* q, int dtype, long long sh,
                                                         long long st, int n, int m_s,
                                                         float* __restrict__ mk) {
  const int h = blockIdx.x;
  __shared__ float xs[kMetricRows][D + 1];
  const int ms = n < m_s ? n : m_s;
  float acc[D * D / 256];
#pragma unroll
  for (int i = 0; i < D * D / 256; ++i) acc[i] = 0.f;
  for (int r0 = 0; r0 < ms; r0 += kMetricRows) {
    __syncthreads();
    for (int e = threadIdx.x; e < kMetricRows * D; e += 256) {
      const int rr = e / D, j = e % D, i = r0 + rr;
      float v = 0.f;
      if (i < ms) {
        const long long row = n <= m_s ? i : (long long)i * n / m_s;
        v = load_elem(q, dtype, h * sh + row * st + j);
      }
      xs[rr][j] = v;
    }
    __syncthreads();
    metric_accumulate<D>(xs, min(kMetricRows, ms - r0), acc);
  }
  metric_store<D>(acc, 1.f / float(ms), mk + (long long)h * D * D);
}

// M_Q of head blockIdx.x from the K/V group centroids (empty groups skipped).
template <int D>
__global__ __launch_bounds__(256) void query_metric_kernel(const float* __restrict__ cent,
                                                           const int32_t* __restrict__ offsets,
                                                           int c, float* __restrict__ mq) {
  const int h = blockIdx.x;
  __shared__ float xs[kMetricRows][D + 1];
  __shared__ int32_t nzl[SPARSEPR_MAX_GROUPS];
  __shared__ float mu[D];
  __shared__ int32_t s_nnz;
  const int32_t* off = offsets + (long long)h * (c + 1);
  const float* ce = cent + (long long)h * c * D;
  {
    // non-empty groups in ascending order: 4 groups per thread, block scan
    __shared__ long long red[4];
    const int b0 = 4 * threadIdx.x;
    bool ne[4];
    long long cnt = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      ne[u] = b0 + u < c && off[b0 + u + 1] > off[b0 + u];
      cnt += ne[u] ? 1 : 0;
    }
    long long tot;
    long long pos = block_exclusive_scan(cnt, red, &tot);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ne[u]) nzl[pos++] = b0 + u;
    if (threadIdx.x == 0) s_nnz = int(tot);
  }
  __syncthreads();
  const int nnz = s_nnz;
  if (threadIdx.x < D) {
    float s = 0.f;
    for (int i = 0; i < nnz; ++i) s += ce[(long long)nzl[i] * D + threadIdx.x];
    mu[threadIdx.x] = s / float(nnz);
  }
  float acc[D * D / 256];
#pragma unroll
  for (int i = 0; i < D * D / 256; ++i) acc[i] = 0.f;
  for (int r0 = 0; r0 < nnz; r0 += kMetricRows) {
    __syncthreads();
    for (int e = threadIdx.x; e < kMetricRows * D; e += 256) {
      const int rr = e / D, j = e % D, i = r0 + rr;
      xs[rr][j] = i < nnz ? ce[(long long)nzl[i] * D + j] - mu[j] : 0.f;
    }
    __syncthreads();
    metric_accumulate<D>(xs, min(kMetricRows, nnz - r0), acc);
  }
  metric_store<D>(acc, 1.f / float(nnz > 0 ? nnz : 1), mq + (long long)h * D * D);
}

constexpr int kEigThreads = 1024;

// ---------------------------------------------------------------------------
// eigenvalue-weighted factor (fp64 tridiagonal eigensolver)
// ---------------------------------------------------------------------------
// The r leading eigenpairs of the symmetric D x D metric in fp64, one block of
// kEigThreads threads per head (r <= 64):
//   a. Householder reduction to tridiagonal form T = Q^T M Q.  Thread t keeps
//      row t / RT, columns CW (t % RT) .. + CW - 1 of the matrix in
//      registers.  Step k publishes column k through LDS, every wave forms
//      v = x - alpha e_1 and beta = 2 / |v|^2 from it, the rows form
//      p = beta A v, and the rank-2 update A -= v w^T + w v^T with
//      w = p - (beta / 2)(p.v) v follows (two barriers per step).  v is kept
//      in fp32 for the back-transformation;
//   b. the r largest eigenvalues of T by multisection of Sturm counts (T
//      normalised by its Gershgorin bound);
//   c. each eigenvector of T from the twisted factorisation of T - lambda I
//      (the twist where |gamma| is smallest).  If the vectors are not
//      orthogonal to 1e-10 (close eigenvalues), they are re-orthogonalised
//      in descending order, and a vector that loses more than half its norm
//      is recomputed by inverse iteration kept orthogonal to the earlier ones;
//   d. U = H_0 ... H_(D-3) Z, 16 lanes per vector (no barriers).
// Output: F[h] (D x rp), column c < r = eigenvector of
// the c-th largest eigenvalue times sqrt(max(lambda, 0) / mean of the r
// retained); basis[h] (D x r) the eigenvectors themselves.
template <int D>
__global__ __launch_bounds__(kEigThreads) void eig_tri_kernel(const float* __restrict__ m, int r,
                                                              int rp, float* __restrict__ f,
                                                              float* __restrict__ basis) {
  constexpr int NT = kEigThreads, RT = NT / D, CW = D / RT, NV = D * (D - 1) / 2;
  constexpr int EPL = D / 64;   // vector elements per lane in one-wave steps
  constexpr int TB = 32;        // targets per batch of the twisted factorisation
  constexpr int GV = 16, RPV = D / GV;   // back-transformation: lanes and rows per vector
  static_assert(NT == 1024 && (D == 64 || D == 128), "layout assumes 1024 threads");
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ double colb[2][D], pbf[2][D];
  __shared__ double td[D], te[D], tb[D], tdn[D], ten[D];
  __shared__ double2 st2[D];
  __shared__ double lamn[64];
  __shared__ double red[NT / 64];
  __shared__ double tbuf[D];
  __shared__ float V[NV];
  __shared__ double Z[64][D];
  __shared__ double W[TB][D];
  constexpr int n = D;
  const int rr = tid / RT, qq = tid % RT, c0 = CW * qq;
  const float* mh = m + (long long)h * D * D;
  double er[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int j = c0 + i;
    er[i] = 0.5 * (double(mh[rr * D + j]) + double(mh[j * D + rr]));
  }
  auto voff = [](int k) { return k * (2 * D - k - 1) / 2; };
  // a. Householder steps k = 0 .. n - 3 (register index KI compile-time)
  auto hh_step = [&](auto ki_c, int kb) __attribute__((always_inline)) {
    constexpr int KI = decltype(ki_c)::value;
    const int k = CW * kb + KI;
    const int par = KI & 1;
    if (qq == kb) colb[par][rr] = er[KI];
    __syncthreads();
    double xs[EPL];
    double ss = 0.0;
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
      const int idx = k + 1 + lane + 64 * e;
      xs[e] = idx < n ? colb[par][idx] : 0.0;
      ss = fma(xs[e], xs[e], ss);
    }
    const double nx2 = wave_sum_f64(ss);
    const double x0 = colb[par][k + 1];
    double alpha = 0.0, beta = 0.0;
    if (nx2 > 0.0) {
      const double nx = sqrt(nx2);
      alpha = x0 > 0.0 ? -nx : nx;
      beta = rcp64(nx2 - alpha * x0);   // 2 / |v|^2, |v|^2 = 2 (|x|^2 - alpha x0)
    }
    if (wid == 0) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int idx = k + 1 + lane + 64 * e;
        if (idx < n) V[voff(k) + idx - k - 1] = float(idx == k + 1 ? xs[e] - alpha : xs[e]);
      }
      if (lane == 0) {
        td[k] = colb[par][k];
        te[k] = alpha;
        tb[k] = beta;
      }
    }
    double vj[CW];
#pragma unroll
    for (int i = 0; i < CW; ++i) {
      const int j = c0 + i;
      const double cj = colb[par][j];
      vj[i] = j > k ? (j == k + 1 ? cj - alpha : cj) : 0.0;
    }
    if (beta != 0.0) {
      double s2 = 0.0;
#pragma unroll
      for (int i = 0; i < CW; ++i) s2 = fma(er[i], vj[i], s2);
      s2 = group_sum_f64<RT>(s2);
      if (qq == 0 && rr > k) pbf[par][rr] = beta * s2;
    }
    __syncthreads();
    if (beta != 0.0) {
      double ps = 0.0;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const int idx = k + 1 + lane + 64 * e;
        if (idx < n) ps = fma(pbf[par][idx], idx == k + 1 ? xs[e] - alpha : xs[e], ps);
      }
      const double K = 0.5 * beta * wave_sum_f64(ps);
      if (rr > k) {
        const double cr = colb[par][rr];
        const double vr = rr == k + 1 ? cr - alpha : cr;
        const double wr = pbf[par][rr] - K * vr;
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          const int j = c0 + i;
          if (j > k) {
            const double wj = pbf[par][j] - K * vj[i];
            er[i] -= fma(vr, wj, wr * vj[i]);
          }
        }
      }
    }
  };
  for (int kb = 0; kb * CW < n - 2; ++kb) {
    [&]<int... KI>(std::integer_sequence<int, KI...>) {
      ((CW * kb + KI < n - 2 ? hh_step(std::integral_constant<int, KI>{}, kb) : void()), ...);
    }(std::make_integer_sequence<int, CW>{});
  }
  // the last 2 x 2 block of T
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int j = c0 + i;
    if (rr == n - 2 && j == n - 2) td[n - 2] = er[i];
    if (rr == n - 1 && j == n - 2) te[n - 2] = er[i];
    if (rr == n - 1 && j == n - 1) td[n - 1] = er[i];
  }
  if (tid == 0) {
    te[n - 1] = 0.0;
    tb[n - 2] = 0.0;
    tb[n - 1] = 0.0;
  }
  __syncthreads();
  const int cap = r < 64 ? (r < n ? r : n) : 64;
  // b. Gershgorin bounds; T normalised by tn = max |bound|
  double glo = __builtin_huge_val(), ghi = -__builtin_huge_val();
  if (tid < n) {
    const double rad = (tid > 0 ? fabs(te[tid - 1]) : 0.0) + (tid + 1 < n ? fabs(te[tid]) : 0.0);
    glo = td[tid] - rad;
    ghi = td[tid] + rad;
  }
  glo = block_min(glo, red);
  ghi = block_max(ghi, red);
  const double tn = fmax(fabs(glo), fabs(ghi));
  if (tid < 64) lamn[tid] = 0.0;
  if (!(tn > 0.0)) {
    // zero metric: every eigenvalue 0, unit vectors
    for (int e = tid; e < 64 * n; e += NT) Z[e / n][e % n] = (e / n) == (e % n) ? 1.0 : 0.0;
    __syncthreads();
  } else {
    if (tid < n) {
      const double inv = 1.0 / tn;
      tdn[tid] = td[tid] * inv;
      const double en = te[tid] * inv;
      ten[tid] = en;
      if (tid + 1 < n) st2[tid] = double2{td[tid + 1] * inv, en * en};
    }
    __syncthreads();
    const double lo0 = glo / tn - 4.0 * kEps64, hi0 = ghi / tn + 4.0 * kEps64;
    int P = 64;
    while (P > 1 && P * cap > 256) P >>= 1;   // waves 0..3: one per SIMD
    const int j = tid / P, s = tid % P;
    const bool act = j < cap;
    const int target = n - 1 - j;       // ascending index of the j-th largest
    const double d0 = tdn[0];
    double a = lo0, b = hi0;
    for (int round = 0; round < 40; ++round) {
      const bool done = !act || (b - a) <= 2.0 * kEps64 * fmax(fabs(a), fabs(b)) + 4.0 * kEps64;
      if (__all(done)) break;
      const double x1 = a + (b - a) * (double(2 * s + 1) / double(2 * P + 1));
      const double x2 = a + (b - a) * (double(2 * s + 2) / double(2 * P + 1));
      int c1 = 0, c2 = 0;
      if (act) sturm_count2(d0, st2, n, x1, x2, c1, c2);
      double na = c2 <= target ? x2 : (c1 <= target ? x1 : a);
      double nb = c1 > target ? x1 : (c2 > target ? x2 : b);
      for (int o = 1; o < P; o <<= 1) {
        na = fmax(na, __shfl_xor(na, o));
        nb = fmin(nb, __shfl_xor(nb, o));
      }
      a = na;
      b = nb;
    }
    if (act && s == 0) lamn[j] = 0.5 * (a + b);
    __syncthreads();
    // c. twisted factorisation, one thread per target, TB targets at a time:
    // forward pivots Dp (in W), ratios e_i / Dp_i (in Z); backward pivots Dm
    // with gamma_i = Dp_i + Dm_i - (d_i - mu), ratios e_(i-1) / Dm_i (in W)
    for (int b0 = 0; b0 < cap; b0 += TB) {
      if (tid < TB && b0 + tid < cap) {
        const int c = b0 + tid;
        const double mu = lamn[c];
        double* zr = Z[c];
        double* wr = W[tid];
        double dp = tdn[0] - mu;
        wr[0] = dp;
        for (int i = 1; i < n; ++i) {
          const double2 s2 = st2[i - 1];
          const double ri = rcp64(fabs(dp) < kTiny ? -kTiny : dp);
          zr[i - 1] = ten[i - 1] * ri;
          dp = (s2.x - mu) - s2.y * ri;
          wr[i] = dp;
        }
        double dm = tdn[n - 1] - mu;
        double gbest = fabs(wr[n - 1]);
        int rt = n - 1;
        for (int i = n - 2; i >= 0; --i) {
          const double ri = rcp64(fabs(dm) < kTiny ? -kTiny : dm);
          const double dpi = wr[i];
          const double ei = ten[i];
          wr[i + 1] = ei * ri;
          const double ai = tdn[i] - mu;
          dm = ai - ei * ei * ri;
          const double g = fabs(dpi + dm - ai);
          if (g < gbest) {
            gbest = g;
            rt = i;
          }
        }
        double z = 1.0, nrm = 1.0;
        for (int i = rt - 1; i >= 0; --i) {
          z = -zr[i] * z;
          zr[i] = z;
          nrm = fma(z, z, nrm);
        }
        zr[rt] = 1.0;
        z = 1.0;
        for (int i = rt + 1; i < n; ++i) {
          z = -wr[i] * z;
          zr[i] = z;
          nrm = fma(z, z, nrm);
        }
        const double sc_n = 1.0 / sqrt(nrm);
        for (int i = 0; i < n; ++i) zr[i] *= sc_n;
      }
      __syncthreads();
    }
    // orthogonality of the computed vectors
    double worst = 0.0;
    for (int e = tid; e < cap * cap; e += NT) {
      const int c1 = e / cap, c2 = e - c1 * cap;
      if (c2 <= c1) {
        double dot = 0.0;
        for (int i = 0; i < n; ++i) dot = fma(Z[c1][i], Z[c2][i], dot);
        const double dev = c2 == c1 ? fabs(dot - 1.0) : fabs(dot);
        worst = dev == dev ? fmax(worst, dev) : 1.0;   // NaN counts as lost
      }
    }
    worst = block_max(worst, red);
    if (!(worst <= 1e-10) && wid == 0) {
      // rare: classical Gram-Schmidt twice in descending order; a vector that
      // loses more than half its norm is recomputed by inverse iteration
      // (LU of T - mu I without pivoting, tiny pivots raised) kept orthogonal
      // to the earlier ones.  Lanes hold EPL elements each.
      for (int c = 0; c < cap; ++c) {
        double zi[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          zi[e] = Z[c][lane + 64 * e];
          if (!(zi[e] == zi[e])) zi[e] = 0.0;
        }
        auto orth = [&]() {
          for (int pass = 0; pass < 2; ++pass)
            for (int c2 = 0; c2 < c; ++c2) {
              double dd = 0.0;
#pragma unroll
              for (int e = 0; e < EPL; ++e) dd = fma(Z[c2][lane + 64 * e], zi[e], dd);
              dd = wave_sum_f64(dd);
#pragma unroll
              for (int e = 0; e < EPL; ++e) zi[e] -= dd * Z[c2][lane + 64 * e];
            }
        };
        auto norm = [&]() {
          double q = 0.0;
#pragma unroll
          for (int e = 0; e < EPL; ++e) q = fma(zi[e], zi[e], q);
          return sqrt(wave_sum_f64(q));
        };
        orth();
        double nz = norm();
        if (!(nz >= 0.5)) {
          const double mu = lamn[c];
#pragma unroll
          for (int e = 0; e < EPL; ++e) {
            uint32_t hsh = uint32_t((lane + 64 * e) * 2654435761u) ^ uint32_t((c + 1) * 40503u);
            hsh ^= hsh >> 13;
            hsh *= 0x5bd1e995u;
            hsh ^= hsh >> 15;
            zi[e] = double(int32_t(hsh & 0xffff) - 32768);
          }
          for (int it = 0; it < 4; ++it) {
            orth();
#pragma unroll
            for (int e = 0; e < EPL; ++e) W[0][lane + 64 * e] = zi[e];
            if (lane == 0) {
              double* y = W[0];
              double u_prev = tdn[0] - mu;
              if (fabs(u_prev) < kEps64) u_prev = kEps64;
              tbuf[0] = u_prev;
              for (int i = 1; i < n; ++i) {
                const double l = ten[i - 1] / u_prev;
                double u = (tdn[i] - mu) - l * ten[i - 1];
                if (fabs(u) < kEps64) u = kEps64;
                y[i] -= l * y[i - 1];
                tbuf[i] = u;
                u_prev = u;
              }
              y[n - 1] /= tbuf[n - 1];
              for (int i = n - 2; i >= 0; --i) y[i] = (y[i] - ten[i] * y[i + 1]) / tbuf[i];
            }
#pragma unroll
            for (int e = 0; e < EPL; ++e) zi[e] = W[0][lane + 64 * e];
            const double nn = norm();
#pragma unroll
            for (int e = 0; e < EPL; ++e) zi[e] = nn > 0.0 ? zi[e] / nn : 0.0;
          }
          orth();
          nz = norm();
        }
#pragma unroll
        for (int e = 0; e < EPL; ++e) Z[c][lane + 64 * e] = nz > 0.0 ? zi[e] / nz : 0.0;
      }
    }
    __syncthreads();
  }
  // d. U = H_0 ... H_(n-3) Z: vector c on lanes GV c .. + GV - 1, rows g + GV u
  const int c = tid / GV, g = tid % GV;
  double z[RPV];
#pragma unroll
  for (int u = 0; u < RPV; ++u) z[u] = c < cap ? Z[c][g + GV * u] : 0.0;
  if (tn > 0.0) {
    for (int k = n - 3; k >= 0; --k) {
      const double beta = tb[k];
      if (beta == 0.0) continue;
      const float* vk = V + voff(k) - (k + 1);   // vk[i] = v_i, i > k
      double dot = 0.0;
#pragma unroll
      for (int u = 0; u < RPV; ++u) {
        const int i = g + GV * u;
        if (i > k) dot = fma(double(vk[i]), z[u], dot);
      }
      dot = beta * group_sum_f64<GV>(dot);
#pragma unroll
      for (int u = 0; u < RPV; ++u) {
        const int i = g + GV * u;
        if (i > k) z[u] = fma(-dot, double(vk[i]), z[u]);
      }
    }
  }
  // scale: mean of the r retained eigenvalues (clamped at 0)
  double mean = 0.0;
  for (int i = 0; i < cap; ++i) mean += fmax(lamn[i] * tn, 0.0);
  mean /= double(r > 0 ? r : 1);
  float* fh = f + (long long)h * D * rp;
  if (c < cap) {
    const double sc = mean > 0.0 ? sqrt(fmax(lamn[c] * tn, 0.0) / mean) : 0.0;
#pragma unroll
    for (int u = 0; u < RPV; ++u) {
      const int i = g + GV * u;
      fh[i * rp + c] = float(z[u] * sc);
      if (basis) basis[(long long)h * D * r + i * r + c] = float(z[u]);
    }
  }
  for (int e = tid; e < D * rp; e += NT) {
    const int cc = e % rp;
    if (cc >= cap) fh[e] = 0.f;
  }
}

// ---------------------------------------------------------------------------
// later calls: subspace-iteration factor (fp64, one block per head)
// ---------------------------------------------------------------------------
// X starts at the previous basis (D x r).  One step: Y = M X; G = Y^T Y;
// G = L L^T by a right-looking Cholesky in which a pivot at or below 1e-10 of
// the largest diagonal entry of G drops its column (L column 0); X = Y L^-T
// by forward substitution, row by row.  After the steps, lambda_j = x_j^T M
// x_j (clamped at 0) and F = X diag(sqrt(lambda / mean lambda)).  Sums run
// in a fixed order (deterministic).  basis_in may alias basis_out.
constexpr double kCholDrop = 1e-10;
template <int D>
__global__ __launch_bounds__(256) void subspace_factor_kernel(const float* __restrict__ m,
                                                              const float* basis_in, int r,
                                                              int rp, int steps,
                                                              float* __restrict__ f,
                                                              float* basis_out) {
  constexpr int TPR = 256 / D, NU = kMaxR / TPR;   // threads per row, columns per thread
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ double X[D][kMaxR + 1];
  __shared__ double G[kMaxR][kMaxR + 1];
  __shared__ double lam[kMaxR];
  __shared__ double s_ref, s_mean;
  __shared__ int32_t s_keep;
  const float* mh = m + (long long)h * D * D;
  const float* bi = basis_in + (long long)h * D * r;
  for (int e = tid; e < D * r; e += 256) X[e / r][e % r] = double(bi[e]);
  __syncthreads();
  const int row = tid / TPR, jc = tid % TPR;
  // acc[u] = (M X)[row][jc + TPR u], k in order
  auto mx = [&](double (&acc)[NU]) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NU; ++u) acc[u] = 0.0;
    const float* mr = mh + (long long)row * D;
    for (int k = 0; k < D; ++k) {
      const double mik = double(mr[k]);
#pragma unroll
      for (int u = 0; u < NU; ++u)
        if (jc + TPR * u < r) acc[u] = fma(mik, X[k][jc + TPR * u], acc[u]);
    }
  };
  for (int step = 0; step < steps; ++step) {
    double acc[NU];
    mx(acc);
    __syncthreads();
#pragma unroll
    for (int u = 0; u < NU; ++u)
      if (jc + TPR * u < r) X[row][jc + TPR * u] = acc[u];
    __syncthreads();
    for (int e = tid; e < r * r; e += 256) {
      const int a = e / r, b = e % r;
      double sacc = 0.0;
      for (int i = 0; i < D; ++i) sacc = fma(X[i][a], X[i][b], sacc);
      G[a][b] = sacc;
    }
    __syncthreads();
    if (tid == 0) {
      double mxd = 0.0;
      for (int j = 0; j < r; ++j) mxd = fmax(mxd, G[j][j]);
      s_ref = mxd;
    }
    __syncthreads();
    for (int j = 0; j < r; ++j) {
      if (tid == 0) {
        const double piv = G[j][j];
        const bool keep = piv > kCholDrop * s_ref && piv > 0.0;
        G[j][j] = keep ? sqrt(piv) : 0.0;
        s_keep = keep ? 1 : 0;
      }
      __syncthreads();
      const bool keep = s_keep != 0;
      const double ljj = G[j][j];
      for (int i = j + 1 + tid; i < r; i += 256) G[i][j] = keep ? G[i][j] / ljj : 0.0;
      __syncthreads();
      if (keep) {
        const int w = r - j - 1;
        for (int e = tid; e < w * w; e += 256) {
          const int i = j + 1 + e / w, l = j + 1 + e % w;
          if (l <= i) G[i][l] = fma(-G[i][j], G[l][j], G[i][l]);
        }
      }
      __syncthreads();
    }
    // X = Y L^-T, one row per thread, in place
    if (tid < D) {
      for (int j = 0; j < r; ++j) {
        double v = X[tid][j];
        for (int k = 0; k < j; ++k) v = fma(-X[tid][k], G[j][k], v);
        X[tid][j] = G[j][j] > 0.0 ? v / G[j][j] : 0.0;
      }
    }
    __syncthreads();
  }
  // Rayleigh quotients: Z = M X staged 64 rows at a time through G
  {
    double acc[NU];
    mx(acc);
    if (tid < kMaxR) lam[tid] = 0.0;
    for (int c0 = 0; c0 < D; c0 += kMaxR) {
      __syncthreads();
      if (row >= c0 && row < c0 + kMaxR) {
#pragma unroll
        for (int u = 0; u < NU; ++u)
          if (jc + TPR * u < r) G[row - c0][jc + TPR * u] = acc[u] * X[row][jc + TPR * u];
      }
      __syncthreads();
      if (tid < r) {
        double sacc = lam[tid];
        for (int i = 0; i < kMaxR && c0 + i < D; ++i) sacc += G[i][tid];
        lam[tid] = sacc;
      }
    }
    __syncthreads();
  }
  if (tid == 0) {
    double sm = 0.0;
    for (int j = 0; j < r; ++j) sm += fmax(lam[j], 0.0);
    s_mean = sm / double(r);
  }
  __syncthreads();
  const double mean = s_mean;
  float* fh = f + (long long)h * D * rp;
  for (int e = tid; e < D * rp; e += 256) {
    const int i = e / rp, j = e % rp;
    float v = 0.f;
    if (j < r && mean > 0.0) v = float(X[i][j] * sqrt(fmax(lam[j], 0.0) / mean));
    fh[e] = v;
  }
  float* bo = basis_out + (long long)h * D * r;
  for (int e = tid; e < D * r; e += 256) bo[e] = float(X[e / r][e % r]);
}

// ---------------------------------------------------------------------------
// projection (phi = x F, optionally RMS-normalised) and its bf16 pair
// ---------------------------------------------------------------------------
// phi^T = F^T x^T on v_mfma_f32_32x32x16_bf16, 4 waves x 32 rows per block:
// lane l owns row l % 32 and 16 of each 32 columns (the partner lane l ^ 32
// the other 16), so the RMS needs one exchange.  F enters as a bf16 pair
// (F = F_hi + F_lo to 2^-16); bf16 rows are exact, fp32 rows are split too
// (x_hi F_hi + x_hi F_lo + x_lo F_hi), fp32 accumulation.
constexpr int kProjTiles = 4;   // 128-row tiles per block (F^T is staged once per block)
template <int D>
__global__ __launch_bounds__(256) void project_kernel(const void* x, int dtype, long long sh,
                                                      long long st, int n,
                                                      const float* __restrict__ f, int r, int rp,
                                                      int rms, uint16_t* __restrict__ hi,
                                                      uint16_t* __restrict__ lo,
                                                      float* __restrict__ out) {
  constexpr int NS = D / 16, LD = D + 8;   // k-steps; LDS row length of F^T (bf16)
  const int h = blockIdx.y, tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int nl = lane & 31, g = lane >> 5;
  __shared__ __attribute__((aligned(16))) uint16_t fth[kMaxR * LD];
  __shared__ __attribute__((aligned(16))) uint16_t ftl[kMaxR * LD];
  const float* fh = f + (long long)h * D * rp;
  // F is read row by row (consecutive threads, consecutive columns)
  for (int e = tid; e < kMaxR * D; e += 256) {
    const int j = e / kMaxR, col = e % kMaxR;
    const float v = col < rp ? fh[j * rp + col] : 0.f;
    const uint16_t b = f32_to_bf16_rne(v);
    fth[col * LD + j] = b;
    ftl[col * LD + j] = f32_to_bf16_rne(v - bf16_to_f32(b));
  }
  __syncthreads();
  for (int tile = 0; tile < kProjTiles; ++tile) {
  const int row = (blockIdx.x * kProjTiles + tile) * 128 + wid * 32 + nl;
  const bool valid = row < n;
  const long long xo = h * sh + (long long)(valid ? row : 0) * st;
  bf16x8_t xh[NS], xl[NS];
  const bool f32in = dtype != SPARSEPR_BF16;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (!f32in) {
      const uint4 a = valid ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + xo +
                                                              16 * s + 8 * g)
                            : make_uint4(0, 0, 0, 0);
      xh[s] = __builtin_bit_cast(bf16x8_t, a);
    } else {
      const float* xr = static_cast<const float*>(x) + xo + 16 * s + 8 * g;
      uint16_t bh[8], bl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = valid ? xr[e] : 0.f;
        bh[e] = f32_to_bf16_rne(v);
        bl[e] = f32_to_bf16_rne(v - bf16_to_f32(bh[e]));
      }
      xh[s] = __builtin_bit_cast(bf16x8_t, bh);
      xl[s] = __builtin_bit_cast(bf16x8_t, bl);
    }
  }
  f32x16_t acc[kMaxR / 32];
#pragma unroll
  for (int cb = 0; cb < kMaxR / 32; ++cb) {
    acc[cb] = f32x16_t{};
    if (32 * cb >= rp) continue;
    const int col = 32 * cb + nl;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const bf16x8_t ah = *reinterpret_cast<const bf16x8_t*>(fth + col * LD + 16 * s + 8 * g);
      const bf16x8_t al = *reinterpret_cast<const bf16x8_t*>(ftl + col * LD + 16 * s + 8 * g);
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xh[s], acc[cb], 0, 0, 0);
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, xh[s], acc[cb], 0, 0, 0);
      if (f32in) acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, xl[s], acc[cb], 0, 0, 0);
    }
  }
  float scale = 1.f;
  if (rms) {
    float ss = 0.f;
#pragma unroll
    for (int cb = 0; cb < kMaxR / 32; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int col = 32 * cb + 8 * (i >> 2) + 4 * g + (i & 3);
        ss += col < r ? acc[cb][i] * acc[cb][i] : 0.f;
      }
    ss += __shfl_xor(ss, 32);
    scale = 1.f / fmaxf(sqrtf(ss / float(r)), 1e-6f);
  }
  if (!valid) continue;
  const long long o = ((long long)h * n + row) * rp;
  // each group of 4 consecutive columns leaves as one 8-byte (bf16) or
  // 16-byte (fp32) store; rp is a multiple of 16, so a group is all in or out
#pragma unroll
  for (int cb = 0; cb < kMaxR / 32; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int col = 32 * cb + 8 * q4 + 4 * g;
      if (col >= rp) continue;
      float v[4];
      uint16_t bh[4], bl[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = acc[cb][4 * q4 + e] * scale;
        bh[e] = f32_to_bf16_rne(v[e]);
        bl[e] = f32_to_bf16_rne(v[e] - bf16_to_f32(bh[e]));
      }
      *reinterpret_cast<uint2*>(hi + o + col) = __builtin_bit_cast(uint2, bh);
      *reinterpret_cast<uint2*>(lo + o + col) = __builtin_bit_cast(uint2, bl);
      if (out) {
        float* op = out + ((long long)h * n + row) * r + col;
        if (col + 4 <= r && (r & 3) == 0) {
          *reinterpret_cast<float4*>(op) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (col + e < r) op[e] = v[e];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// k-means
// ---------------------------------------------------------------------------
// Centre c of head h as fp32 (cent), bf16 pair and |c|^2 (fp32, wave sum).
template <int RP>
SPR_DEV void store_center(int h, int c, int C, float v, float* cent, uint16_t* chi, uint16_t* clo,
                          float* cnorm) {
  const int lane = threadIdx.x & 63;
  const long long o = ((long long)h * C + c) * RP;
  float sq = 0.f;
  if (lane < RP) {
    cent[o + lane] = v;
    const uint16_t bh = f32_to_bf16_rne(v);
    chi[o + lane] = bh;
    clo[o + lane] = f32_to_bf16_rne(v - bf16_to_f32(bh));
    sq = v * v;
  }
  sq = wave_sum(sq);
  if (lane == 0) cnorm[(long long)h * C + c] = sq;
}

// Initial centres: the feature rows init[h][c] (hi + lo).  One wave per centre.
template <int RP>
__global__ __launch_bounds__(256) void kmeans_init_kernel(const uint16_t* __restrict__ xh,
                                                          const uint16_t* __restrict__ xl, int n,
                                                          const int32_t* __restrict__ init, int C,
                                                          float* cent, uint16_t* chi,
                                                          uint16_t* clo, float* cnorm) {
  const int h = blockIdx.y, c = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (c >= C) return;
  int row = init[(long long)h * C + c];
  row = row < 0 ? 0 : (row >= n ? n - 1 : row);   // out-of-range indices are clamped
  float v = 0.f;
  if (lane < RP) {
    const long long o = ((long long)h * n + row) * RP + lane;
    v = bf16_to_f32(xh[o]) + bf16_to_f32(xl[o]);
  }
  store_center<RP>(h, c, C, v, cent, chi, clo, cnorm);
}

// Initial centres of a later call: the previous centroids cent[h][c] (original
// space, D values) mapped by the current factor F (D x rp): u = c F (fp32, in
// order), RMS-normalised over the r coordinates (floor 1e-6) for query
// coordinates.  One wave per centre, lane j < RP owns coordinate j.
template <int D, int RP>
__global__ __launch_bounds__(256) void kmeans_init_proj_kernel(const float* __restrict__ prev,
                                                               const float* __restrict__ f, int r,
                                                               int rms, int C, float* cent,
                                                               uint16_t* chi, uint16_t* clo,
                                                               float* cnorm) {
  const int h = blockIdx.y, c = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (c >= C) return;
  const float* pc = prev + ((long long)h * C + c) * D;
  const float* fh = f + (long long)h * D * RP;
  float u = 0.f;
  if (lane < RP)
    for (int i = 0; i < D; ++i) u = fmaf(pc[i], fh[i * RP + lane], u);
  if (rms) {
    const float ss = wave_sum(lane < r ? u * u : 0.f);
    u *= 1.f / fmaxf(sqrtf(ss / float(r)), 1e-6f);
  }
  store_center<RP>(h, c, C, u, cent, chi, clo, cnorm);
}

// Update: mean of each cluster's rows (perm/offsets from the stable sort of
// the labels); an empty cluster keeps its centre.  One block per cluster:
// thread (ph, ch) adds chunk ch (8 coordinates, hi + lo of the bf16 pair) of
// the cluster's rows ph, ph + phases, ... in order, and wave 0 adds the phase
// partials of each coordinate in a fixed order.
template <int RP>
__global__ __launch_bounds__(256) void kmeans_update_kernel(
    const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl, int n, int C, float* cent,
    uint16_t* chi, uint16_t* clo, float* cnorm) {
  constexpr int CPR = RP / 8, PH = 256 / CPR;
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const int ch = tid % CPR, ph = tid / CPR;
  __shared__ float part[PH * CPR][8];
  const int32_t* off = offsets + (long long)h * (C + 1);
  const int b0 = off[c], b1 = off[c + 1];
  const int32_t* pr = perm + (long long)h * n;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4& a, const uint4& b) __attribute__((always_inline)) {
    const uint32_t wa[4] = {a.x, a.y, a.z, a.w}, wb[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += __uint_as_float(wa[e] << 16) + __uint_as_float(wb[e] << 16);
      acc[2 * e + 1] += __uint_as_float(wa[e] & 0xffff0000u) + __uint_as_float(wb[e] & 0xffff0000u);
    }
  };
  if (ph < PH) {
    int r = b0 + ph;
    for (; r + PH < b1; r += 2 * PH) {
      const long long o0 = ((long long)h * n + pr[r]) * RP + 8 * ch;
      const long long o1 = ((long long)h * n + pr[r + PH]) * RP + 8 * ch;
      const uint4 a0 = *reinterpret_cast<const uint4*>(xh + o0);
      const uint4 l0 = *reinterpret_cast<const uint4*>(xl + o0);
      const uint4 a1 = *reinterpret_cast<const uint4*>(xh + o1);
      const uint4 l1 = *reinterpret_cast<const uint4*>(xl + o1);
      add(a0, l0);
      add(a1, l1);
    }
    for (; r < b1; r += PH) {
      const long long o = ((long long)h * n + pr[r]) * RP + 8 * ch;
      add(*reinterpret_cast<const uint4*>(xh + o), *reinterpret_cast<const uint4*>(xl + o));
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) part[tid][e] = acc[e];
  }
  __syncthreads();
  if (tid >= 64) return;
  const int j = tid;
  float v = 0.f;
  if (j < RP) {
    if (b1 > b0) {
      float t = 0.f;
      for (int p2 = 0; p2 < PH; ++p2) t += part[p2 * CPR + j / 8][j % 8];
      v = t / float(b1 - b0);
    } else {
      v = cent[((long long)h * C + c) * RP + j];
    }
  }
  store_center<RP>(h, c, C, v, cent, chi, clo, cnorm);
}

// Assignment: label = argmin_c |c|^2 - 2 x.c = argmax_c x.c - |c|^2 / 2, ties
// to the smaller c.  Block = kAssignWaves waves, each wave two sets of 32
// rows that share every centre fragment read from LDS (one LDS read feeds two
// products).  Centres pass through LDS 128 at a time (rows padded by 16
// bytes, so the 16 rows read by one 16-lane group hit distinct banks).
// S^T tile = C_tile X^T on v_mfma_f32_32x32x16_bf16: lane l owns row l % 32
// of each set and 16 centres of each 32-centre block.  The accumulator
// starts at -|c|^2 / 2 (-inf past the last centre), so the products land on
// the score itself and the argmax needs one compare per centre.
constexpr int kCenterTile = 128;
constexpr int kAssignWaves = 8;
constexpr int kRowSets = 2;
constexpr int kAssignRows = 32 * kRowSets * kAssignWaves;   // rows per block
template <int RP>
__global__ __launch_bounds__(64 * kAssignWaves, 4) void kmeans_assign_kernel(
    const uint16_t* __restrict__ xh, const uint16_t* __restrict__ xl, int n,
    const uint16_t* __restrict__ chi, const uint16_t* __restrict__ clo,
    const float* __restrict__ cnorm, int C, int32_t* __restrict__ labels) {
  constexpr int NS = RP / 16, LD = RP + 8;   // k-steps, LDS row length (bf16)
  constexpr int NT = 64 * kAssignWaves;
  constexpr int CH = kCenterTile * (RP / 8);  // 16-byte chunks of one tile (hi or lo)
  const int h = blockIdx.y, tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  const int nl = lane & 31, g = lane >> 5;
  __shared__ __attribute__((aligned(16))) uint16_t sh[kCenterTile * LD];
  __shared__ __attribute__((aligned(16))) uint16_t sl[kCenterTile * LD];
  __shared__ __attribute__((aligned(16))) float sn[kCenterTile];
  int row[kRowSets];
  bf16x8_t bh[kRowSets][NS], bl[kRowSets][NS];
#pragma unroll
  for (int u = 0; u < kRowSets; ++u) {
    row[u] = blockIdx.x * kAssignRows + (wid * kRowSets + u) * 32 + nl;
    const long long o = ((long long)h * n + (row[u] < n ? row[u] : 0)) * RP;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint4 a = row[u] < n ? *reinterpret_cast<const uint4*>(xh + o + 16 * s + 8 * g)
                                 : make_uint4(0, 0, 0, 0);
      const uint4 b = row[u] < n ? *reinterpret_cast<const uint4*>(xl + o + 16 * s + 8 * g)
                                 : make_uint4(0, 0, 0, 0);
      bh[u][s] = __builtin_bit_cast(bf16x8_t, a);
      bl[u][s] = __builtin_bit_cast(bf16x8_t, b);
    }
  }
  float best[kRowSets];
  int bi[kRowSets];
#pragma unroll
  for (int u = 0; u < kRowSets; ++u) {
    best[u] = -__builtin_huge_valf();
    bi[u] = 0;   // a valid label even if no candidate compares above -inf (NaN input)
  }
  const uint16_t* ch = chi + (long long)h * C * RP;
  const uint16_t* cl = clo + (long long)h * C * RP;
  const float* cn = cnorm + (long long)h * C;
  for (int t0 = 0; t0 < C; t0 += kCenterTile) {
    __syncthreads();   // every wave is done with the previous tile
    for (int e = tid; e < CH; e += NT) {
      const int cc = e / (RP / 8), c8 = e % (RP / 8), c = t0 + cc;
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (c < C) {
        a = *reinterpret_cast<const uint4*>(ch + (long long)c * RP + 8 * c8);
        b = *reinterpret_cast<const uint4*>(cl + (long long)c * RP + 8 * c8);
      }
      *reinterpret_cast<uint4*>(sh + cc * LD + 8 * c8) = a;
      *reinterpret_cast<uint4*>(sl + cc * LD + 8 * c8) = b;
    }
    for (int e = tid; e < kCenterTile; e += NT)
      sn[e] = t0 + e < C ? -0.5f * cn[t0 + e] : -__builtin_huge_valf();
    __syncthreads();
#pragma unroll 1
    for (int j = 0; j < kCenterTile / 32; ++j) {
      if (t0 + 32 * j >= C) break;
      // accumulators in the C layout: register 4 q + r holds centre
      // 32 j + 8 q + 4 g + r, i.e. four consecutive scores per q
      f32x16_t acc[kRowSets];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 v4 = *reinterpret_cast<const float4*>(sn + 32 * j + 8 * q + 4 * g);
#pragma unroll
        for (int u = 0; u < kRowSets; ++u) {
          acc[u][4 * q] = v4.x;
          acc[u][4 * q + 1] = v4.y;
          acc[u][4 * q + 2] = v4.z;
          acc[u][4 * q + 3] = v4.w;
        }
      }
      const int crow = 32 * j + nl;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8_t ah =
            *reinterpret_cast<const bf16x8_t*>(sh + crow * LD + 16 * s + 8 * g);
        const bf16x8_t al =
            *reinterpret_cast<const bf16x8_t*>(sl + crow * LD + 16 * s + 8 * g);
        // per accumulator the same three products in the same order
#pragma unroll
        for (int u = 0; u < kRowSets; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh[u][s], acc[u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kRowSets; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[u][s], acc[u], 0, 0, 0);
#pragma unroll
        for (int u = 0; u < kRowSets; ++u)
          acc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh[u][s], acc[u], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kRowSets; ++u) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if (acc[u][i] > best[u]) {
            best[u] = acc[u][i];
            bi[u] = t0 + 32 * j + 8 * (i >> 2) + 4 * g + (i & 3);
          }
        }
      }
    }
  }
#pragma unroll
  for (int u = 0; u < kRowSets; ++u) {
    // the two lanes of a row hold interleaved centre subsets
    const float ob = __shfl_xor(best[u], 32);
    const int oi = __shfl_xor(bi[u], 32);
    if (ob > best[u] || (ob == best[u] && oi < bi[u])) {
      best[u] = ob;
      bi[u] = oi;
    }
    if (g == 0 && row[u] < n) labels[(long long)h * n + row[u]] = bi[u];
  }
}

// Mean of each group's rows in the original space (fp32).  One block per
// group: thread (ph, ch) adds the 16-byte chunk ch of rows ph, ph + phases,
// ... of the group in order (8 bf16 or 4 fp32 values), and the phase partials
// of each dimension are added in a fixed order.  An empty group takes its
// initial row init[h][c] when init is given and keeps its entry otherwise
// (the centroid of an earlier call).  Rows are 16-byte aligned (as for the
// layout call).
template <int D>
__global__ __launch_bounds__(256) void key_centroid_kernel(const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ offsets,
                                                           const void* k, int dtype, long long sh,
                                                           long long st, int n, int C,
                                                           const int32_t* __restrict__ init,
                                                           float* __restrict__ cent) {
  const int h = blockIdx.y, c = blockIdx.x, tid = threadIdx.x;
  const bool bf = dtype == SPARSEPR_BF16;
  const int epc = bf ? 8 : 4;             // elements per 16-byte chunk
  const int cpr = D / epc, phases = 256 / cpr;
  const int ch = tid % cpr, ph = tid / cpr;
  __shared__ float part[256][8];
  const int32_t* off = offsets + (long long)h * (C + 1);
  const int b0 = off[c], b1 = off[c + 1];
  const int32_t* pr = perm + (long long)h * n;
  const size_t es = bf ? 2 : 4;
  const char* base = static_cast<const char*>(k) + (long long)h * sh * es;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  auto add = [&](const uint4& w) __attribute__((always_inline)) {
    if (bf) {
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(ws[e] << 16);
        acc[2 * e + 1] += __uint_as_float(ws[e] & 0xffff0000u);
      }
    } else {
      acc[0] += __uint_as_float(w.x);
      acc[1] += __uint_as_float(w.y);
      acc[2] += __uint_as_float(w.z);
      acc[3] += __uint_as_float(w.w);
    }
  };
  int r = b0 + ph;
  for (; r + 3 * phases < b1; r += 4 * phases) {
    uint4 w[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      w[u] = *reinterpret_cast<const uint4*>(base + ((long long)pr[r + u * phases] * st) * es +
                                             ch * 16);
#pragma unroll
    for (int u = 0; u < 4; ++u) add(w[u]);
  }
  for (; r < b1; r += phases)
    add(*reinterpret_cast<const uint4*>(base + ((long long)pr[r] * st) * es + ch * 16));
#pragma unroll
  for (int e = 0; e < 8; ++e) part[tid][e] = acc[e];
  __syncthreads();
  for (int j = tid; j < D; j += 256) {
    const int cj = j / epc, e = j % epc;
    float t = 0.f;
    for (int p2 = 0; p2 < phases; ++p2) t += part[p2 * cpr + cj][e];
    float* out = cent + ((long long)h * C + c) * D + j;
    if (b1 > b0) {
      *out = t / float(b1 - b0);
    } else if (init) {
      int row = init[(long long)h * C + c];
      row = row < 0 ? 0 : (row >= n ? n - 1 : row);
      *out = load_elem(k, dtype, h * sh + (long long)row * st + j);
    }
  }
}

struct RcpWs {
  float *metric, *factor, *cent, *cnorm, *kcent;
  uint16_t *xh, *xl, *chi, *clo;
  int32_t *perm, *offsets;
  void* sort_ws;
};

RcpWs carve_rcp(void* base, const sparsepr_dims* d, size_t* used) {
  Carver cv(base);
  const size_t H = d->heads, D = d->head_dim;
  const size_t nmax = d->n_q > d->n_k ? d->n_q : d->n_k;
  const int cmax = d->c_q > d->c_k ? d->c_q : d->c_k;
  RcpWs w;
  w.metric = cv.take<float>(H * D * D);
  w.factor = cv.take<float>(H * D * kMaxR);
  w.cent = cv.take<float>(H * cmax * kMaxR);
  w.cnorm = cv.take<float>(H * cmax);
  w.kcent = cv.take<float>(H * d->c_k * D);
  w.xh = cv.take<uint16_t>(H * nmax * kMaxR);
  w.xl = cv.take<uint16_t>(H * nmax * kMaxR);
  w.chi = cv.take<uint16_t>(H * cmax * kMaxR);
  w.clo = cv.take<uint16_t>(H * cmax * kMaxR);
  w.perm = cv.take<int32_t>(H * nmax);
  w.offsets = cv.take<int32_t>(H * (cmax + 1));
  const size_t sq = group_sort_ws_bytes(d->heads, d->n_q, d->c_q);
  const size_t sk = group_sort_ws_bytes(d->heads, d->n_k, d->c_k);
  w.sort_ws = cv.take<char>(sq > sk ? sq : sk);
  if (used) *used = cv.used;
  return w;
}

// init == nullptr: the centres were set by kmeans_init_proj_kernel
template <int RP>
int32_t run_kmeans(const RcpWs& w, int H, int n, int C, const int32_t* init, int iters,
                   int32_t* labels, hipStream_t stream) {
  const dim3 gc((C + 3) / 4, H);
  if (init) {
    kmeans_init_kernel<RP><<<gc, 256, 0, stream>>>(w.xh, w.xl, n, init, C, w.cent, w.chi, w.clo,
                                                   w.cnorm);
    SPR_LAUNCH_CHECK();
  }
  for (int it = 0; it < iters; ++it) {
    kmeans_assign_kernel<RP><<<dim3((n + kAssignRows - 1) / kAssignRows, H), 64 * kAssignWaves,
                               0, stream>>>(
        w.xh, w.xl, n, w.chi, w.clo, w.cnorm, C, labels);
    SPR_LAUNCH_CHECK();
    if (it + 1 == iters) break;   // the partition is the last assignment
    int32_t st = group_sort(labels, H, n, C, w.perm, w.offsets, w.sort_ws, stream);
    if (st != SPARSEPR_OK) return st;
    kmeans_update_kernel<RP><<<dim3(C, H), 256, 0, stream>>>(w.perm, w.offsets, w.xh, w.xl, n, C,
                                                             w.cent, w.chi, w.clo, w.cnorm);
    SPR_LAUNCH_CHECK();
  }
  return SPARSEPR_OK;
}

int32_t kmeans_rp(int rp, const RcpWs& w, int H, int n, int C, const int32_t* init, int iters,
                  int32_t* labels, hipStream_t stream) {
  switch (rp) {
    case 16: return run_kmeans<16>(w, H, n, C, init, iters, labels, stream);
    case 32: return run_kmeans<32>(w, H, n, C, init, iters, labels, stream);
    case 48: return run_kmeans<48>(w, H, n, C, init, iters, labels, stream);
    default: return run_kmeans<64>(w, H, n, C, init, iters, labels, stream);
  }
}

template <int D>
void init_proj(int rp, const float* prev, const RcpWs& w, int r, int rms, int H, int C,
               hipStream_t stream) {
  const dim3 gc((C + 3) / 4, H);
  switch (rp) {
    case 16: kmeans_init_proj_kernel<D, 16><<<gc, 256, 0, stream>>>(prev, w.factor, r, rms, C, w.cent, w.chi, w.clo, w.cnorm); break;
    case 32: kmeans_init_proj_kernel<D, 32><<<gc, 256, 0, stream>>>(prev, w.factor, r, rms, C, w.cent, w.chi, w.clo, w.cnorm); break;
    case 48: kmeans_init_proj_kernel<D, 48><<<gc, 256, 0, stream>>>(prev, w.factor, r, rms, C, w.cent, w.chi, w.clo, w.cnorm); break;
    default: kmeans_init_proj_kernel<D, 64><<<gc, 256, 0, stream>>>(prev, w.factor, r, rms, C, w.cent, w.chi, w.clo, w.cnorm); break;
  }
}

// The state of a later call (all four set, or all null for a call that
// keeps none): bases [H][D][r] and original-space centroids [H][C][D].
struct RcpState {
  int warm;
  float *basis_q, *basis_k, *cent_q, *cent_k;
};

template <int D>
int32_t rcp_run(const sparsepr_dims* d, int m_s, int r_k, int r_q, int iters, const void* q,
                const void* k, const int32_t* init_q, const int32_t* init_k, int32_t* labels_q,
                int32_t* labels_kv, float* phi_q, float* phi_k, const RcpState& s,
                const RcpWs& w, hipStream_t stream) {
  const int H = d->heads;
  const int rpk = (r_k + 15) / 16 * 16, rpq = (r_q + 15) / 16 * 16;
  const bool keep = s.cent_k != nullptr;
  // key-response coordinates and K/V groups
  key_metric_kernel<D><<<H, 256, 0, stream>>>(q, d->dtype, d->q_stride_head, d->q_stride_tok,
                                              d->n_q, m_s, w.metric);
  SPR_LAUNCH_CHECK();
  if (s.warm)
    subspace_factor_kernel<D><<<H, 256, 0, stream>>>(w.metric, s.basis_k, r_k, rpk, 2, w.factor,
                                                     s.basis_k);
  else
    eig_tri_kernel<D><<<H, kEigThreads, 0, stream>>>(w.metric, r_k, rpk, w.factor, s.basis_k);
  SPR_LAUNCH_CHECK();
  project_kernel<D><<<dim3((d->n_k + 128 * kProjTiles - 1) / (128 * kProjTiles), H), 256, 0, stream>>>(
      k, d->dtype, d->kv_stride_head, d->kv_stride_tok, d->n_k, w.factor, r_k, rpk, 0, w.xh, w.xl,
      phi_k);
  SPR_LAUNCH_CHECK();
  if (s.warm) {
    init_proj<D>(rpk, s.cent_k, w, r_k, 0, H, d->c_k, stream);
    SPR_LAUNCH_CHECK();
  }
  int32_t st = kmeans_rp(rpk, w, H, d->n_k, d->c_k, s.warm ? nullptr : init_k, iters, labels_kv,
                         stream);
  if (st != SPARSEPR_OK) return st;
  // query-response coordinates from the K/V groups, then query groups; the
  // K/V centroids go straight to the state when it is kept
  st = group_sort(labels_kv, H, d->n_k, d->c_k, w.perm, w.offsets, w.sort_ws, stream);
  if (st != SPARSEPR_OK) return st;
  float* kcent = keep ? s.cent_k : w.kcent;
  key_centroid_kernel<D><<<dim3(d->c_k, H), 256, 0, stream>>>(
      w.perm, w.offsets, k, d->dtype, d->kv_stride_head, d->kv_stride_tok, d->n_k, d->c_k,
      s.warm ? nullptr : init_k, kcent);
  SPR_LAUNCH_CHECK();
  query_metric_kernel<D><<<H, 256, 0, stream>>>(kcent, w.offsets, d->c_k, w.metric);
  SPR_LAUNCH_CHECK();
  if (s.warm)
    subspace_factor_kernel<D><<<H, 256, 0, stream>>>(w.metric, s.basis_q, r_q, rpq, 2, w.factor,
                                                     s.basis_q);
  else
    eig_tri_kernel<D><<<H, kEigThreads, 0, stream>>>(w.metric, r_q, rpq, w.factor, s.basis_q);
  SPR_LAUNCH_CHECK();
  project_kernel<D><<<dim3((d->n_q + 128 * kProjTiles - 1) / (128 * kProjTiles), H), 256, 0, stream>>>(
      q, d->dtype, d->q_stride_head, d->q_stride_tok, d->n_q, w.factor, r_q, rpq, 1, w.xh, w.xl,
      phi_q);
  SPR_LAUNCH_CHECK();
  if (s.warm) {
    init_proj<D>(rpq, s.cent_q, w, r_q, 1, H, d->c_q, stream);
    SPR_LAUNCH_CHECK();
  }
  st = kmeans_rp(rpq, w, H, d->n_q, d->c_q, s.warm ? nullptr : init_q, iters, labels_q, stream);
  if (st != SPARSEPR_OK || !keep) return st;
  // query group centroids for the next call
  st = group_sort(labels_q, H, d->n_q, d->c_q, w.perm, w.offsets, w.sort_ws, stream);
  if (st != SPARSEPR_OK) return st;
  key_centroid_kernel<D><<<dim3(d->c_q, H), 256, 0, stream>>>(
      w.perm, w.offsets, q, d->dtype, d->q_stride_head, d->q_stride_tok, d->n_q, d->c_q,
      s.warm ? nullptr : init_q, s.cent_q);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}

}  // namespace

size_t rcp_ws_bytes(const sparsepr_dims* d) {
  size_t used = 0;
  carve_rcp(nullptr, d, &used);
  return used;
}

}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_rcp_partition(const sparsepr_dims* dims, int32_t m_s, int32_t r_k,
                                          int32_t r_q, int32_t iters, const void* q,
                                          const void* k, const int32_t* init_q,
                                          const int32_t* init_k, int32_t* labels_q,
                                          int32_t* labels_kv, float* phi_q, float* phi_k,
                                          void* ws, size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!q || !k || !init_q || !init_k || !labels_q || !labels_kv) return SPARSEPR_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k)) return SPARSEPR_ERR_INVALID;
  if (m_s < 1 || iters < 1 || r_k < 1 || r_q < 1 || r_k > kMaxR || r_q > kMaxR ||
      r_k > dims->head_dim || r_q > dims->head_dim)
    return SPARSEPR_ERR_INVALID;
  const size_t need = rcp_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  const RcpWs w = carve_rcp(ws, dims, nullptr);
  const RcpState s{0, nullptr, nullptr, nullptr, nullptr};
  if (dims->head_dim == 128)
    return rcp_run<128>(dims, m_s, r_k, r_q, iters, q, k, init_q, init_k, labels_q, labels_kv,
                        phi_q, phi_k, s, w, stream);
  return rcp_run<64>(dims, m_s, r_k, r_q, iters, q, k, init_q, init_k, labels_q, labels_kv,
                     phi_q, phi_k, s, w, stream);
}

extern "C" int32_t sparsepr_rcp_partition_ex(const sparsepr_dims* dims, int32_t m_s, int32_t r_k,
                                             int32_t r_q, int32_t iters, int32_t warm,
                                             const void* q, const void* k, const int32_t* init_q,
                                             const int32_t* init_k, float* basis_q,
                                             float* basis_k, float* cent_q, float* cent_k,
                                             int32_t* labels_q, int32_t* labels_kv, float* phi_q,
                                             float* phi_k, void* ws, size_t ws_bytes,
                                             hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!q || !k || !labels_q || !labels_kv || !basis_q || !basis_k || !cent_q || !cent_k)
    return SPARSEPR_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k)) return SPARSEPR_ERR_INVALID;
  if (warm != 0 && warm != 1) return SPARSEPR_ERR_INVALID;
  if (!warm && (!init_q || !init_k)) return SPARSEPR_ERR_INVALID;
  if (m_s < 1 || iters < 1 || r_k < 1 || r_q < 1 || r_k > kMaxR || r_q > kMaxR ||
      r_k > dims->head_dim || r_q > dims->head_dim)
    return SPARSEPR_ERR_INVALID;
  const size_t need = rcp_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  const RcpWs w = carve_rcp(ws, dims, nullptr);
  const RcpState s{warm, basis_q, basis_k, cent_q, cent_k};
  if (dims->head_dim == 128)
    return rcp_run<128>(dims, m_s, r_k, r_q, iters, q, k, init_q, init_k, labels_q, labels_kv,
                        phi_q, phi_k, s, w, stream);
  return rcp_run<64>(dims, m_s, r_k, r_q, iters, q, k, init_q, init_k, labels_q, labels_kv,
                     phi_q, phi_k, s, w, stream);
}
