// S6-S8: probe selection, exact probe rows and the correction fit.
//
// SparsePR paper, Appendix A.2 (Algorithm A.1): per non-empty query group,
// rows are ranked by distance to the group centroid (ties by token index);
// groups are ordered by decreasing size (ties by group id); traversal t
// takes the t-th row of every group that still has one, until M probes.
// Because groups are ordered by size, the groups still holding a t-th row
// are exactly the first G(t) groups of that order, so the probe taken from
// group a in traversal t sits at position S(t) + rank(a), where
// S(t) = sum_a min(n_a, t).  Every group therefore finds its probe slots
// without a sequential walk.
//
// Appendix A.1: with the retained (S) and omitted (U) key sets of the probe's
// group, Z_S, N_S, Z_U, N_U are the softmax partition sums and value
// numerators; O_sp = N_S/Z_S, O_dense = (N_S+N_U)/(Z_S+Z_U), and the residual
// R = O_dense - O_sp = w_U (Z_S N_U - Z_U N_S) / (Z Z_S) is formed without
// cancelling the retained part.  The probe kernel accumulates the four sums
// (separate running maxima for S and U) over key chunks; a merge kernel
// combines the chunks in fp64.
//
// Appendix A.2 / D.3 fit, per head in fp64: coverage weights |G_a|/m_a (the
// review's step (4)), unit-sum weights for the means and the feature scale
// sqrt(var + 1e-6), unit-mean weights for the ridge; the ridge is solved in
// its dual (M x M) form B = Xw^T (Xw Xw^T + lam I)^-1 Rw with Xw = W~^1/2
// Xbar, Rw = W~^1/2 Rbar; the right singular vectors of Rw come from an
// fp64 symmetric eigensolve of Rw Rw^T (Householder reduction to tridiagonal
// form, bisection, twisted factorisations); finally B is folded with the
// projection into A = diag(1/s) B Psi and c = mu_R - (mu_x A) Psi^T.

#include <type_traits>

#include "common.h"
#include "mfma_tiles.h"
#include "f64_lanes.h"
#include "lds_dma.h"

namespace spr {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunks = 64;        // key chunks per head in the probe-row kernel
constexpr int kMaxM = SPARSEPR_MAX_PROBES;

// ---------------------------------------------------------------------------
// plan: group ranks, per-group probe counts, S(t) table, default outputs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ off_q, int c_q,
                                                   int n_q, int m, int32_t* __restrict__ m_a,
                                                   int32_t* __restrict__ rank_out,
                                                   int32_t* __restrict__ s_tab,
                                                   int32_t* __restrict__ probe_rows,
                                                   int32_t* __restrict__ probe_tokens,
                                                   int32_t* __restrict__ probe_group) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ int32_t na[SPARSEPR_MAX_GROUPS];
  __shared__ int32_t cnt[kMaxM + 2];
  __shared__ int32_t S[kMaxM + 2];
  __shared__ int32_t sh_T;
  const int32_t* o = off_q + (long long)h * (c_q + 1);
  for (int a = tid; a < c_q; a += blockDim.x) na[a] = o[a + 1] - o[a];
  for (int i = tid; i < kMaxM + 2; i += blockDim.x) cnt[i] = 0;
  const int me = m < n_q ? m : n_q;
  for (int i = tid; i < m; i += blockDim.x) {
    probe_rows[(long long)h * m + i] = -1;
    probe_tokens[(long long)h * m + i] = -1;
    probe_group[(long long)h * m + i] = -1;
  }
  __syncthreads();
  // histogram of min(n_a, M+1): G(j) = #{a : n_a >= j}
  for (int a = tid; a < c_q; a += blockDim.x) {
    int v = na[a] < kMaxM + 1 ? na[a] : kMaxM + 1;
    if (v > 0) atomicAdd(&cnt[v], 1);
  }
  __syncthreads();
  if (tid == 0) {
    int ge = 0;  // #{a : n_a >= j}, built from the top
    int Gj[kMaxM + 2];
    for (int j = kMaxM + 1; j >= 1; --j) {
      ge += cnt[j];
      Gj[j] = ge;
    }
    S[0] = 0;
    int T = 0;
    for (int t = 1; t <= kMaxM + 1; ++t) {
      S[t] = S[t - 1] + Gj[t];
      if (T == 0 && S[t] >= me) T = t;
    }
    sh_T = T;
  }
  __syncthreads();
  const int T = sh_T;
  const int F = T - 1;
  const int rem = me - S[F];
  for (int a = tid; a < c_q; a += blockDim.x) {
    int r = -1, ma = 0;
    if (na[a] > 0) {
      r = 0;
      for (int b = 0; b < c_q; ++b)
        if (na[b] > na[a] || (na[b] == na[a] && b < a)) ++r;
      ma = na[a] < F ? na[a] : F;
      if (na[a] > F && r < rem) ++ma;
    }
    m_a[(long long)h * c_q + a] = ma;
    rank_out[(long long)h * c_q + a] = r;
  }
  for (int t = tid; t <= kMaxM + 1; t += blockDim.x) s_tab[(long long)h * (kMaxM + 2) + t] = S[t];
}

// ---------------------------------------------------------------------------
// select: the m_a nearest rows of each probed group, in (distance, row) order
// ---------------------------------------------------------------------------
template <typename T>
SPR_DEV float to_f32(T x);
template <>
SPR_DEV float to_f32<uint16_t>(uint16_t x) { return bf16_to_f32(x); }
template <>
SPR_DEV float to_f32<float>(float x) { return x; }

template <typename T>
__global__ __launch_bounds__(256) void select_kernel(
    const T* __restrict__ q_g, const double* __restrict__ cen, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ perm_q, const int32_t* __restrict__ m_a,
    const int32_t* __restrict__ rank, const int32_t* __restrict__ s_tab, int n_q, int c_q, int d,
    int m, double* __restrict__ dist, int32_t* __restrict__ probe_rows,
    int32_t* __restrict__ probe_tokens, int32_t* __restrict__ probe_group) {
  const int a = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int ma = m_a[(long long)h * c_q + a];
  if (ma == 0) return;
  __shared__ double cs[128];
  __shared__ double rd[4];
  __shared__ int32_t ri[4];
  const int32_t* o = off_q + (long long)h * (c_q + 1);
  const int lo = o[a], hi = o[a + 1];
  const double* c = cen + ((long long)h * c_q + a) * d;
  for (int j = tid; j < d; j += 256) cs[j] = c[j];
  __syncthreads();
  double* dh = dist + (long long)h * n_q;
  // a row's coordinates in order, read 16 bytes at a time when rows are
  // 16-byte aligned (the same sum as element by element)
  constexpr int EPV = 16 / sizeof(T);
  const bool vec = d % EPV == 0;
  for (int r = lo + tid; r < hi; r += 256) {
    const T* x = q_g + ((long long)h * n_q + r) * d;
    double s = 0.0;
    if (vec) {
      for (int j0 = 0; j0 < d; j0 += EPV) {
        const uint4 w = *reinterpret_cast<const uint4*>(x + j0);
        T e[EPV];
        __builtin_memcpy(e, &w, 16);
#pragma unroll
        for (int u = 0; u < EPV; ++u) {
          const double t = double(to_f32(e[u])) - cs[j0 + u];
          s = fma(t, t, s);
        }
      }
    } else {
      for (int j = 0; j < d; ++j) {
        const double t = double(to_f32(x[j])) - cs[j];
        s = fma(t, t, s);
      }
    }
    dh[r] = sqrt(s);
  }
  __syncthreads();
  const int rk = rank[(long long)h * c_q + a];
  double pd = -1.0;
  int pr = -1;
  for (int t = 0; t < ma; ++t) {
    double bd = __builtin_huge_val();
    int br = 0x7fffffff;
    for (int r = lo + tid; r < hi; r += 256) {
      double v = dh[r];
      bool after = v > pd || (v == pd && r > pr);
      if (after && (v < bd || (v == bd && r < br))) { bd = v; br = r; }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      double v2 = __shfl_xor(bd, off);
      int r2 = __shfl_xor(br, off);
      if (v2 < bd || (v2 == bd && r2 < br)) { bd = v2; br = r2; }
    }
    __syncthreads();
    if ((tid & 63) == 0) { rd[tid >> 6] = bd; ri[tid >> 6] = br; }
    __syncthreads();
    bd = rd[0];
    br = ri[0];
    for (int w = 1; w < 4; ++w)
      if (rd[w] < bd || (rd[w] == bd && ri[w] < br)) { bd = rd[w]; br = ri[w]; }
    if (tid == 0) {
      const int pos = s_tab[(long long)h * (kMaxM + 2) + t] + rk;
      probe_rows[(long long)h * m + pos] = br;
      probe_tokens[(long long)h * m + pos] = perm_q[(long long)h * n_q + br];
      probe_group[(long long)h * m + pos] = a;
    }
    pd = bd;
    pr = br;
  }
}

// ---------------------------------------------------------------------------
// exact probe rows: retained / omitted partial sums per key chunk (VALU)
// ---------------------------------------------------------------------------
// Thread layout: probe p = tid / 4 (64 probes), dim slice sl = tid % 4 of
// D/4 dims.  Partial record per (head, chunk, probe): [mS, mU, ZS, ZU] and
// NS[D], NU[D].
// values: bf16 inputs arrive as fp16(v * 2^-v_shift) from the layout call
template <typename T>
SPR_DEV float v_to_f32(T x, float scale);
template <>
SPR_DEV float v_to_f32<uint16_t>(uint16_t x, float scale) {
  return float(__builtin_bit_cast(_Float16, x)) * scale;
}
template <>
SPR_DEV float v_to_f32<float>(float x, float scale) { return x; }

template <typename T, int D>
__global__ __launch_bounds__(256) void probe_rows_kernel(
    const T* __restrict__ q_g, const T* __restrict__ k_g, const T* __restrict__ v_g,
    const int32_t* __restrict__ v_shift,
    const int32_t* __restrict__ off_k, const int32_t* __restrict__ rowptr,
    const int32_t* __restrict__ col, const int32_t* __restrict__ probe_rows,
    const int32_t* __restrict__ probe_group, int n_q, int n_k, int c_q, int c_k, int m,
    float scale_log2, float* __restrict__ part_s, float* __restrict__ part_n) {
  constexpr int DPL = D / 4;
  constexpr int TK = 32;
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int p = tid >> 2, sl = tid & 3;
  __shared__ uint32_t mask[kMaxM][32];
  __shared__ float ks[TK][D + 4];
  __shared__ float vs[TK][D + 4];
  __shared__ int32_t kgrp[TK];
  __shared__ int32_t okl[SPARSEPR_MAX_GROUPS + 1];
  for (int i = tid; i < kMaxM * 32; i += 256) (&mask[0][0])[i] = 0u;
  const int32_t* ok = off_k + (long long)h * (c_k + 1);
  for (int i = tid; i <= c_k; i += 256) okl[i] = ok[i];
  __syncthreads();
  const bool pvalid = p < m && probe_rows[(long long)h * m + p] >= 0;
  const int grp = pvalid ? probe_group[(long long)h * m + p] : 0;
  if (pvalid) {
    const int32_t* rp = rowptr + (long long)h * (c_q + 1);
    const int32_t* cl = col + (long long)h * c_q * c_k;
    for (int i = rp[grp] + sl; i < rp[grp + 1]; i += 4) {
      const int b = cl[i];
      atomicOr(&mask[p][b >> 5], 1u << (b & 31));
    }
  }
  float q[DPL];
  {
    const int row = pvalid ? probe_rows[(long long)h * m + p] : 0;
    const T* qr = q_g + ((long long)h * n_q + row) * D + sl * DPL;
#pragma unroll
    for (int i = 0; i < DPL; ++i) q[i] = pvalid ? to_f32(qr[i]) : 0.f;
  }
  float ns[DPL], nu[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) ns[i] = nu[i] = 0.f;
  const float NEG = -__builtin_huge_valf();
  float mS = NEG, mU = NEG, zS = 0.f, zU = 0.f;
  const int per = (n_k + kChunks - 1) / kChunks;
  const int k0 = chunk * per, k1 = min(n_k, k0 + per);
  const T* Kh = k_g + (long long)h * n_k * D;
  const T* Vh = v_g + (long long)h * n_k * D;
  const float vscale = __builtin_ldexpf(1.f, v_shift[h]);
  for (int t0 = k0; t0 < k1; t0 += TK) {
    __syncthreads();
    for (int e = tid; e < TK * D; e += 256) {
      const int r = e / D, j = e % D;
      const int row = t0 + r;
      float kv = 0.f, vv = 0.f;
      if (row < k1) {
        kv = to_f32(Kh[(long long)row * D + j]);
        vv = v_to_f32(Vh[(long long)row * D + j], vscale);
      }
      ks[r][j] = kv;
      vs[r][j] = vv;
    }
    if (tid < TK) {
      const int row = t0 + tid;
      int g = -1;
      if (row < k1) {
        int lo = 0, hi = c_k - 1;  // largest b with okl[b] <= row
        while (lo < hi) {
          int mid = (lo + hi + 1) >> 1;
          if (okl[mid] <= row) lo = mid;
          else hi = mid - 1;
        }
        g = lo;
      }
      kgrp[tid] = g;
    }
    __syncthreads();
    float s[TK];
    bool in[TK];
    float tS = NEG, tU = NEG;
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) acc = fmaf(q[i], ks[j][sl * DPL + i], acc);
      acc += __shfl_xor(acc, 1);
      acc += __shfl_xor(acc, 2);
      const int g = kgrp[j];
      const bool ok_key = g >= 0;
      in[j] = ok_key && ((mask[p][g >> 5] >> (g & 31)) & 1u);
      s[j] = ok_key ? acc * scale_log2 : NEG;
      if (ok_key) {
        if (in[j]) tS = fmaxf(tS, s[j]);
        else tU = fmaxf(tU, s[j]);
      }
    }
    const float nS = fmaxf(mS, tS), nU = fmaxf(mU, tU);
    const float aS = nS == NEG ? 1.f : exp2f(mS - nS);
    const float aU = nU == NEG ? 1.f : exp2f(mU - nU);
    mS = nS;
    mU = nU;
    zS *= aS;
    zU *= aU;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      ns[i] *= aS;
      nu[i] *= aU;
    }
#pragma unroll
    for (int j = 0; j < TK; ++j) {
      const float e = s[j] == NEG ? 0.f : exp2f(s[j] - (in[j] ? mS : mU));
      const float eS = in[j] ? e : 0.f, eU = in[j] ? 0.f : e;
      zS += eS;
      zU += eU;
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        const float v = vs[j][sl * DPL + i];
        ns[i] = fmaf(eS, v, ns[i]);
        nu[i] = fmaf(eU, v, nu[i]);
      }
    }
  }
  if (p >= m) return;
  const long long rec = ((long long)h * kChunks + chunk) * m + p;
  if (sl == 0) {
    float* ps = part_s + rec * 4;
    ps[0] = mS;
    ps[1] = mU;
    ps[2] = zS;
    ps[3] = zU;
  }
  float* pn = part_n + rec * 2 * D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    pn[sl * DPL + i] = ns[i];
    pn[D + sl * DPL + i] = nu[i];
  }
}

// ---------------------------------------------------------------------------
// exact probe rows, bf16 inputs: MFMA version
// ---------------------------------------------------------------------------
// Four waves per block sweep one key chunk in 64-key tiles: wave w handles
// probes 32 (w & 1) .. +32 and half of the output dims (w >> 1), so every wave
// forms the scores of its 32 probes (the cheap part) and accumulates the
// numerators of its dims only.  Tiles are double buffered in LDS and loaded
// straight from global memory one tile ahead; the per-probe retained-key
// masks of a tile are built one tile ahead as well.  QK^T is a bf16 MFMA
// (exact products); each score is classified as retained (its K/V group is
// selected for the probe's query group) or omitted.  The retained and omitted
// classes keep separate running maxima.  PV runs on fp16 MFMA with P split
// into hi + lo halves, so the partial numerators carry ~2^-22 relative error.
template <int D>
__global__ __launch_bounds__(256, 2) void probe_rows_mfma_kernel(
    const uint16_t* __restrict__ q_g, const uint16_t* __restrict__ k_g,
    const uint16_t* __restrict__ v_g, const int32_t* __restrict__ v_shift,
    const int32_t* __restrict__ off_k, const int32_t* __restrict__ rowptr,
    const int32_t* __restrict__ col, const int32_t* __restrict__ probe_rows,
    const int32_t* __restrict__ probe_group, int n_q, int n_k, int c_q, int c_k, int m,
    float c2, float* __restrict__ part_s, float* __restrict__ part_n) {
  constexpr int CPR = D / 8, NS = D / 16, NDB = D / 32, NDH = NDB / 2;
  constexpr int RPI = 64 / CPR;       // tile rows per 1 KB wave load
  const int chunk = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, n = lane & 31,
            g = lane >> 5;
  const int ph = wid & 1, dh = wid >> 1;
  __shared__ uint4 kt0[64 * CPR], kt1[64 * CPR], vt0[64 * CPR], vt1[64 * CPR];
  __shared__ uint32_t mask[kMaxM][32];
  __shared__ int32_t okl[SPARSEPR_MAX_GROUPS + 1];
  __shared__ unsigned long long tmask[2][kMaxM];
  for (int i = tid; i < kMaxM * 32; i += 256) (&mask[0][0])[i] = 0u;
  const int32_t* ok = off_k + (long long)h * (c_k + 1);
  for (int i = tid; i <= c_k; i += 256) okl[i] = ok[i];
  __syncthreads();
  {
    const int pp = tid >> 2, quarter = tid & 3;
    if (pp < m && probe_rows[(long long)h * m + pp] >= 0) {
      const int grp = probe_group[(long long)h * m + pp];
      const int32_t* rp = rowptr + (long long)h * (c_q + 1);
      const int32_t* cl = col + (long long)h * c_q * c_k;
      for (int i = rp[grp] + quarter; i < rp[grp + 1]; i += 4) {
        const int b = cl[i];
        atomicOr(&mask[pp][b >> 5], 1u << (b & 31));
      }
    }
  }
  const int p = ph * 32 + n;
  const bool pvalid = p < m && probe_rows[(long long)h * m + p] >= 0;
  bf16x8_t qf[NS];
  {
    const int row = pvalid ? probe_rows[(long long)h * m + p] : 0;
    const uint16_t* qr = q_g + ((long long)h * n_q + row) * D;
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      const uint4 w = pvalid ? *reinterpret_cast<const uint4*>(qr + 16 * s2 + 8 * g)
                             : make_uint4(0, 0, 0, 0);
      qf[s2] = __builtin_bit_cast(bf16x8_t, w);
    }
  }
  const int per = (n_k + kChunks - 1) / kChunks;
  const int k0 = chunk * per, k1 = min(n_k, k0 + per);
  const uint32_t head_bytes = uint32_t(n_k) * D * 2;
  const v4i32_t krs =
      head_rsrc(reinterpret_cast<const char*>(k_g) + (long long)h * n_k * D * 2, head_bytes);
  const v4i32_t vrs =
      head_rsrc(reinterpret_cast<const char*>(v_g) + (long long)h * n_k * D * 2, head_bytes);
  const float NEG = -__builtin_huge_valf();
  const float slack = 8.f / c2;
  float mS = NEG, mU = NEG, zS = 0.f, zU = 0.f;
  f32x16_t oS[NDH], oU[NDH];
#pragma unroll
  for (int i = 0; i < NDH; ++i) oS[i] = oU[i] = f32x16_t{};

  // wave w moves tile rows 16 w .. 16 w + 15 of K and of V (rows past the
  // head's end read as zero; rows past the chunk are masked by `tail`)
  auto issue = [&](int t0, uint4* kb, uint4* vb) __attribute__((always_inline)) {
    const int lrow = lane / CPR, lpc = lane % CPR;
#pragma unroll
    for (int i = 0; i < 16 / RPI; ++i) {
      const int r0 = wid * 16 + i * RPI;
      const int r = r0 + lrow;
      const uint32_t roff = uint32_t(t0 + r) * (D * 2);
      lds_dma16(krs, __builtin_amdgcn_readfirstlane(lds_addr_of(kb + r0 * CPR)),
                roff + (lpc ^ (r & (CPR - 1))) * 16);
      lds_dma16(vrs, __builtin_amdgcn_readfirstlane(lds_addr_of(vb + r0 * CPR)),
                roff + (lpc ^ swz_v<D>(r)) * 16);
    }
  };
  // retained-key mask of the tile at t0 for probe tid (tid < kMaxM); gb walks
  // the K/V groups forward (the tiles of a chunk are visited in order)
  int gb = 0;
  if (tid < kMaxM) {
    int lo = 0, hi = c_k - 1;   // group of key k0: largest b with okl[b] <= k0
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (okl[mid] <= k0) lo = mid;
      else hi = mid - 1;
    }
    gb = lo;
  }
  auto tile_mask = [&](int t0, unsigned long long* out) __attribute__((always_inline)) {
    if (tid >= kMaxM) return;
    unsigned long long bits = 0ull;
    while (gb < c_k - 1 && okl[gb + 1] <= t0) ++gb;
    if (tid < m && probe_rows[(long long)h * m + tid] >= 0) {
      const int last = min(t0 + 64, k1) - 1;
      for (int b = gb; b < c_k && okl[b] <= last; ++b) {
        if (!((mask[tid][b >> 5] >> (b & 31)) & 1u)) continue;
        const int a0 = max(okl[b], t0) - t0, a1 = min(okl[b + 1], last + 1) - t0;
        if (a1 <= a0) continue;
        const unsigned long long span = a1 - a0 >= 64 ? ~0ull : ((1ull << (a1 - a0)) - 1ull);
        bits |= span << a0;
      }
    }
    out[tid] = bits;
  };

  // Q fragments complete before any tile load is in flight (vmcnt counts both)
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();   // group masks complete
  if (k0 < k1) {
    issue(k0, kt0, vt0);
    tile_mask(k0, tmask[0]);
  }
  auto step = [&](auto stage, int t0) __attribute__((always_inline)) {
    constexpr int stg = decltype(stage)::value;
    // tile t0 in its stage and its masks visible; every wave is past the
    // previous tile, whose stage now receives the next one
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t0 + 64 < k1) {
      if constexpr (stg == 0) issue(t0 + 64, kt1, vt1);
      else issue(t0 + 64, kt0, vt0);
      tile_mask(t0 + 64, tmask[stg ^ 1]);
    }
    const uint4* kt = stg == 0 ? kt0 : kt1;
    const uint4* vt = stg == 0 ? vt0 : vt1;
    f32x16_t s0, s1;
    const int tail = k1 - t0;
    // scores of the tile; keys at or past the chunk end take no part: their
    // scores become -inf, so they raise no maximum and their exponentials are
    // 0 in both classes (this and the passes below are branch-free: selects,
    // no conditional exponentials)
    auto scores = [&]() __attribute__((always_inline)) {
      s0 = f32x16_t{};
      s1 = f32x16_t{};
#pragma unroll
      for (int s2 = 0; s2 < NS; ++s2) {
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag<D>(kt, n, s2, g), qf[s2], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag<D>(kt, 32 + n, s2, g), qf[s2], s1, 0,
                                                     0, 0);
      }
      if (tail < 64) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (c_key(0, r, g) >= tail) s0[r] = NEG;
          if (c_key(1, r, g) >= tail) s1[r] = NEG;
        }
      }
    };
    scores();
    // this lane's 16 keys of each 32-key block as a 16-bit retained mask:
    // keys 8 (r / 4) + 4 g + r % 4 of block 0 and 32 + the same of block 1
    const unsigned long long bits64 = tmask[stg][p];
    uint32_t mb0 = 0, mb1 = 0;
    {
      const uint32_t lo = uint32_t(bits64) >> (4 * g), hi = uint32_t(bits64 >> 32) >> (4 * g);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        mb0 |= ((lo >> (8 * q4)) & 0xfu) << (4 * q4);
        mb1 |= ((hi >> (8 * q4)) & 0xfu) << (4 * q4);
      }
    }
    // Class references are lazy: a tile's exponents x = s c2 - reference
    // (log2 units) are formed against the running references as they stand,
    // and the class maxima of x are taken only on a tile where a class
    // appears for the first time in the chunk or some x exceeds 8 (a score
    // past its reference by more than the slack).  There a class with a
    // reference raises it by d = max(class max of x, 0) and a new class takes
    // its maximum as the reference; the running sums and numerators scale by
    // 2^-d and the exponents drop by d.  Any reference gives the same sums; a
    // reference is always a score seen (at most the class's running maximum)
    // and never more than the slack below it, so every exponential stays at
    // or below 2^8 and the class's largest at or above 1.
    {
      const float offS = mS == NEG ? 0.f : -mS * c2, offU = mU == NEG ? 0.f : -mU * c2;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ia = (mb0 >> r) & 1u, ib = (mb1 >> r) & 1u;
        s0[r] = __builtin_fmaf(s0[r], c2, ia ? offS : offU);
        s1[r] = __builtin_fmaf(s1[r], c2, ib ? offS : offU);
      }
    }
    float xmax = NEG;
#pragma unroll
    for (int r = 0; r < 16; ++r) xmax = fmaxf(xmax, fmaxf(s0[r], s1[r]));
    // a class with keys in this lane's part of the tile and no reference yet
    // (keys past the chunk end count as omitted here: harmless, they only
    // send the tile down the branch below)
    const bool first = (mS == NEG && (mb0 | mb1) != 0u) || (mU == NEG && (mb0 & mb1) != 0xffffu);
    if (__ballot(first || !(xmax <= 8.f))) {
      float tS = NEG, tU = NEG;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ia = (mb0 >> r) & 1u, ib = (mb1 >> r) & 1u;
        tS = fmaxf(tS, fmaxf(ia ? s0[r] : NEG, ib ? s1[r] : NEG));
        tU = fmaxf(tU, fmaxf(ia ? NEG : s0[r], ib ? NEG : s1[r]));
      }
      tS = fmaxf(tS, __shfl_xor(tS, 32));
      tU = fmaxf(tU, __shfl_xor(tU, 32));
      // no key of the class here: no change (d = 0)
      const float dS = tS == NEG ? 0.f : (mS == NEG ? tS : fmaxf(tS, 0.f));
      const float dU = tU == NEG ? 0.f : (mU == NEG ? tU : fmaxf(tU, 0.f));
      const float aS = mS == NEG ? 1.f : __builtin_amdgcn_exp2f(-dS);
      const float aU = mU == NEG ? 1.f : __builtin_amdgcn_exp2f(-dU);
      if (tS != NEG) mS = mS == NEG ? tS / c2 : mS + dS / c2;
      if (tU != NEG) mU = mU == NEG ? tU / c2 : mU + dU / c2;
      zS *= aS;
      zU *= aU;
#pragma unroll
      for (int db = 0; db < NDH; ++db) {
        oS[db] *= aS;
        oU[db] *= aU;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ia = (mb0 >> r) & 1u, ib = (mb1 >> r) & 1u;
        s0[r] -= ia ? dS : dU;
        s1[r] -= ib ? dS : dU;
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = __builtin_amdgcn_exp2f(s0[r]);
      s1[r] = __builtin_amdgcn_exp2f(s1[r]);
    }
    // P as hi + lo fp16 halves, two keys per 32-bit word; the class of each
    // half is a 16-bit mask (sign-extended key bit), so one AND moves a word
    // into the retained or the omitted operand, and the class sums are taken
    // from the same halves the products use
    const f16x2_t one2 = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t sh[4], sl[4], uh[4], ul[4];
      const uint32_t mu = (u >> 1) ? mb1 : mb0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int r0 = 8 * (u & 1) + 2 * jj;
        const float e0 = (u >> 1) ? s1[r0] : s0[r0];
        const float e1 = (u >> 1) ? s1[r0 + 1] : s0[r0 + 1];
        const _Float16 h0 = static_cast<_Float16>(e0), h1 = static_cast<_Float16>(e1);
        const _Float16 l0 = static_cast<_Float16>(e0 - float(h0));
        const _Float16 l1 = static_cast<_Float16>(e1 - float(h1));
        const uint32_t hw = __builtin_bit_cast(uint32_t, f16x2_t{h0, h1});
        const uint32_t lw = __builtin_bit_cast(uint32_t, f16x2_t{l0, l1});
        const uint32_t m0 = uint32_t(int32_t(mu << (31 - r0)) >> 31);
        const uint32_t m1 = uint32_t(int32_t(mu << (30 - r0)) >> 31);
        const uint32_t mw = (m0 & 0x0000ffffu) | (m1 & 0xffff0000u);
        sh[jj] = hw & mw;
        sl[jj] = lw & mw;
        uh[jj] = hw & ~mw;
        ul[jj] = lw & ~mw;
        zS = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, sh[jj]), one2, zS, false);
        zS = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, sl[jj]), one2, zS, false);
        zU = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, uh[jj]), one2, zU, false);
        zU = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, ul[jj]), one2, zU, false);
      }
      const f16x8_t fsh = __builtin_bit_cast(f16x8_t, sh), fsl = __builtin_bit_cast(f16x8_t, sl);
      const f16x8_t fuh = __builtin_bit_cast(f16x8_t, uh), ful = __builtin_bit_cast(f16x8_t, ul);
#pragma unroll
      for (int db = 0; db < NDH; ++db) {
        const f16x8_t vf = v_frag<D>(vt, lane, u, dh * NDH + db);
        oS[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, fsh, oS[db], 0, 0, 0);
        oS[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, fsl, oS[db], 0, 0, 0);
        oU[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, fuh, oU[db], 0, 0, 0);
        oU[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, ful, oU[db], 0, 0, 0);
      }
    }
  };
  for (int t0 = k0; t0 < k1; t0 += 128) {
    step(std::integral_constant<int, 0>{}, t0);
    if (t0 + 64 < k1) step(std::integral_constant<int, 1>{}, t0 + 64);
  }
  zS += __shfl_xor(zS, 32);
  zU += __shfl_xor(zU, 32);
  if (p >= m) return;
  const long long rec = ((long long)h * kChunks + chunk) * m + p;
  if (g == 0 && dh == 0) {
    float* ps = part_s + rec * 4;
    ps[0] = mS == NEG ? NEG : mS * c2;
    ps[1] = mU == NEG ? NEG : mU * c2;
    ps[2] = zS;
    ps[3] = zU;
  }
  const float vs = __builtin_ldexpf(1.f, v_shift[h]);
  float* pn = part_n + rec * 2 * D;
#pragma unroll
  for (int db = 0; db < NDH; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dd = 32 * (dh * NDH + db) + 8 * (r >> 2) + 4 * g + (r & 3);
      pn[dd] = oS[db][r] * vs;
      pn[D + dd] = oU[db][r] * vs;
    }
}

// ---------------------------------------------------------------------------
// merge chunks (fp64): O_dense, O_sp and R at every probe
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_s,
                                                   const float* __restrict__ part_n, int m,
                                                   int me, int d, float* __restrict__ o_dense,
                                                   float* __restrict__ o_sparse,
                                                   double* __restrict__ xp,
                                                   double* __restrict__ rp) {
  const int p = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  if (p >= me) return;
  __shared__ double fS[kChunks], fU[kChunks];
  __shared__ double sh[4];  // MS, MU, zS, zU
  const float NEGF = -__builtin_huge_valf();
  if (tid < 64) {
    // running maxima and partition sums over the chunks (one wave)
    double ms = -__builtin_huge_val(), mu = -__builtin_huge_val();
    for (int c = tid; c < kChunks; c += 64) {
      const float* ps = part_s + (((long long)h * kChunks + c) * m + p) * 4;
      ms = fmax(ms, double(ps[0]));
      mu = fmax(mu, double(ps[1]));
    }
    ms = wave_max(ms);
    mu = wave_max(mu);
    double zs = 0.0, zu = 0.0;
    for (int c = tid; c < kChunks; c += 64) {
      const float* ps = part_s + (((long long)h * kChunks + c) * m + p) * 4;
      const double a = ps[0] == NEGF ? 0.0 : exp2(double(ps[0]) - ms);
      const double b = ps[1] == NEGF ? 0.0 : exp2(double(ps[1]) - mu);
      fS[c] = a;
      fU[c] = b;
      zs += a * ps[2];
      zu += b * ps[3];
    }
    zs = wave_sum(zs);
    zu = wave_sum(zu);
    if (tid == 0) {
      sh[0] = ms;
      sh[1] = mu;
      sh[2] = zs;
      sh[3] = zu;
    }
  }
  __syncthreads();
  const double MS = sh[0], MU = sh[1], zS = sh[2], zU = sh[3];
  // common reference for the dense row
  const double M = fmax(MS, MU);
  const double wS = MS == -__builtin_huge_val() ? 0.0 : exp2(MS - M);
  const double wU = MU == -__builtin_huge_val() ? 0.0 : exp2(MU - M);
  const double Z = zS * wS + zU * wU;
  for (int j = tid; j < d; j += 128) {
    double nS = 0, nU = 0;
    for (int c = 0; c < kChunks; ++c) {
      const float* pn = part_n + (((long long)h * kChunks + c) * m + p) * 2 * d;
      nS += fS[c] * pn[j];
      nU += fU[c] * pn[d + j];
    }
    const double x = nS / zS;
    const double od = (nS * wS + nU * wU) / Z;
    const double r = wU * (zS * nU - zU * nS) / (Z * zS);
    const long long o = ((long long)h * m + p) * d + j;
    o_dense[o] = float(od);
    if (o_sparse) o_sparse[o] = float(x);
    xp[o] = x;
    rp[o] = r;
  }
}

// ---------------------------------------------------------------------------
// fit (fp64, one block per head)
// ---------------------------------------------------------------------------
struct FitArgs {
  const int32_t* off_q;
  const int32_t* m_a;
  const int32_t* probe_group;
  const double* xp;   // [H][m][d]
  const double* rp;   // [H][m][d]
  double* xw;         // [H][m][d] scratch
  double* rw;         // [H][m][d] scratch
  double* zbuf;       // [H][64][64] scratch
  double* abuf;       // [H][d][64] scratch (A, fp64)
  double* pbuf;       // [H][d][64] scratch (Psi, fp64)
  float* corr_a;
  float* corr_psi_t;
  float* corr_c;
  float* corr_g;      // [H][d] diagonal gain (may be null for the full estimator)
  int c_q, m, me, d, rank;
  int estimator;      // SPARSEPR_EST_*
  double lambda;
};

constexpr int kLd = kMaxM + 1;
constexpr int kFitThreads = 512;   // threads of the fit kernel (8 waves, 2 per SIMD)
typedef double f64x4_t __attribute__((ext_vector_type(4)));
// Value of lane (lane & ~3) + q of the quad (q uniform).
SPR_DEV double quad_bcast_f64(double v, int q) {
  switch (q) {
    case 0: return dpp_f64<0x00>(v);
    case 1: return dpp_f64<0x55>(v);
    case 2: return dpp_f64<0xAA>(v);
    default: return dpp_f64<0xFF>(v);
  }
}

// v[i] for a uniform runtime i, as a chain of selects on register values
// (the empty asm keeps the compiler from turning the chain into an indexed
// load, which would move the whole array to scratch memory)
SPR_DEV double pick16(const double (&v)[16], int i) {
  double r = v[0];
#pragma unroll
  for (int t = 1; t < 16; ++t) {
    double x = v[t];
    asm volatile("" : "+v"(x));
    r = i == t ? x : r;
  }
  return r;
}

// U = H_0 ... H_(n-3) Z for `cap` vectors (rows c of zs): groups of GB
// lanes per vector, lane g keeps elements g*EPL .. +EPL in registers.
template <int GB>
SPR_DEV void back_transform(double* zs, const double* vs, const double* tbeta, int n, int cap,
                            int tid) {
  constexpr int EPL = 64 / GB;
  const int c = tid / GB, g = tid % GB;
  if (c >= cap) return;
  double* zc = zs + c * kLd;
  const int i0 = g * EPL;
  double zv[EPL];
#pragma unroll
  for (int t = 0; t < EPL; ++t) zv[t] = i0 + t < n ? zc[i0 + t] : 0.0;
  for (int k = n - 3; k >= 0; --k) {
    const double bk = tbeta[k];
    if (bk == 0.0) continue;   // uniform: tbeta is shared
    const double* vk = vs + k * kLd;
    double vv[EPL];
    double dot = 0.0;
#pragma unroll
    for (int t = 0; t < EPL; ++t) {
      const int i = i0 + t;
      vv[t] = i > k && i < n ? vk[i] : 0.0;
      dot = fma(vv[t], zv[t], dot);
    }
    dot = group_sum_any<GB>(dot);
    const double tt = bk * dot;
#pragma unroll
    for (int t = 0; t < EPL; ++t) zv[t] = fma(-tt, vv[t], zv[t]);
  }
#pragma unroll
  for (int t = 0; t < EPL; ++t)
    if (i0 + t < n) zc[i0 + t] = zv[t];
}


__global__ __launch_bounds__(kFitThreads) void fit_kernel(FitArgs f) {
  const int h = blockIdx.x, tid = threadIdx.x;
  const int me = f.me, d = f.d;
  const int lane = tid & 63, wid = tid >> 6;
  __shared__ double w[kMaxM], sqw[kMaxM];
  __shared__ double mux[128], mur[128], sc[128], isc[128];
  __shared__ double part[2][256];
  // pool: X and R staged (phases 1-4), then G / G^-1, E / Householder
  // vectors, eigenvector rows Zs, scratch rows Ws
  __shared__ __align__(16) double pool[4 * kMaxM * kLd];
  double* G = pool;
  double* E = pool + kMaxM * kLd;
  double* Zs = pool + 2 * kMaxM * kLd;
  double* Ws = pool + 3 * kMaxM * kLd;
  __shared__ double gjrow[2][2][kMaxM];   // Gauss-Jordan pivot row (A part, B part), by parity
  __shared__ double colE[2][kMaxM], pbuf[2][kMaxM];
  __shared__ double td[kMaxM], te[kMaxM], tbeta[kMaxM];      // T and the reflectors
  __shared__ double tdn[kMaxM], ten[kMaxM];                   // normalised T
  __shared__ double2 st2[kMaxM];                              // (d_(i+1), e_i^2), normalised
  __shared__ double lamn[kMaxM], tbuf[kMaxM];
  __shared__ double red[kFitThreads / 64];
  __shared__ double tcol[kMaxM];
  __shared__ double sh_sw;
  __shared__ int32_t sh_k;

  const double* X = f.xp + (long long)h * f.m * d;
  const double* R = f.rp + (long long)h * f.m * d;
  double* Xw = f.xw + (long long)h * f.m * d;
  double* Rw = f.rw + (long long)h * f.m * d;
  const int ldx = d + 1;            // padded row stride of the staged X and R
  double* Xs = pool;                // me x ldx
  double* Rs = pool + 2 * kMaxM * kLd;

  // 1. coverage weights |G_a| / m_a and their sum; X and R staged in LDS
  const int32_t* oq = f.off_q + (long long)h * (f.c_q + 1);
  if (tid < me) {
    const int a = f.probe_group[(long long)h * f.m + tid];
    w[tid] = double(oq[a + 1] - oq[a]) / double(f.m_a[(long long)h * f.c_q + a]);
  }
  {
    // 16-byte loads, all in flight before the first store (me * d / 2 <= 4096)
    const int n2 = me * d / 2;
    constexpr int NL = 4096 / kFitThreads;
    double2 xv[NL], rv[NL];
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int e = tid + kFitThreads * t;
      xv[t] = e < n2 ? reinterpret_cast<const double2*>(X)[e] : double2{0.0, 0.0};
      rv[t] = e < n2 ? reinterpret_cast<const double2*>(R)[e] : double2{0.0, 0.0};
    }
#pragma unroll
    for (int t = 0; t < NL; ++t) {
      const int e = tid + kFitThreads * t;
      if (e < n2) {
        const int p = (2 * e) / d, j = 2 * e - p * d;
        Xs[p * ldx + j] = xv[t].x;
        Xs[p * ldx + j + 1] = xv[t].y;
        Rs[p * ldx + j] = rv[t].x;
        Rs[p * ldx + j + 1] = rv[t].y;
      }
    }
  }
  __syncthreads();
  if (wid == 0) {
    const double sw = wave_sum_f64(lane < me ? w[lane] : 0.0);
    if (lane == 0) sh_sw = sw;
  }
  __syncthreads();
  const double sw = sh_sw;
  if (tid < me) sqw[tid] = sqrt(double(me) * w[tid] / sw);   // sqrt of the unit-mean weight
  // 2. weighted means and feature scale (unit-sum weights): column j = tid % d,
  // the NP = 256 / d threads of a column take rows p = tid / d (+ NP)
  const int NP = 256 / d, jc = tid % d, pp0 = tid / d;
  if (tid < 256) {
    double mx = 0.0, mr = 0.0;
    for (int p = pp0; p < me; p += NP) {
      const double wh = w[p] / sw;
      mx = fma(wh, Xs[p * ldx + jc], mx);
      mr = fma(wh, Rs[p * ldx + jc], mr);
    }
    part[0][tid] = mx;
    part[1][tid] = mr;
  }
  __syncthreads();
  if (tid < d) {
    double mx = 0.0, mr = 0.0;
    for (int i = 0; i < NP; ++i) {
      mx += part[0][tid + i * d];
      mr += part[1][tid + i * d];
    }
    mux[tid] = mx;
    mur[tid] = mr;
  }
  __syncthreads();
  if (tid < 256) {
    const double mx = mux[jc];
    double var = 0.0;
    for (int p = pp0; p < me; p += NP) {
      const double t = Xs[p * ldx + jc] - mx;
      var = fma(w[p] / sw * t, t, var);
    }
    part[0][tid] = var;
  }
  __syncthreads();
  if (tid < d) {
    double var = 0.0;
    for (int i = 0; i < NP; ++i) var += part[0][tid + i * d];
    sc[tid] = sqrt(var + 1e-6);
    isc[tid] = 1.0 / sc[tid];
  }
  __syncthreads();
  // 3. weighted, standardised features and centred residuals, in place in
  // LDS (rows past me are zero) and to global memory for the last step
  for (int e = tid; e < kMaxM * d; e += kFitThreads) {
    const int p = e / d, j = e - p * d;
    double xv = 0.0, rv = 0.0;
    if (p < me) {
      xv = sqw[p] * (Xs[p * ldx + j] - mux[j]) * isc[j];
      rv = sqw[p] * (Rs[p * ldx + j] - mur[j]);
      Xw[p * d + j] = xv;
      Rw[p * d + j] = rv;
    }
    Xs[p * ldx + j] = xv;
    Rs[p * ldx + j] = rv;
  }
  __syncthreads();
  float* ocg = f.corr_g ? f.corr_g + (long long)h * d : nullptr;
  if (f.estimator != SPARSEPR_EST_FULL) {
    // restricted estimators ([paper] §5 Table 4, App. D.4): B = 0 (mean),
    // a I (scalar, penalty lam d a^2) or diag(b) (diagonal), each minimising
    // sum_p w~_p |Rbar_p - xbar_p B|^2 + lam |B|_F^2; folded to
    // out = o + g * o + c with g = diag(B) / s, c = mu_R - mu_x * g
    double sxr = 0.0, sxx = 0.0;
    if (tid < d)
      for (int p = 0; p < me; ++p) {
        const double xv = Xs[p * ldx + tid], rv = Rs[p * ldx + tid];
        sxr = fma(xv, rv, sxr);
        sxx = fma(xv, xv, sxx);
      }
    const double tr = block_sum(sxr, red);
    const double tx = block_sum(sxx, red);
    if (tid < d) {
      double b = 0.0;
      if (f.estimator == SPARSEPR_EST_SCALAR) b = tr / (tx + f.lambda * double(d));
      else if (f.estimator == SPARSEPR_EST_DIAGONAL) b = sxr / (sxx + f.lambda);
      const double g = b / sc[tid];
      if (ocg) ocg[tid] = float(g);
      f.corr_c[(long long)h * d + tid] = float(mur[tid] - mux[tid] * g);
    }
    for (int e = tid; e < d * f.rank; e += kFitThreads) {
      f.corr_a[(long long)h * d * f.rank + e] = 0.f;
      f.corr_psi_t[(long long)h * f.rank * d + e] = 0.f;
    }
    return;
  }
  if (ocg)
    for (int j = tid; j < d; j += 256) ocg[j] = 0.f;
  // 4. Gram matrices G = Xw Xw^T + lam I and E = Rw Rw^T on fp64 MFMA
  // (v_mfma_f64_16x16x4: operand lane l holds row l % 16 at k = l / 16;
  // result lane l holds column l % 16 of rows l / 16 + 4 i): wave w forms
  // rows 16 w .. 16 w + 15 of both.
  {
    const int r16 = lane & 15, kq = lane >> 4;
    const int gw = wid & 3;   // only waves 0..3 form products
    f64x4_t gacc[4], eacc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) gacc[t] = eacc[t] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    for (int kk = 0; wid < 4 && kk < d; kk += 4) {
      const double ax = Xs[(16 * gw + r16) * ldx + kk + kq];
      const double ar = Rs[(16 * gw + r16) * ldx + kk + kq];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const double bx = Xs[(16 * t + r16) * ldx + kk + kq];
        const double br = Rs[(16 * t + r16) * ldx + kk + kq];
        gacc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(ax, bx, gacc[t], 0, 0, 0);
        eacc[t] = __builtin_amdgcn_mfma_f64_16x16x4f64(ar, br, eacc[t], 0, 0, 0);
      }
    }
    __syncthreads();   // X and R are no longer read; G and E overwrite them
    if (wid < 4) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 16 * gw + kq + 4 * i, col = 16 * t + r16;
          G[row * kLd + col] = gacc[t][i] + (row == col ? f.lambda : 0.0);
          E[row * kLd + col] = eacc[t][i];
        }
    }
  }
  __syncthreads();
  // 5. One pass over k = 0 .. n-1 with two barriers per step does both
  //   a. Gauss-Jordan elimination of [G | I] (G is symmetric positive
  //      definite, so no pivoting; rows keep their scale, so the left half
  //      ends diagonal): afterwards row i of G^-1 is row i of the right half
  //      over the final a_ii;
  //   b. Householder reduction of E to tridiagonal form T = Q^T E Q: step k
  //      maps column k below the diagonal onto alpha e_1 with
  //      H = I - beta v v^T (v kept in row k of E; d, e in td, te).
  // Thread t keeps row t / RT, columns CW (t % RT) .. + CW - 1 of both
  // matrices in registers (RT = threads per row, CW = 64 / RT columns each):
  // the threads of a row are adjacent lanes of one DPP row.
  constexpr int RT = kFitThreads / 64, CW = 64 / RT;
  const int n = me;
  const int rr = tid / RT, qq = tid % RT, c0 = CW * qq;
  double ga[CW], gb[CW], er[CW];
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int j = c0 + i;
    const bool in = rr < n && j < n;
    ga[i] = in ? G[rr * kLd + j] : 0.0;
    gb[i] = in && rr == j ? 1.0 : 0.0;
    er[i] = in ? E[rr * kLd + j] : 0.0;
  }
  __syncthreads();   // E is reused for the Householder vectors below
  // step k = CW kb + KI: the register index KI is a compile-time constant
  auto elim_step = [&](auto ki_c, int kb) __attribute__((always_inline)) {
    constexpr int KI = decltype(ki_c)::value;
    const int k = CW * kb + KI;
    const int par = KI & 1;
    // publish: Gauss-Jordan pivot row k, column k of E
    if (rr == k) {
#pragma unroll
      for (int i = 0; i < CW; i += 2) {
        reinterpret_cast<double2*>(&gjrow[par][0][c0 + i])[0] = double2{ga[i], ga[i + 1]};
        reinterpret_cast<double2*>(&gjrow[par][1][c0 + i])[0] = double2{gb[i], gb[i + 1]};
      }
    }
    if (qq == kb && rr < n) colE[par][rr] = er[KI];
    __syncthreads();
    // a. rows i != k: row_i -= (a_ik / a_kk) row_k
    {
      const double aik = __shfl(ga[KI], (lane & ~(RT - 1)) | kb);
      const double fct = rr == k ? 0.0 : aik * rcp64(gjrow[par][0][k]);
#pragma unroll
      for (int i = 0; i < CW; i += 2) {
        const double2 ka = reinterpret_cast<const double2*>(&gjrow[par][0][c0 + i])[0];
        const double2 kbv = reinterpret_cast<const double2*>(&gjrow[par][1][c0 + i])[0];
        ga[i] = fma(-fct, ka.x, ga[i]);
        ga[i + 1] = fma(-fct, ka.y, ga[i + 1]);
        gb[i] = fma(-fct, kbv.x, gb[i]);
        gb[i + 1] = fma(-fct, kbv.y, gb[i + 1]);
      }
    }
    // b. Householder step k (k + 2 < n): x = E[k+1.., k]
    const int m = n - k - 1;
    const bool hh = k + 2 < n;
    double alpha = 0.0, beta = 0.0;
    double vj[CW];
    if (hh) {
      double xraw = colE[par][(k + 1 + lane) & (kMaxM - 1)];
      asm volatile("" : "+v"(xraw));
      const double xl = lane < m ? xraw : 0.0;
      const double x0 = colE[par][k + 1];
      const double nx2 = wave_sum_f64(xl * xl);
      if (nx2 > 0.0) {
        const double nx = sqrt(nx2);
        alpha = x0 > 0.0 ? -nx : nx;
        beta = rcp64(nx2 - alpha * x0);   // 2 / |v|^2, |v|^2 = 2 (|x|^2 - alpha x0)
      }
      if (wid == 0) {
        // v = x - alpha e_1, stored in row k of E (entries k+1 ..)
        if (lane < m) E[k * kLd + k + 1 + lane] = lane == 0 ? xl - alpha : xl;
        if (lane == 0) {
          td[k] = colE[par][k];
          te[k] = alpha;
          tbeta[k] = beta;
        }
      }
      // v at this thread's columns (0 outside k+1 .. n-1)
      double cv[CW];
#pragma unroll
      for (int i = 0; i < CW; i += 2) {
        const double2 c2 = reinterpret_cast<const double2*>(&colE[par][c0 + i])[0];
        cv[i] = c2.x;
        cv[i + 1] = c2.y;
      }
#pragma unroll
      for (int i = 0; i < CW; ++i) {
        const int j = c0 + i;
        vj[i] = j > k && j < n ? (j == k + 1 ? cv[i] - alpha : cv[i]) : 0.0;
      }
      if (beta != 0.0) {
        // p_r = beta sum_j E[r][j] v_j over j > k, RT threads per row
        double s2 = 0.0;
#pragma unroll
        for (int i = 0; i < CW; ++i) s2 = fma(er[i], vj[i], s2);
        s2 = group_sum_f64<RT>(s2);
        if (qq == 0 && rr > k && rr < n) pbuf[par][rr] = beta * s2;
      }
    }
    __syncthreads();
    if (hh && beta != 0.0) {
      // w = p - (beta/2)(p.v) v;  E22 <- E22 - v w^T - w v^T
      const int li = (k + 1 + lane) & (kMaxM - 1);
      double craw = colE[par][li], praw = pbuf[par][li];
      asm volatile("" : "+v"(craw), "+v"(praw));
      const double vl = lane < m ? (lane == 0 ? craw - alpha : craw) : 0.0;
      const double pl = lane < m ? praw : 0.0;
      const double K = 0.5 * beta * wave_sum_f64(pl * vl);
      if (rr > k && rr < n) {
        const double vr = rr == k + 1 ? colE[par][rr] - alpha : colE[par][rr];
        const double wr = pbuf[par][rr] - K * vr;
        double pj[CW];
#pragma unroll
        for (int i = 0; i < CW; i += 2) {
          const double2 p2 = reinterpret_cast<const double2*>(&pbuf[par][c0 + i])[0];
          pj[i] = p2.x;
          pj[i + 1] = p2.y;
        }
#pragma unroll
        for (int i = 0; i < CW; ++i) {
          const int j = c0 + i;
          const double wj = j > k && j < n ? pj[i] - K * vj[i] : 0.0;
          er[i] -= fma(vr, wj, wr * vj[i]);
        }
      }
    }
  };
  static_assert(CW == 8, "the unrolled steps below assume 8 columns per thread");
  for (int kb = 0; kb * CW < n; ++kb) {
    const int kn = n - CW * kb;   // steps left in this block (uniform)
    elim_step(std::integral_constant<int, 0>{}, kb);
    if (kn > 1) elim_step(std::integral_constant<int, 1>{}, kb);
    if (kn > 2) elim_step(std::integral_constant<int, 2>{}, kb);
    if (kn > 3) elim_step(std::integral_constant<int, 3>{}, kb);
    if (kn > 4) elim_step(std::integral_constant<int, 4>{}, kb);
    if (kn > 5) elim_step(std::integral_constant<int, 5>{}, kb);
    if (kn > 6) elim_step(std::integral_constant<int, 6>{}, kb);
    if (kn > 7) elim_step(std::integral_constant<int, 7>{}, kb);
  }
  // the final a_rr sits in column rr: lane (rr, rr / CW), register rr % CW
  {
    double arr = 0.0;
#pragma unroll
    for (int i = 0; i < CW; ++i) arr = c0 + i == rr ? ga[i] : arr;
    arr = group_sum_f64<RT>(arr);   // the row's threads: one holds a_rr, the rest 0
    const double ia = rr < n ? 1.0 / arr : 0.0;
#pragma unroll
    for (int i = 0; i < CW; ++i) gb[i] *= ia;
  }
  // G^-1 to LDS (rows of the right half); the last 2 x 2 block of T
#pragma unroll
  for (int i = 0; i < CW; ++i) {
    const int j = c0 + i;
    if (rr < n && j < n) G[rr * kLd + j] = gb[i];
    if (n >= 2 && rr == n - 2 && j == n - 2) td[n - 2] = er[i];
    if (n >= 2 && rr == n - 1 && j == n - 2) te[n - 2] = er[i];
    if (rr == n - 1 && j == n - 1) td[n - 1] = er[i];
  }
  if (tid == 0) {
    te[n - 1] = 0.0;
    if (n >= 2) tbeta[n - 2] = 0.0;
    tbeta[n - 1] = 0.0;
  }
  __syncthreads();
  // 6. Leading eigenpairs of T (and so of E):
  //   a. the `cap` largest eigenvalues by multisection of Sturm counts: the
  //      lanes of one wave share a target and test points of its interval;
  //   b. each eigenvector of T from the twisted factorisation of T - lambda I
  //      (forward and backward pivots; the twist where |gamma| is smallest);
  //   c. the vectors are checked for orthogonality; a set that is not (close
  //      eigenvalues) is re-orthogonalised, and a vector lost that way is
  //      recomputed by inverse iteration orthogonal to the earlier ones;
  //   d. back-transformation U = H_0 H_1 ... H_(n-3) Z.
  int cap = f.rank < n ? f.rank : n;
  cap = cap < d ? cap : d;
  // Gershgorin bounds of T; T is normalised by tn = max |bound|
  double glo = __builtin_huge_val(), ghi = -__builtin_huge_val();
  if (tid < n) {
    const double rad = (tid > 0 ? fabs(te[tid - 1]) : 0.0) + (tid + 1 < n ? fabs(te[tid]) : 0.0);
    glo = td[tid] - rad;
    ghi = td[tid] + rad;
  }
  glo = block_min(glo, red);
  ghi = block_max(ghi, red);
  const double tn = fmax(fabs(glo), fabs(ghi));
  if (tn > 0.0) {
    if (tid < kMaxM) lamn[tid] = 0.0;
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
      // wave-uniform stop: every active interval at the rounding level of |T|
      const bool done = !act || (b - a) <= 2.0 * kEps64 * fmax(fabs(a), fabs(b)) + 4.0 * kEps64;
      if (__all(done)) break;
      // 2 P interior points of [a, b], two per lane
      const double x1 = a + (b - a) * (double(2 * s + 1) / double(2 * P + 1));
      const double x2 = a + (b - a) * (double(2 * s + 2) / double(2 * P + 1));
      int c1 = 0, c2 = 0;
      if (act) sturm_count2(d0, st2, n, x1, x2, c1, c2);
      // new interval: largest point with count <= target, smallest point
      // with count > target (over the P lanes of the target)
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
    // b. twisted factorisation, one thread per target: forward pivots Dp
    // (kept in Ws), ratios e_i / Dp_i (kept in Zs); backward pivots Dm with
    // gamma_i = Dp_i + Dm_i - (d_i - mu), ratios e_(i-1) / Dm_i (kept in Ws)
    if (tid < cap) {
      const int c = tid;
      const double mu = lamn[c];
      double* zr = Zs + c * kLd;
      double* wr = Ws + c * kLd;
      double dp = tdn[0] - mu;
      wr[0] = dp;
      for (int i = 1; i < n; ++i) {
        const double2 s2 = st2[i - 1];            // (d_i, e_(i-1)^2)
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
      // z: z_rt = 1, z_i = -(e_i / Dp_i) z_(i+1) below, -(e_(i-1) / Dm_i) z_(i-1) above
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
    // c. orthogonality of the computed vectors
    double worst = 0.0;
    for (int e = tid; e < cap * cap; e += kFitThreads) {
      const int c1 = e / cap, c2 = e - c1 * cap;
      if (c2 <= c1) {
        double dot = 0.0;
        for (int i = 0; i < n; ++i) dot = fma(Zs[c1 * kLd + i], Zs[c2 * kLd + i], dot);
        const double dev = c2 == c1 ? fabs(dot - 1.0) : fabs(dot);
        worst = dev == dev ? fmax(worst, dev) : 1.0;   // NaN counts as lost
      }
    }
    worst = block_max(worst, red);
    if (!(worst <= 1e-10) && wid == 0) {
      // rare: classical Gram-Schmidt twice, in descending order; a vector
      // that loses more than half its norm is recomputed by inverse
      // iteration (Thomas solves of T - mu I) kept orthogonal to the earlier
      // ones.  Lanes hold vector elements.
      for (int c = 0; c < cap; ++c) {
        double* zc = Zs + c * kLd;
        double zi = lane < n ? zc[lane] : 0.0;
        if (!(zi == zi)) zi = 0.0;
        auto orth = [&](double v) {
          for (int pass = 0; pass < 2; ++pass)
            for (int c2 = 0; c2 < c; ++c2) {
              const double u = lane < n ? Zs[c2 * kLd + lane] : 0.0;
              v -= wave_sum_f64(u * v) * u;
            }
          return v;
        };
        zi = orth(zi);
        double nz = sqrt(wave_sum_f64(zi * zi));
        if (!(nz >= 0.5)) {
          const double mu = lamn[c];
          // deterministic start: a fixed pseudo-random vector per target
          uint32_t hsh = uint32_t(lane * 2654435761u) ^ uint32_t((c + 1) * 40503u);
          hsh ^= hsh >> 13;
          hsh *= 0x5bd1e995u;
          hsh ^= hsh >> 15;
          zi = lane < n ? double(int32_t(hsh & 0xffff) - 32768) : 0.0;
          for (int it = 0; it < 4; ++it) {
            zi = orth(zi);
            if (lane < n) Ws[lane] = zi;
            if (lane == 0) {
              // (T - mu I) y = b, LU without pivoting, tiny pivots raised
              double u_prev = tdn[0] - mu;
              if (fabs(u_prev) < kEps64) u_prev = kEps64;
              tbuf[0] = u_prev;
              for (int i = 1; i < n; ++i) {
                const double l = ten[i - 1] / u_prev;
                double u = (tdn[i] - mu) - l * ten[i - 1];
                if (fabs(u) < kEps64) u = kEps64;
                Ws[i] -= l * Ws[i - 1];
                tbuf[i] = u;
                u_prev = u;
              }
              Ws[n - 1] /= tbuf[n - 1];
              for (int i = n - 2; i >= 0; --i) Ws[i] = (Ws[i] - ten[i] * Ws[i + 1]) / tbuf[i];
            }
            zi = lane < n ? Ws[lane] : 0.0;
            const double nn = sqrt(wave_sum_f64(zi * zi));
            zi = nn > 0.0 ? zi / nn : 0.0;
          }
          zi = orth(zi);
          nz = sqrt(wave_sum_f64(zi * zi));
        }
        zi = nz > 0.0 ? zi / nz : 0.0;
        if (lane < n) zc[lane] = zi;
      }
    }
    __syncthreads();
    // d. U = H_0 ... H_(n-3) Z
    // GB lanes per vector with GB * cap <= kFitThreads
    static_assert(kFitThreads == 512, "back-transformation groups assume 512 threads");
    if (cap <= 8) back_transform<64>(Zs, E, tbeta, n, cap, tid);
    else if (cap <= 16) back_transform<32>(Zs, E, tbeta, n, cap, tid);
    else if (cap <= 32) back_transform<16>(Zs, E, tbeta, n, cap, tid);
    else back_transform<8>(Zs, E, tbeta, n, cap, tid);
  } else {
    if (tid < kMaxM) lamn[tid] = 0.0;
  }
  __syncthreads();
  // 7. kept directions: descending eigenvalues above the resolution of the
  // Gram route (64 eps lambda_1) and with sigma > 1e-10 sigma_1
  if (tid == 0) {
    const double l1 = lamn[0] * tn;
    const double s1 = l1 > 0 ? sqrt(l1) : 0.0;
    int k = 0;
    if (s1 > 0) {
      const double floor_l = 64.0 * 2.220446049250313e-16 * l1;
      for (int i = 0; i < cap; ++i) {
        const double li = lamn[i] * tn;
        if (li > floor_l && sqrt(li) > 1e-10 * s1) ++k;
        else break;
      }
    }
    sh_k = k;
  }
  __syncthreads();
  const int k = sh_k;
  // 8. y_c = G^-1 (u_c sigma_c), into row c of Ws
  for (int e = tid; e < k * n; e += kFitThreads) {
    const int c = e / n, i = e - c * n;
    const double sig = sqrt(lamn[c] * tn);
    double s = 0.0;
    for (int p = 0; p < n; ++p) s = fma(G[i * kLd + p], Zs[c * kLd + p], s);
    Ws[c * kLd + i] = s * sig;
  }
  __syncthreads();
  // A[:, c] = diag(1/s) Xw^T y_c,  Psi[:, c] = Rw^T u_c / sigma_c: Xw and Rw
  // staged again into the free G and E areas; thread (column j, c-phase)
  // runs over the probes, CB c at a time
  double* Ab = f.abuf + (long long)h * d * kMaxM;
  double* Pb = f.pbuf + (long long)h * d * kMaxM;
  for (int pass = 0; pass < 2; ++pass) {
    const double* src = pass == 0 ? Xw : Rw;
    double* st = G;                      // me x d, contiguous over G and E
    {
      const int n2 = me * d / 2;
      constexpr int NL = 4096 / kFitThreads;
      double2 v2[NL];
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int e = tid + kFitThreads * t;
        v2[t] = e < n2 ? reinterpret_cast<const double2*>(src)[e] : double2{0.0, 0.0};
      }
#pragma unroll
      for (int t = 0; t < NL; ++t) {
        const int e = tid + kFitThreads * t;
        if (e < n2) reinterpret_cast<double2*>(st)[e] = v2[t];
      }
    }
    __syncthreads();
    const double* vecs = pass == 0 ? Ws : Zs;
    // CB directions per thread: 4 keeps every thread busy for k = 16 at
    // d = 128 (8 left half of them idle)
    constexpr int CB = 4;
    for (int cb = (tid / d) * CB; cb < k; cb += (kFitThreads / d) * CB) {
      double acc[CB];
#pragma unroll
      for (int c = 0; c < CB; ++c) acc[c] = 0.0;
      for (int p = 0; p < me; ++p) {
        const double xv = st[p * d + jc];
#pragma unroll
        for (int c = 0; c < CB; ++c) {
          const int cc = cb + c < k ? cb + c : k - 1;
          acc[c] = fma(xv, vecs[cc * kLd + p], acc[c]);
        }
      }
#pragma unroll
      for (int c = 0; c < CB; ++c)
        if (cb + c < k) {
          if (pass == 0) Ab[jc * kMaxM + cb + c] = acc[c] * isc[jc];
          else Pb[jc * kMaxM + cb + c] = acc[c] / sqrt(lamn[cb + c] * tn);
        }
    }
    __syncthreads();
  }
  // 9. c = mu_R - (mu_x A) Psi^T
  if (tid < k) {
    double t = 0.0;
    for (int j = 0; j < d; ++j) t = fma(mux[j], Ab[j * kMaxM + tid], t);
    tcol[tid] = t;
  }
  __syncthreads();
  float* oa = f.corr_a + (long long)h * d * f.rank;
  float* op = f.corr_psi_t + (long long)h * f.rank * d;
  float* ocv = f.corr_c + (long long)h * d;
  for (int e = tid; e < d * f.rank; e += kFitThreads) {
    const int j = e / f.rank, c = e % f.rank;
    oa[e] = c < k ? float(Ab[j * kMaxM + c]) : 0.f;
  }
  for (int e = tid; e < f.rank * d; e += kFitThreads) {
    const int c = e / d, j = e % d;
    op[e] = c < k ? float(Pb[j * kMaxM + c]) : 0.f;
  }
  for (int j = tid; j < d; j += 256) {
    double v = mur[j];
    for (int c = 0; c < k; ++c) v -= tcol[c] * Pb[j * kMaxM + c];
    ocv[j] = float(v);
  }
}

// Probe features of a response-coupled partition: rows of `feat` (token
// order) copied to group-major order and their fp64 mean per group, so the
// select kernel measures distances in that space.  One block per group.
// With `chunked` (rows of whole 16-byte chunks, 16-byte aligned arrays),
// thread (ph, ch) copies chunk ch of rows ph, ph + phases, ...; otherwise
// thread (rl, j) handles feature j of rows rl, rl + 4, ....  Either way each
// thread adds its rows in order and the partials are combined in a fixed
// order.
__global__ __launch_bounds__(256) void feat_group_kernel(const float* __restrict__ feat,
                                                         const int32_t* __restrict__ perm_q,
                                                         const int32_t* __restrict__ off_q,
                                                         int n_q, int c_q, int fd, int chunked,
                                                         float* __restrict__ feat_g,
                                                         double* __restrict__ feat_cen) {
  const int a = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int32_t* o = off_q + (long long)h * (c_q + 1);
  const int lo = o[a], hi = o[a + 1];
  const int32_t* pr = perm_q + (long long)h * n_q;
  if (chunked) {
    // 16-byte chunks: thread (ph, ch) copies chunk ch of rows ph, ph + phases,
    // ... in order and adds them in fp64; phase partials in a fixed order
    __shared__ double pc[256][4];
    const int cpr = fd / 4, phases = 256 / cpr;
    const int ch = tid % cpr, ph = tid / cpr;
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    if (ph < phases) {
      for (int r = lo + ph; r < hi; r += phases) {
        const float4 v = *reinterpret_cast<const float4*>(feat + ((long long)h * n_q + pr[r]) * fd +
                                                          4 * ch);
        *reinterpret_cast<float4*>(feat_g + ((long long)h * n_q + r) * fd + 4 * ch) = v;
        acc[0] += double(v.x);
        acc[1] += double(v.y);
        acc[2] += double(v.z);
        acc[3] += double(v.w);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pc[tid][e] = acc[e];
    }
    __syncthreads();
    for (int j = tid; j < fd; j += 256) {
      double t = 0.0;
      for (int p2 = 0; p2 < phases; ++p2) t += pc[p2 * cpr + j / 4][j % 4];
      feat_cen[((long long)h * c_q + a) * fd + j] = hi > lo ? t / double(hi - lo) : 0.0;
    }
    return;
  }
  const int rl = tid >> 6, j = tid & 63;
  __shared__ double part[4][64];
  double s = 0.0;
  if (j < fd) {
#pragma unroll 4
    for (int r = lo + rl; r < hi; r += 4) {
      const float v = feat[((long long)h * n_q + pr[r]) * fd + j];
      feat_g[((long long)h * n_q + r) * fd + j] = v;
      s += double(v);
    }
  }
  part[rl][j] = s;
  __syncthreads();
  if (rl == 0 && j < fd)
    feat_cen[((long long)h * c_q + a) * fd + j] =
        hi > lo ? (((part[0][j] + part[1][j]) + part[2][j]) + part[3][j]) / double(hi - lo) : 0.0;
}

struct ProbeWs {
  int32_t *m_a, *rank, *s_tab, *group;
  double* dist;
  float *part_s, *part_n;
  double *xp, *rp, *xw, *rw, *z, *a, *psi;
};

ProbeWs carve_probe(void* base, const sparsepr_dims* d, int m) {
  Carver cv(base);
  const size_t H = d->heads;
  ProbeWs w;
  w.m_a = cv.take<int32_t>(H * d->c_q);
  w.rank = cv.take<int32_t>(H * d->c_q);
  w.s_tab = cv.take<int32_t>(H * (kMaxM + 2));
  w.group = cv.take<int32_t>(H * m);
  w.dist = cv.take<double>(H * d->n_q);
  w.part_s = cv.take<float>(H * kChunks * m * 4);
  w.part_n = cv.take<float>(H * kChunks * m * 2 * d->head_dim);
  w.xp = cv.take<double>(H * m * d->head_dim);
  w.rp = cv.take<double>(H * m * d->head_dim);
  w.xw = cv.take<double>(H * m * d->head_dim);
  w.rw = cv.take<double>(H * m * d->head_dim);
  w.z = cv.take<double>(H * kMaxM * kMaxM);
  w.a = cv.take<double>(H * d->head_dim * kMaxM);
  w.psi = cv.take<double>(H * d->head_dim * kMaxM);
  // record the size in the last pointer slot via a dummy take
  return w;
}

}  // namespace

size_t probe_ws_bytes(const sparsepr_dims* d, int32_t m, int32_t rank) {
  (void)rank;
  Carver cv(nullptr);
  const size_t H = d->heads;
  cv.take<int32_t>(H * d->c_q);
  cv.take<int32_t>(H * d->c_q);
  cv.take<int32_t>(H * (kMaxM + 2));
  cv.take<int32_t>(H * m);
  cv.take<double>(H * d->n_q);
  cv.take<float>(H * kChunks * m * 4);
  cv.take<float>(H * kChunks * m * 2 * d->head_dim);
  cv.take<double>(H * m * d->head_dim);
  cv.take<double>(H * m * d->head_dim);
  cv.take<double>(H * m * d->head_dim);
  cv.take<double>(H * m * d->head_dim);
  cv.take<double>(H * kMaxM * kMaxM);
  cv.take<double>(H * d->head_dim * kMaxM);
  cv.take<double>(H * d->head_dim * kMaxM);
  return cv.used;
}

// probe_ws_bytes plus group-major feature rows and fp64 feature centroids
// (feature dimension up to SPARSEPR_MAX_RANK)
size_t probe_feat_ws_bytes(const sparsepr_dims* d, int32_t m, int32_t rank) {
  Carver cv(nullptr);
  const size_t H = d->heads;
  cv.take<float>(H * d->n_q * SPARSEPR_MAX_RANK);
  cv.take<double>(H * d->c_q * SPARSEPR_MAX_RANK);
  return probe_ws_bytes(d, m, rank) + cv.used;
}

}  // namespace spr

using namespace spr;

namespace {
// S6: the probe plan and the probe rows of every group (Algorithm A.1); the
// per-group probe counts and each probe's group stay in the workspace for
// the fit stage.
int32_t select_stage(const sparsepr_dims* dims, int32_t m, const int32_t* offsets_q,
                     const int32_t* perm_q, const double* centroid_q, const float* feat,
                     int32_t fd, const void* q_g, int32_t* probe_rows, int32_t* probe_tokens,
                     const ProbeWs& w, void* ws, hipStream_t stream) {
  const int H = dims->heads, d = dims->head_dim;
  plan_kernel<<<H, 1024, 0, stream>>>(offsets_q, dims->c_q, dims->n_q, m, w.m_a, w.rank, w.s_tab,
                                      probe_rows, probe_tokens, w.group);
  SPR_LAUNCH_CHECK();
  if (feat) {
    // feature rows and centroids after the standard workspace
    Carver cv(static_cast<char*>(ws) + probe_ws_bytes(dims, m, 0));
    float* feat_g = cv.take<float>(size_t(H) * dims->n_q * fd);
    double* feat_cen = cv.take<double>(size_t(H) * dims->c_q * fd);
    // 16-byte chunks when rows are whole chunks and both arrays start on 16 bytes
    const int chunked = fd % 4 == 0 && (reinterpret_cast<uintptr_t>(feat) & 15) == 0 &&
                        (reinterpret_cast<uintptr_t>(feat_g) & 15) == 0;
    feat_group_kernel<<<dim3(dims->c_q, H), 256, 0, stream>>>(feat, perm_q, offsets_q, dims->n_q,
                                                              dims->c_q, fd, chunked, feat_g,
                                                              feat_cen);
    SPR_LAUNCH_CHECK();
    select_kernel<float><<<dim3(dims->c_q, H), 256, 0, stream>>>(
        feat_g, feat_cen, offsets_q, perm_q, w.m_a, w.rank, w.s_tab, dims->n_q, dims->c_q, fd, m,
        w.dist, probe_rows, probe_tokens, w.group);
  } else if (dims->dtype == SPARSEPR_BF16) {
    select_kernel<uint16_t><<<dim3(dims->c_q, H), 256, 0, stream>>>(
        static_cast<const uint16_t*>(q_g), centroid_q, offsets_q, perm_q, w.m_a, w.rank,
        w.s_tab, dims->n_q, dims->c_q, d, m, w.dist, probe_rows, probe_tokens, w.group);
  } else {
    select_kernel<float><<<dim3(dims->c_q, H), 256, 0, stream>>>(
        static_cast<const float*>(q_g), centroid_q, offsets_q, perm_q, w.m_a, w.rank, w.s_tab,
        dims->n_q, dims->c_q, d, m, w.dist, probe_rows, probe_tokens, w.group);
  }
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}

// S7-S8: exact probe rows (retained / omitted sums over the routed cells),
// their merge, and the fit, for the probes the select stage left in the
// workspace.
int32_t fit_stage(const sparsepr_dims* dims, int32_t m, int32_t rank, double lambda,
                  int32_t estimator, float* corr_g, const int32_t* offsets_q,
                  const int32_t* offsets_kv, const int32_t* cell_rowptr, const int32_t* cell_col,
                  const void* q_g, const void* k_g, const void* v_g, const int32_t* v_shift,
                  float softmax_scale, const int32_t* probe_rows, float* o_probe_dense,
                  float* o_probe_sparse, float* corr_a, float* corr_psi_t, float* corr_c,
                  const ProbeWs& w, hipStream_t stream) {
  const int H = dims->heads, d = dims->head_dim;
  const int me = m < dims->n_q ? m : dims->n_q;
  const float sl2 = softmax_scale * kLog2e;
  if (dims->dtype == SPARSEPR_BF16) {
    auto* qq = static_cast<const uint16_t*>(q_g);
    auto* kk = static_cast<const uint16_t*>(k_g);
    auto* vv = static_cast<const uint16_t*>(v_g);
    if (d == 128)
      probe_rows_mfma_kernel<128><<<dim3(kChunks, H), 256, 0, stream>>>(
          qq, kk, vv, v_shift, offsets_kv, cell_rowptr, cell_col, probe_rows, w.group, dims->n_q,
          dims->n_k, dims->c_q, dims->c_k, m, sl2, w.part_s, w.part_n);
    else
      probe_rows_mfma_kernel<64><<<dim3(kChunks, H), 256, 0, stream>>>(
          qq, kk, vv, v_shift, offsets_kv, cell_rowptr, cell_col, probe_rows, w.group, dims->n_q,
          dims->n_k, dims->c_q, dims->c_k, m, sl2, w.part_s, w.part_n);
  } else {
    auto* qq = static_cast<const float*>(q_g);
    auto* kk = static_cast<const float*>(k_g);
    auto* vv = static_cast<const float*>(v_g);
    if (d == 128)
      probe_rows_kernel<float, 128><<<dim3(kChunks, H), 256, 0, stream>>>(
          qq, kk, vv, v_shift, offsets_kv, cell_rowptr, cell_col, probe_rows, w.group, dims->n_q,
          dims->n_k, dims->c_q, dims->c_k, m, sl2, w.part_s, w.part_n);
    else
      probe_rows_kernel<float, 64><<<dim3(kChunks, H), 256, 0, stream>>>(
          qq, kk, vv, v_shift, offsets_kv, cell_rowptr, cell_col, probe_rows, w.group, dims->n_q,
          dims->n_k, dims->c_q, dims->c_k, m, sl2, w.part_s, w.part_n);
  }
  SPR_LAUNCH_CHECK();
  merge_kernel<<<dim3(me, H), 128, 0, stream>>>(w.part_s, w.part_n, m, me, d, o_probe_dense,
                                                o_probe_sparse, w.xp, w.rp);
  SPR_LAUNCH_CHECK();
  FitArgs fa;
  fa.off_q = offsets_q;
  fa.m_a = w.m_a;
  fa.probe_group = w.group;
  fa.xp = w.xp;
  fa.rp = w.rp;
  fa.xw = w.xw;
  fa.rw = w.rw;
  fa.zbuf = w.z;
  fa.abuf = w.a;
  fa.pbuf = w.psi;
  fa.corr_a = corr_a;
  fa.corr_psi_t = corr_psi_t;
  fa.corr_c = corr_c;
  fa.corr_g = corr_g;
  fa.estimator = estimator;
  fa.c_q = dims->c_q;
  fa.m = m;
  fa.me = me;
  fa.d = d;
  fa.rank = rank;
  fa.lambda = lambda;
  fit_kernel<<<H, kFitThreads, 0, stream>>>(fa);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}

// argument checks of the select stage (dims already checked)
int32_t check_select(int32_t m, const int32_t* offsets_q, const int32_t* perm_q,
                     const double* centroid_q, const float* feat, int32_t fd, const void* q_g,
                     const int32_t* probe_rows, const int32_t* probe_tokens) {
  if (m < 1 || m > SPARSEPR_MAX_PROBES) return SPARSEPR_ERR_INVALID;
  if (feat ? (fd < 1 || fd > SPARSEPR_MAX_RANK) : (!centroid_q || !q_g)) return SPARSEPR_ERR_INVALID;
  if (!offsets_q || !perm_q || !probe_rows || !probe_tokens) return SPARSEPR_ERR_INVALID;
  return SPARSEPR_OK;
}

// argument checks of the fit stage (dims already checked)
int32_t check_fit(int32_t m, int32_t rank, double lambda, int32_t estimator, const float* corr_g,
                  const int32_t* offsets_q, const int32_t* offsets_kv, const int32_t* cell_rowptr,
                  const int32_t* cell_col, const void* q_g, const void* k_g, const void* v_g,
                  const int32_t* v_shift, const int32_t* probe_rows, const float* o_probe_dense,
                  const float* corr_a, const float* corr_psi_t, const float* corr_c) {
  if (m < 1 || m > SPARSEPR_MAX_PROBES || rank < 0 || rank > SPARSEPR_MAX_RANK || !(lambda >= 0.0))
    return SPARSEPR_ERR_INVALID;
  if (estimator < SPARSEPR_EST_FULL || estimator > SPARSEPR_EST_DIAGONAL) return SPARSEPR_ERR_INVALID;
  if (estimator != SPARSEPR_EST_FULL && !corr_g) return SPARSEPR_ERR_INVALID;
  if (!offsets_q || !offsets_kv || !cell_rowptr || !cell_col || !q_g || !k_g || !v_g ||
      !v_shift || !probe_rows || !o_probe_dense || !corr_a || !corr_psi_t || !corr_c)
    return SPARSEPR_ERR_INVALID;
  if (estimator == SPARSEPR_EST_FULL && rank > 0 && lambda == 0.0)
    return SPARSEPR_ERR_INVALID;  // dual solve needs lam > 0
  return SPARSEPR_OK;
}

int32_t probe_fit_impl(const sparsepr_dims* dims, int32_t m, int32_t rank, double lambda,
                       int32_t estimator, float* corr_g,
                       const int32_t* offsets_q, const int32_t* offsets_kv, const int32_t* perm_q,
                       const int32_t* cell_rowptr, const int32_t* cell_col,
                       const double* centroid_q, const float* feat, int32_t fd, const void* q_g,
                       const void* k_g, const void* v_g, const int32_t* v_shift,
                       float softmax_scale, int32_t* probe_rows, int32_t* probe_tokens,
                       float* o_probe_dense, float* o_probe_sparse, float* corr_a,
                       float* corr_psi_t, float* corr_c, void* ws, size_t ws_bytes,
                       hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  st = check_select(m, offsets_q, perm_q, centroid_q, feat, fd, q_g, probe_rows, probe_tokens);
  if (st != SPARSEPR_OK) return st;
  st = check_fit(m, rank, lambda, estimator, corr_g, offsets_q, offsets_kv, cell_rowptr,
                 cell_col, q_g, k_g, v_g, v_shift, probe_rows, o_probe_dense, corr_a, corr_psi_t,
                 corr_c);
  if (st != SPARSEPR_OK) return st;
  const size_t need = feat ? probe_feat_ws_bytes(dims, m, rank) : probe_ws_bytes(dims, m, rank);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  ProbeWs w = carve_probe(ws, dims, m);
  st = select_stage(dims, m, offsets_q, perm_q, centroid_q, feat, fd, q_g, probe_rows,
                    probe_tokens, w, ws, stream);
  if (st != SPARSEPR_OK) return st;
  return fit_stage(dims, m, rank, lambda, estimator, corr_g, offsets_q, offsets_kv, cell_rowptr,
                   cell_col, q_g, k_g, v_g, v_shift, softmax_scale, probe_rows, o_probe_dense,
                   o_probe_sparse, corr_a, corr_psi_t, corr_c, w, stream);
}
}  // namespace

extern "C" int32_t sparsepr_probe_fit(const sparsepr_dims* dims, int32_t m, int32_t rank,
                                      double lambda, const int32_t* offsets_q,
                                      const int32_t* offsets_kv, const int32_t* perm_q,
                                      const int32_t* cell_rowptr, const int32_t* cell_col,
                                      const double* centroid_q, const void* q_g, const void* k_g,
                                      const void* v_g, const int32_t* v_shift,
                                      float softmax_scale, int32_t* probe_rows,
                                      int32_t* probe_tokens, float* o_probe_dense,
                                      float* o_probe_sparse, float* corr_a, float* corr_psi_t,
                                      float* corr_c, void* ws, size_t ws_bytes,
                                      hipStream_t stream) {
  return probe_fit_impl(dims, m, rank, lambda, SPARSEPR_EST_FULL, nullptr, offsets_q, offsets_kv,
                        perm_q, cell_rowptr, cell_col, centroid_q, nullptr, 0, q_g, k_g, v_g,
                        v_shift, softmax_scale,
                        probe_rows, probe_tokens, o_probe_dense, o_probe_sparse, corr_a,
                        corr_psi_t, corr_c, ws, ws_bytes, stream);
}

extern "C" int32_t sparsepr_probe_fit_ex(
    const sparsepr_dims* dims, int32_t m, int32_t rank, double lambda, int32_t estimator,
    const int32_t* offsets_q, const int32_t* offsets_kv, const int32_t* perm_q,
    const int32_t* cell_rowptr, const int32_t* cell_col, const double* centroid_q,
    const float* probe_feat, int32_t feat_dim, const void* q_g, const void* k_g, const void* v_g,
    const int32_t* v_shift, float softmax_scale, int32_t* probe_rows, int32_t* probe_tokens,
    float* o_probe_dense, float* o_probe_sparse, float* corr_a, float* corr_psi_t, float* corr_c,
    float* corr_g, void* ws, size_t ws_bytes, hipStream_t stream) {
  return probe_fit_impl(dims, m, rank, lambda, estimator, corr_g, offsets_q, offsets_kv, perm_q,
                        cell_rowptr, cell_col, probe_feat ? nullptr : centroid_q, probe_feat,
                        feat_dim, q_g, k_g, v_g, v_shift, softmax_scale, probe_rows, probe_tokens,
                        o_probe_dense, o_probe_sparse, corr_a, corr_psi_t, corr_c, ws, ws_bytes,
                        stream);
}

extern "C" int32_t sparsepr_probe_select(const sparsepr_dims* dims, int32_t m,
                                         const int32_t* offsets_q, const int32_t* perm_q,
                                         const double* centroid_q, const float* probe_feat,
                                         int32_t feat_dim, const void* q_g, int32_t* probe_rows,
                                         int32_t* probe_tokens, void* ws, size_t ws_bytes,
                                         hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  st = check_select(m, offsets_q, perm_q, probe_feat ? nullptr : centroid_q, probe_feat,
                    feat_dim, q_g, probe_rows, probe_tokens);
  if (st != SPARSEPR_OK) return st;
  const size_t need = probe_feat ? probe_feat_ws_bytes(dims, m, 0) : probe_ws_bytes(dims, m, 0);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  const ProbeWs w = carve_probe(ws, dims, m);
  return select_stage(dims, m, offsets_q, perm_q, probe_feat ? nullptr : centroid_q, probe_feat,
                      feat_dim, q_g, probe_rows, probe_tokens, w, ws, stream);
}

extern "C" int32_t sparsepr_probe_fit_selected(
    const sparsepr_dims* dims, int32_t m, int32_t rank, double lambda, int32_t estimator,
    const int32_t* offsets_q, const int32_t* offsets_kv, const int32_t* cell_rowptr,
    const int32_t* cell_col, const void* q_g, const void* k_g, const void* v_g,
    const int32_t* v_shift, float softmax_scale, const int32_t* probe_rows, float* o_probe_dense,
    float* o_probe_sparse, float* corr_a, float* corr_psi_t, float* corr_c, float* corr_g,
    void* ws, size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  st = check_fit(m, rank, lambda, estimator, corr_g, offsets_q, offsets_kv, cell_rowptr, cell_col,
                 q_g, k_g, v_g, v_shift, probe_rows, o_probe_dense, corr_a, corr_psi_t, corr_c);
  if (st != SPARSEPR_OK) return st;
  if (!ws || ws_bytes < probe_ws_bytes(dims, m, rank)) return SPARSEPR_ERR_WORKSPACE;
  const ProbeWs w = carve_probe(ws, dims, m);
  return fit_stage(dims, m, rank, lambda, estimator, corr_g, offsets_q, offsets_kv, cell_rowptr,
                   cell_col, q_g, k_g, v_g, v_shift, softmax_scale, probe_rows, o_probe_dense,
                   o_probe_sparse, corr_a, corr_psi_t, corr_c, w, stream);
}
