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
// Xbar, Rw = W~^1/2 Rbar; the right singular vectors of Rw come from a
// cyclic Jacobi eigensolve of Rw Rw^T; finally B is folded with the
// projection into A = diag(1/s) B Psi and c = mu_R - (mu_x A) Psi^T.

#include <type_traits>

#include "common.h"
#include "mfma_tiles.h"
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
    f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
    for (int s2 = 0; s2 < NS; ++s2) {
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag<D>(kt, n, s2, g), qf[s2], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_frag<D>(kt, 32 + n, s2, g), qf[s2], s1, 0, 0,
                                                   0);
    }
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
    const int tail = k1 - t0;
    // keys at or past the chunk end take no part: clear them from both classes
    uint32_t va = 0xffffu, vb_ = 0xffffu;
    if (tail < 64) {
      va = 0;
      vb_ = 0;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        va |= uint32_t(c_key(0, r, g) < tail) << r;
        vb_ |= uint32_t(c_key(1, r, g) < tail) << r;
      }
    }
    float tS = NEG, tU = NEG;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float xa = s0[r], xb = s1[r];
      if ((va >> r) & 1u) {
        if ((mb0 >> r) & 1u) tS = fmaxf(tS, xa);
        else tU = fmaxf(tU, xa);
      }
      if ((vb_ >> r) & 1u) {
        if ((mb1 >> r) & 1u) tS = fmaxf(tS, xb);
        else tU = fmaxf(tU, xb);
      }
    }
    tS = fmaxf(tS, __shfl_xor(tS, 32));
    tU = fmaxf(tU, __shfl_xor(tU, 32));
    if (__ballot(tS > mS + slack)) {
      const float nm = fmaxf(mS, tS);
      const float al = nm == NEG ? 1.f : __builtin_amdgcn_exp2f((mS - nm) * c2);
      mS = nm;
      zS *= al;
#pragma unroll
      for (int db = 0; db < NDH; ++db) oS[db] *= al;
    }
    if (__ballot(tU > mU + slack)) {
      const float nm = fmaxf(mU, tU);
      const float al = nm == NEG ? 1.f : __builtin_amdgcn_exp2f((mU - nm) * c2);
      mU = nm;
      zU *= al;
#pragma unroll
      for (int db = 0; db < NDH; ++db) oU[db] *= al;
    }
    const float mcS = mS * c2, mcU = mU * c2;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const bool ia = (mb0 >> r) & 1u, ib = (mb1 >> r) & 1u;
      const float ea = ((va >> r) & 1u)
                           ? __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], c2, ia ? -mcS : -mcU))
                           : 0.f;
      const float eb = ((vb_ >> r) & 1u)
                           ? __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], c2, ib ? -mcS : -mcU))
                           : 0.f;
      s0[r] = ea;
      s1[r] = eb;
      zS += ia ? ea : 0.f;
      zU += ia ? 0.f : ea;
      zS += ib ? eb : 0.f;
      zU += ib ? 0.f : eb;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f16x8_t sh, sl, uh, ul;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 8 * (u & 1) + j;
        const float e = (u >> 1) ? s1[r] : s0[r];
        const _Float16 eh = static_cast<_Float16>(e);
        const _Float16 el = static_cast<_Float16>(e - float(eh));
        const bool in = ((u >> 1) ? (mb1 >> r) : (mb0 >> r)) & 1u;
        const _Float16 z16 = static_cast<_Float16>(0.f);
        sh[j] = in ? eh : z16;
        sl[j] = in ? el : z16;
        uh[j] = in ? z16 : eh;
        ul[j] = in ? z16 : el;
      }
#pragma unroll
      for (int db = 0; db < NDH; ++db) {
        const f16x8_t vf = v_frag<D>(vt, lane, u, dh * NDH + db);
        oS[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, sh, oS[db], 0, 0, 0);
        oS[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, sl, oS[db], 0, 0, 0);
        oU[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, uh, oU[db], 0, 0, 0);
        oU[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, ul, oU[db], 0, 0, 0);
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

__global__ __launch_bounds__(256) void fit_kernel(FitArgs f) {
  const int h = blockIdx.x, tid = threadIdx.x;
  const int me = f.me, d = f.d;
  __shared__ double w[kMaxM], wt[kMaxM];
  __shared__ double mux[128], mur[128], sc[128];
  __shared__ double G[kMaxM * kLd];   // Cholesky factor (lower)
  __shared__ double E[kMaxM * kLd];   // Rw Rw^T, diagonalised in place
  __shared__ double U[kMaxM * kLd];   // eigenvectors (columns)
  __shared__ double xs[kMaxM][33], rs2[kMaxM][33];   // column chunk staging
  __shared__ int32_t order[kMaxM];
  __shared__ double red[4];
  __shared__ double tcol[kMaxM];
  __shared__ int32_t sh_k;
  __shared__ int32_t sh_rot[2], sh_big[2];   // per sweep parity

  const double* X = f.xp + (long long)h * f.m * d;
  const double* R = f.rp + (long long)h * f.m * d;
  double* Xw = f.xw + (long long)h * f.m * d;
  double* Rw = f.rw + (long long)h * f.m * d;

  // 1. coverage weights |G_a| / m_a
  const int32_t* oq = f.off_q + (long long)h * (f.c_q + 1);
  if (tid < me) {
    const int a = f.probe_group[(long long)h * f.m + tid];
    w[tid] = double(oq[a + 1] - oq[a]) / double(f.m_a[(long long)h * f.c_q + a]);
  }
  __syncthreads();
  double sw = 0.0;
  for (int p = 0; p < me; ++p) sw += w[p];
  if (tid < me) wt[tid] = double(me) * w[tid] / sw;
  // 2. weighted means and feature scale (unit-sum weights)
  if (tid < d) {
    double mx = 0, mr = 0;
    for (int p = 0; p < me; ++p) {
      const double wh = w[p] / sw;
      mx += wh * X[p * d + tid];
      mr += wh * R[p * d + tid];
    }
    double var = 0;
    for (int p = 0; p < me; ++p) {
      const double t = X[p * d + tid] - mx;
      var += (w[p] / sw) * t * t;
    }
    mux[tid] = mx;
    mur[tid] = mr;
    sc[tid] = sqrt(var + 1e-6);
  }
  __syncthreads();
  // 3. weighted, standardised features and centred residuals
  for (int e = tid; e < me * d; e += 256) {
    const int p = e / d, j = e % d;
    const double sq = sqrt(wt[p]);
    Xw[e] = sq * (X[e] - mux[j]) / sc[j];
    Rw[e] = sq * (R[e] - mur[j]);
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
        const double xv = Xw[p * d + tid], rv = Rw[p * d + tid];
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
    for (int e = tid; e < d * f.rank; e += 256) {
      f.corr_a[(long long)h * d * f.rank + e] = 0.f;
      f.corr_psi_t[(long long)h * f.rank * d + e] = 0.f;
    }
    return;
  }
  if (ocg)
    for (int j = tid; j < d; j += 256) ocg[j] = 0.f;
  // 4. Gram matrices G = Xw Xw^T + lam I and E = Rw Rw^T, 32 columns of the
  // weighted features / residuals staged in LDS at a time
  for (int e = tid; e < me * me; e += 256) {
    const int pp = e / me, qq = e - (e / me) * me;
    G[pp * kLd + qq] = pp == qq ? f.lambda : 0.0;
    E[pp * kLd + qq] = 0.0;
    U[pp * kLd + qq] = pp == qq ? 1.0 : 0.0;
  }
  for (int d0 = 0; d0 < d; d0 += 32) {
    __syncthreads();
    for (int e = tid; e < me * 32; e += 256) {
      const int pp = e >> 5, jj = e & 31;
      xs[pp][jj] = Xw[pp * d + d0 + jj];
      rs2[pp][jj] = Rw[pp * d + d0 + jj];
    }
    __syncthreads();
    for (int e = tid; e < me * me; e += 256) {
      const int pp = e / me, qq = e - (e / me) * me;
      double gx = 0.0, gr = 0.0;
#pragma unroll 8
      for (int jj = 0; jj < 32; ++jj) {
        gx = fma(xs[pp][jj], xs[qq][jj], gx);
        gr = fma(rs2[pp][jj], rs2[qq][jj], gr);
      }
      G[pp * kLd + qq] += gx;
      E[pp * kLd + qq] += gr;
    }
  }
  __syncthreads();
  // 5. Cholesky G = L L^T (right-looking, lower triangle); thread t updates
  // rows i = k+1+t/4 (+64) and columns j = k+1+t%4 (+4)
  for (int k = 0; k < me; ++k) {
    const double piv = sqrt(G[k * kLd + k]);
    __syncthreads();
    for (int i = k + 1 + tid; i < me; i += 256) G[i * kLd + k] /= piv;
    if (tid == 0) G[k * kLd + k] = piv;
    __syncthreads();
    for (int i = k + 1 + (tid >> 2); i < me; i += 64) {
      const double lik = G[i * kLd + k];
      for (int j = k + 1 + (tid & 3); j <= i; j += 4) G[i * kLd + j] -= lik * G[j * kLd + k];
    }
  }
  __syncthreads();
  // 6. cyclic Jacobi on E with round-robin disjoint pairs (thread t works on
  // pair t/8, columns t%8 + 8l; the eight threads of a pair, one wave's
  // lanes, each compute the pair's rotation from E, so no broadcast and no
  // barrier separate it from the row pass: a wave's LDS accesses run in
  // order, and other pairs touch other rows).  A rotation
  // is skipped when |a_pq| is negligible next to the diagonal and next to the
  // trace (the Gram route resolves eigenvalues to ~1e-16 of the trace).  The
  // iteration stops after a sweep without rotations, or after a sweep in
  // which every rotation had |a_pq| below 1e-8 sqrt(a_pp a_qq) or below
  // 1e-10 of the trace: convergence is quadratic, so what the next sweep
  // would rotate is at the rounding level of the trace.  Rotation parameters use the hardware reciprocal / reciprocal
  // square root refined by two Newton steps (about an ulp; c^2 + s^2 = 1 to
  // rounding).
  {
    auto rcp64 = [](double y) {
      double r = __builtin_amdgcn_rcp(y);
      r = r * fma(-y, r, 2.0);
      r = r * fma(-y, r, 2.0);
      return r;
    };
    auto rsq64 = [](double y) {
      double r = __builtin_amdgcn_rsq(y);
      r = r * fma(-0.5 * y * r, r, 1.5);
      r = r * fma(-0.5 * y * r, r, 1.5);
      return r;
    };
    double trp = 0.0;
    for (int i = tid; i < me; i += 256) trp += fabs(E[i * kLd + i]);
    const double tr = block_sum(trp, red);
    const double abs_floor = 1e-300 + 1e-14 * tr;
    const int mp = (me + 1) & ~1;   // even player count; player me is a dummy if me is odd
    const int npair = mp / 2;
    const int pi = tid >> 3, cj = tid & 7;
    if (tid == 0) {
      sh_rot[0] = 0;
      sh_big[0] = 0;
    }
    __syncthreads();
    for (int sweep = 0; sweep < 20; ++sweep) {
      // flags of sweep s live in slot s & 1.  Slot par ^ 1 (read by every
      // thread at the end of the previous sweep) is cleared for the next
      // sweep only after this sweep's first barrier, which every thread
      // reaches after that read
      const int par = sweep & 1;
      for (int rnd = 0; rnd < mp - 1; ++rnd) {
        int p2 = 0, q2 = 0;
        double ci = 1.0, si = 0.0;
        if (pi < npair) {
          int pp, qq;
          if (pi == 0) { pp = mp - 1; qq = rnd; }
          else {
            pp = rnd + pi; pp -= pp >= mp - 1 ? mp - 1 : 0;
            qq = rnd - pi; qq += qq < 0 ? mp - 1 : 0;
          }
          if (pp < me && qq < me) {
            const double apq = E[pp * kLd + qq];
            const double app = E[pp * kLd + pp], aqq = E[qq * kLd + qq];
            const double apq2 = apq * apq, dd = fabs(app * aqq);
            if (apq2 > 1e-30 * dd && fabs(apq) > abs_floor) {
              const double tau = (aqq - app) * rcp64(2.0 * apq);
              const double u = fma(tau, tau, 1.0);
              const double t = (tau >= 0 ? 1.0 : -1.0) * rcp64(fabs(tau) + u * rsq64(u));
              ci = rsq64(fma(t, t, 1.0));
              si = t * ci;
              p2 = pp;
              q2 = qq;
              if (cj == 0) {
                sh_rot[par] = 1;
                if (apq2 > 1e-16 * dd && fabs(apq) > 1e-10 * tr) sh_big[par] = 1;
              }
            }
          }
        }
        const bool act = si != 0.0;
        if (act)   // rows: E <- J^T E
          for (int j = cj; j < me; j += 8) {
            const double x1 = E[p2 * kLd + j], x2 = E[q2 * kLd + j];
            E[p2 * kLd + j] = ci * x1 - si * x2;
            E[q2 * kLd + j] = si * x1 + ci * x2;
          }
        __syncthreads();
        if (rnd == 0 && tid == 0) {
          sh_rot[par ^ 1] = 0;
          sh_big[par ^ 1] = 0;
        }
        if (act)   // columns: E <- E J, U <- U J
          for (int j = cj; j < me; j += 8) {
            const double x1 = E[j * kLd + p2], x2 = E[j * kLd + q2];
            E[j * kLd + p2] = ci * x1 - si * x2;
            E[j * kLd + q2] = si * x1 + ci * x2;
            const double u1 = U[j * kLd + p2], u2 = U[j * kLd + q2];
            U[j * kLd + p2] = ci * u1 - si * u2;
            U[j * kLd + q2] = si * u1 + ci * u2;
          }
        __syncthreads();
      }
      if (!sh_rot[par] || !sh_big[par]) break;
    }
  }
  __syncthreads();
  // 7. order eigenvalues (descending, ties by index), decide kept directions
  if (tid < me) {
    const double li = E[tid * kLd + tid];
    int r = 0;
    for (int j = 0; j < me; ++j) {
      const double lj = E[j * kLd + j];
      if (lj > li || (lj == li && j < tid)) ++r;
    }
    order[r] = tid;
  }
  __syncthreads();
  if (tid == 0) {
    const double l1 = E[order[0] * kLd + order[0]];
    const double s1 = l1 > 0 ? sqrt(l1) : 0.0;
    int k = 0;
    if (s1 > 0) {
      const double floor_l = 64.0 * 2.220446049250313e-16 * l1;  // resolution of the Gram route
      for (int i = 0; i < me; ++i) {
        const double li = E[order[i] * kLd + order[i]];
        if (li > floor_l && sqrt(li) > 1e-10 * s1) ++k;
        else break;
      }
    }
    int cap = f.rank < me ? f.rank : me;
    cap = cap < d ? cap : d;
    sh_k = k < cap ? k : cap;
  }
  __syncthreads();
  const int k = sh_k;
  double* Z = f.zbuf + (long long)h * kMaxM * kMaxM;
  // 8. z_c = G^-1 (u_c sigma_c): forward then backward substitution, one thread per c
  if (tid < k) {
    const int ii = order[tid];
    const double sig = sqrt(E[ii * kLd + ii]);
    double* z = Z + tid * kMaxM;
    for (int i = 0; i < me; ++i) {
      double s = U[i * kLd + ii] * sig;
      for (int j = 0; j < i; ++j) s -= G[i * kLd + j] * z[j];
      z[i] = s / G[i * kLd + i];
    }
    for (int i = me - 1; i >= 0; --i) {
      double s = z[i];
      for (int j = i + 1; j < me; ++j) s -= G[j * kLd + i] * z[j];
      z[i] = s / G[i * kLd + i];
    }
  }
  __syncthreads();
  double* Ab = f.abuf + (long long)h * d * kMaxM;
  double* Pb = f.pbuf + (long long)h * d * kMaxM;
  for (int e = tid; e < d * k; e += 256) {
    const int j = e / k, c = e % k;
    const int ii = order[c];
    const double sig = sqrt(E[ii * kLd + ii]);
    const double* z = Z + c * kMaxM;
    double bpsi = 0.0, psi = 0.0;
    for (int p = 0; p < me; ++p) {
      bpsi = fma(Xw[p * d + j], z[p], bpsi);
      psi = fma(Rw[p * d + j], U[p * kLd + ii], psi);
    }
    Ab[j * kMaxM + c] = bpsi / sc[j];
    Pb[j * kMaxM + c] = psi / sig;
  }
  __syncthreads();
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
  for (int e = tid; e < d * f.rank; e += 256) {
    const int j = e / f.rank, c = e % f.rank;
    oa[e] = c < k ? float(Ab[j * kMaxM + c]) : 0.f;
  }
  for (int e = tid; e < f.rank * d; e += 256) {
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
  if (m < 1 || m > SPARSEPR_MAX_PROBES || rank < 0 || rank > SPARSEPR_MAX_RANK || !(lambda >= 0.0))
    return SPARSEPR_ERR_INVALID;
  if (feat ? (fd < 1 || fd > SPARSEPR_MAX_RANK) : !centroid_q) return SPARSEPR_ERR_INVALID;
  if (estimator < SPARSEPR_EST_FULL || estimator > SPARSEPR_EST_DIAGONAL) return SPARSEPR_ERR_INVALID;
  if (estimator != SPARSEPR_EST_FULL && !corr_g) return SPARSEPR_ERR_INVALID;
  if (!offsets_q || !offsets_kv || !perm_q || !cell_rowptr || !cell_col || !q_g ||
      !k_g || !v_g || !v_shift || !probe_rows || !probe_tokens || !o_probe_dense || !corr_a || !corr_psi_t ||
      !corr_c)
    return SPARSEPR_ERR_INVALID;
  if (estimator == SPARSEPR_EST_FULL && rank > 0 && lambda == 0.0)
    return SPARSEPR_ERR_INVALID;  // dual solve needs lam > 0
  const size_t need = feat ? probe_feat_ws_bytes(dims, m, rank) : probe_ws_bytes(dims, m, rank);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  ProbeWs w = carve_probe(ws, dims, m);
  const int H = dims->heads, d = dims->head_dim;
  const int me = m < dims->n_q ? m : dims->n_q;
  plan_kernel<<<H, 1024, 0, stream>>>(offsets_q, dims->c_q, dims->n_q, m, w.m_a, w.rank, w.s_tab,
                                      probe_rows, probe_tokens, w.group);
  SPR_LAUNCH_CHECK();
  const float sl2 = softmax_scale * kLog2e;
  if (feat) {
    // feature rows and centroids after the standard workspace
    Carver cv(static_cast<char*>(ws) + probe_ws_bytes(dims, m, rank));
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
    SPR_LAUNCH_CHECK();
  }
  if (dims->dtype == SPARSEPR_BF16) {
    if (!feat) {
      select_kernel<uint16_t><<<dim3(dims->c_q, H), 256, 0, stream>>>(
          static_cast<const uint16_t*>(q_g), centroid_q, offsets_q, perm_q, w.m_a, w.rank,
          w.s_tab, dims->n_q, dims->c_q, d, m, w.dist, probe_rows, probe_tokens, w.group);
      SPR_LAUNCH_CHECK();
    }
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
    if (!feat) {
      select_kernel<float><<<dim3(dims->c_q, H), 256, 0, stream>>>(
          static_cast<const float*>(q_g), centroid_q, offsets_q, perm_q, w.m_a, w.rank, w.s_tab,
          dims->n_q, dims->c_q, d, m, w.dist, probe_rows, probe_tokens, w.group);
      SPR_LAUNCH_CHECK();
    }
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
  fit_kernel<<<H, 256, 0, stream>>>(fa);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
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
