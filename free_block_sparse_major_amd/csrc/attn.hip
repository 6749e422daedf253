// S5: renormalised hard-drop attention over routed cells.
//
// SparsePR paper §3: a query of group a attends only to the keys (and their
// values) of the K/V groups selected for a, and the softmax is normalised
// over those keys.  The review of the paper (method summary, step (3)) runs
// this on the group-major layout with a variable-length block-sparse kernel.
//
// Work decomposition.  One work item = (head h, query group a, 128-row query
// tile).  The selected K/V groups of a are in ascending b, so in group-major
// K/V memory they form runs; the item streams the concatenation of its cells
// in 64-key tiles that cross cell boundaries (only the stream's last tile is
// masked), so no per-cell padding is spent.
//
// bf16 kernel (MFMA 32x32x16, fp32 accumulation), 4 waves, 32 query rows per
// wave.  Scores are formed transposed, S^T = K Q^T, so each lane owns one
// query and 32 of the tile's 64 keys; the row max/sum need a single exchange
// with the partner lane (lane ^ 32).  O^T = V^T P^T is accumulated likewise
// (one query per lane).  K is staged in LDS row-major with an XOR swizzle of
// 16-byte chunks; V is transposed into LDS (d rows) with keys reordered so
// the 8 keys a lane's P fragment holds are contiguous.  K/V tiles are double
// buffered in LDS and prefetched through registers one tile ahead.
// PV runs on fp16 MFMA: P (in [0, 1]) is rounded to fp16 and V is converted
// to fp16 after an exact power-of-two scale per head (chosen from the head's
// largest |v| so every normal bf16 value converts without rounding); O is
// scaled back at the end.  Rounding P to bf16 instead costs ~1.5e-3 relative
// error on O, which the fitted correction then amplifies past 2e-3.

#include "common.h"

namespace spr {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnArgs {
  const int32_t* off_q;
  const int32_t* off_k;
  const int32_t* rowptr;
  const int32_t* col;
  const void* q;
  const void* k;
  const void* v;
  float* o;
  float* lse;
  const int32_t* tiles;  // [H*c_q + 1] exclusive prefix of per-group tile counts
  const uint32_t* vmax;  // [H] largest |v| bit pattern of the head (bf16 path)
  int H, n_q, n_k, c_q, c_k;
  float scale_log2;      // softmax_scale * log2(e)
  int grid_blocks;       // launched blocks (multiple of 8)
};

// tiles[h*c_q + a] = sum over earlier (h, a) of ceil(n_a / tq); tiles[H*c_q] = total.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ off_q, int H,
                                                         int c_q, int tq,
                                                         int32_t* __restrict__ tiles,
                                                         uint32_t* __restrict__ vmax) {
  __shared__ long long red[16];
  for (int i = threadIdx.x; i < H; i += blockDim.x) vmax[i] = 0u;
  const long long len = (long long)H * c_q;
  const long long per = (len + blockDim.x - 1) / blockDim.x;
  const long long lo = per * threadIdx.x, hi = lo + per < len ? lo + per : len;
  auto count = [&](long long e) -> int {
    int h = int(e / c_q), a = int(e - (long long)h * c_q);
    const int32_t* o = off_q + (long long)h * (c_q + 1);
    int n = o[a + 1] - o[a];
    return (n + tq - 1) / tq;
  };
  long long s = 0;
  for (long long e = lo; e < hi; ++e) s += count(e);
  long long tot;
  long long run = block_exclusive_scan(s, red, &tot);
  for (long long e = lo; e < hi; ++e) {
    tiles[e] = int32_t(run);
    run += count(e);
  }
  if (threadIdx.x == 0) tiles[len] = int32_t(tot);
}

// Largest |v| of every head as a bf16 bit pattern (sign cleared); positive
// bf16 patterns order like their values.
constexpr int kVmaxRows = 1024;
__global__ __launch_bounds__(256) void vmax_kernel(const uint16_t* __restrict__ v, int n_k, int d,
                                                  uint32_t* __restrict__ vmax) {
  const int h = blockIdx.y;
  const long long r0 = (long long)blockIdx.x * kVmaxRows;
  const long long r1 = r0 + kVmaxRows < n_k ? r0 + kVmaxRows : n_k;
  const uint4* src = reinterpret_cast<const uint4*>(v + ((long long)h * n_k) * d);
  const long long c0 = r0 * d / 8, c1 = r1 * d / 8;
  uint32_t mx = 0;
  for (long long c = c0 + threadIdx.x; c < c1; c += 256) {
    const uint4 w = src[c];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mx = max(mx, ws[j] & 0x7fffu);
      mx = max(mx, (ws[j] >> 16) & 0x7fffu);
    }
  }
  mx = wave_max(mx);
  if ((threadIdx.x & 63) == 0) atomicMax(&vmax[h], mx);
}

// Maps a launched block to (h, a, tile-in-group).  Blocks are dealt to the 8
// XCDs round-robin by id; the remap gives each XCD a contiguous range of
// work items so tiles of one query group (same K/V stream) share an L2.
SPR_DEV bool locate_item(const AttnArgs& p, int& h, int& a, int& kt) {
  const int bid = blockIdx.x;
  const int per_xcd = p.grid_blocks >> 3;
  const int lid = (bid & 7) * per_xcd + (bid >> 3);
  const int total = p.tiles[p.H * p.c_q];
  if (lid >= total) return false;
  int lo = 0, hi = p.H * p.c_q - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (p.tiles[mid] <= lid) lo = mid;
    else hi = mid - 1;
  }
  h = lo / p.c_q;
  a = lo - h * p.c_q;
  kt = lid - p.tiles[lo];
  return true;
}

// Loads the cell list of (h, a) into LDS: cstart = first K/V row of each
// selected cell, cpos = exclusive prefix of the cell lengths; returns the
// stream length L.  256 threads, <= 1024 cells.
SPR_DEV int load_cells(const AttnArgs& p, int h, int a, int32_t* cstart, int32_t* cpos,
                       long long* red) {
  const int32_t* rp = p.rowptr + (long long)h * (p.c_q + 1);
  const int c0 = rp[a], nc = rp[a + 1] - c0;
  const int32_t* cl = p.col + (long long)h * p.c_q * p.c_k + c0;
  const int32_t* ok = p.off_k + (long long)h * (p.c_k + 1);
  int len[4];
  long long s = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int i = 4 * threadIdx.x + j;
    len[j] = 0;
    if (i < nc) {
      int b = cl[i];
      int st = ok[b];
      cstart[i] = st;
      len[j] = ok[b + 1] - st;
    }
    s += len[j];
  }
  long long tot;
  long long run = block_exclusive_scan(s, red, &tot);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int i = 4 * threadIdx.x + j;
    if (i < nc) cpos[i] = int32_t(run);
    run += len[j];
  }
  if (threadIdx.x == 0) cpos[nc] = int32_t(tot);
  __syncthreads();
  return int(tot);
}

// largest c with cpos[c] <= pos (cells are non-empty, so cpos is increasing)
SPR_DEV int find_cell(const int32_t* cpos, int nc, int pos) {
  int lo = 0, hi = nc - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cpos[mid] <= pos) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// bf16 MFMA kernel
// ---------------------------------------------------------------------------
template <int D>
struct SmemBf16 {
  uint16_t k[2][64 * D];
  uint16_t vt[2][D * 64];
  int32_t cstart[SPARSEPR_MAX_GROUPS];
  int32_t cpos[SPARSEPR_MAX_GROUPS + 1];
  long long red[4];
};

// key position inside a 64-key tile of V^T: quads 1 and 2 of every 16 keys swap
SPR_DEV int vt_key_pos(int kq) {
  const int q4 = kq & 3;
  const int pq = q4 == 1 ? 2 : (q4 == 2 ? 1 : q4);
  return 16 * (kq >> 2) + 4 * pq;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_bf16_kernel(AttnArgs p) {
  constexpr int DCH = D / 8;          // 16-byte chunks per row
  constexpr int NBLK = 16 * DCH;      // (key quad, dim chunk) load blocks per tile
  constexpr int NS = D / 16;          // k-steps of the QK^T product
  constexpr int NDB = D / 32;         // 32-wide d blocks of the output
  __shared__ SmemBf16<D> sm;

  int h, a, kt;
  if (!locate_item(p, h, a, kt)) return;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, n = lane & 31, g = lane >> 5;
  const int32_t* oq = p.off_q + (long long)h * (p.c_q + 1);
  const int r0 = oq[a] + kt * 128;
  const int nrows = min(128, oq[a + 1] - r0);
  const int nc = p.rowptr[(long long)h * (p.c_q + 1) + a + 1] -
                 p.rowptr[(long long)h * (p.c_q + 1) + a];
  const int L = load_cells(p, h, a, sm.cstart, sm.cpos, sm.red);

  const uint16_t* Kh = static_cast<const uint16_t*>(p.k) + (long long)h * p.n_k * D;
  const uint16_t* Vh = static_cast<const uint16_t*>(p.v) + (long long)h * p.n_k * D;
  // V scale 2^-sv puts the head's largest |v| in [2^14, 2^15): fp16 keeps
  // every bf16 mantissa exactly down to 2^-28 of that maximum
  int sv;
  {
    const int E = int((p.vmax[h] >> 7) & 0xffu);
    sv = (E == 0 ? -127 : E - 127) - 14;
    sv = sv < -100 ? -100 : (sv > 100 ? 100 : sv);
  }
  const float vscale = __builtin_ldexpf(1.f, -sv);

  // query fragments: lane holds row n, dims 16s + 8g .. +8
  const int qloc = wid * 32 + n;
  const bool wave_active = wid * 32 < nrows;
  const bool row_valid = qloc < nrows;
  bf16x8_t qf[NS];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) +
                           ((long long)h * p.n_q + r0 + (row_valid ? qloc : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      uint4 w = row_valid ? *reinterpret_cast<const uint4*>(qrow + 16 * s + 8 * g)
                          : make_uint4(0, 0, 0, 0);
      qf[s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // loader role: key quad kq (keys 4kq..4kq+3 of the tile), dim chunk dc
  const bool loader = tid < NBLK;
  const int kq = tid / DCH, dc = tid % DCH;
  uint4 kreg[4], vreg[4];
  auto load_tile = [&](int t) {
    if (!loader) return;
    const int p0 = t * 64 + 4 * kq;
    int c = p0 < L ? find_cell(sm.cpos, nc, p0) : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = p0 + i;
      if (pos < L) {
        while (sm.cpos[c + 1] <= pos) ++c;
        const long long row = sm.cstart[c] + (pos - sm.cpos[c]);
        kreg[i] = *reinterpret_cast<const uint4*>(Kh + row * D + 8 * dc);
        vreg[i] = *reinterpret_cast<const uint4*>(Vh + row * D + 8 * dc);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store_tile = [&](int buf) {
    if (!loader) return;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * kq + i;
      const int pc = dc ^ (r & (DCH - 1));
      *reinterpret_cast<uint4*>(&sm.k[buf][r * D + pc * 8]) = kreg[i];
    }
    const int kpos = vt_key_pos(kq);
    const int chunk = kpos >> 3, half = (kpos >> 2) & 1;
    uint32_t hv[4][4];  // [key][dim pair] fp16 pairs
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int m2 = 0; m2 < 4; ++m2) {
        const _Float16 lo16 = static_cast<_Float16>(__uint_as_float(w[m2] << 16) * vscale);
        const _Float16 hi16 = static_cast<_Float16>(__uint_as_float(w[m2] & 0xffff0000u) * vscale);
        hv[i][m2] = uint32_t(__builtin_bit_cast(uint16_t, lo16)) |
                    (uint32_t(__builtin_bit_cast(uint16_t, hi16)) << 16);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int m = j >> 1;
      uint32_t lo, hi;
      if ((j & 1) == 0) {
        lo = (hv[0][m] & 0xffffu) | (hv[1][m] << 16);
        hi = (hv[2][m] & 0xffffu) | (hv[3][m] << 16);
      } else {
        lo = (hv[0][m] >> 16) | (hv[1][m] & 0xffff0000u);
        hi = (hv[2][m] >> 16) | (hv[3][m] & 0xffff0000u);
      }
      const int d = 8 * dc + j;
      const int pc = chunk ^ ((d >> 1) & 7);
      *reinterpret_cast<uint2*>(&sm.vt[buf][d * 64 + pc * 8 + half * 4]) = make_uint2(lo, hi);
    }
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const float sl2 = p.scale_log2;

  auto compute = [&](int t, int buf) {
    f32x16_t sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16_t{};
      const int r = 32 * kb + n;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int pc = (2 * s + g) ^ (r & (DCH - 1));
        const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&sm.k[buf][r * D + pc * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, qf[s], sacc[kb], 0, 0, 0);
      }
    }
    const int tail = L - t * 64;   // valid keys in this tile (may exceed 64)
    float mloc = -__builtin_huge_valf();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 32 * kb + 8 * (i >> 2) + 4 * g + (i & 3);
        float x = kk < tail ? sacc[kb][i] * sl2 : -__builtin_huge_valf();
        sacc[kb][i] = x;
        mloc = fmaxf(mloc, x);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = __builtin_amdgcn_exp2f(sacc[kb][i] - m_new);
        sacc[kb][i] = e;
        lsum += e;
      }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    f16x8_t pf[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int kb = u >> 1, base = 8 * (u & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[u][j] = static_cast<_Float16>(sacc[kb][base + j]);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = 32 * db + n;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int pc = (2 * u + g) ^ ((d >> 1) & 7);
        const f16x8_t af = *reinterpret_cast<const f16x8_t*>(&sm.vt[buf][d * 64 + pc * 8]);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, pf[u], oacc[db], 0, 0, 0);
      }
    }
  };

  const int ntiles = (L + 63) / 64;
  load_tile(0);
  store_tile(0);
  if (ntiles > 1) load_tile(1);
  __syncthreads();
  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (wave_active) compute(t, buf);
    if (t + 1 < ntiles) store_tile(buf ^ 1);
    if (t + 2 < ntiles) load_tile(t + 2);
    __syncthreads();
  }

  if (!row_valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = __builtin_ldexpf(1.f, sv) / l_tot;
  float* orow = p.o + ((long long)h * p.n_q + r0 + qloc) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v = make_float4(oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv,
                             oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
      *reinterpret_cast<float4*>(orow + 32 * db + 8 * i4 + 4 * g) = v;
    }
  if (g == 0 && p.lse) p.lse[(long long)h * p.n_q + r0 + qloc] = (m_run + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 VALU kernel: LPQ lanes per query, 32 dims per lane, 32-key LDS tiles
// ---------------------------------------------------------------------------
template <int D>
struct SmemF32 {
  float k[32][D + 4];
  float v[32][D + 4];
  int32_t cstart[SPARSEPR_MAX_GROUPS];
  int32_t cpos[SPARSEPR_MAX_GROUPS + 1];
  long long red[4];
};

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs p) {
  constexpr int LPQ = D / 32;
  constexpr int TQ = 256 / LPQ;
  __shared__ SmemF32<D> sm;
  int h, a, kt;
  if (!locate_item(p, h, a, kt)) return;
  const int tid = threadIdx.x;
  const int32_t* oq = p.off_q + (long long)h * (p.c_q + 1);
  const int r0 = oq[a] + kt * TQ;
  const int nrows = min(TQ, oq[a + 1] - r0);
  const int nc = p.rowptr[(long long)h * (p.c_q + 1) + a + 1] -
                 p.rowptr[(long long)h * (p.c_q + 1) + a];
  const int L = load_cells(p, h, a, sm.cstart, sm.cpos, sm.red);
  const float* Kh = static_cast<const float*>(p.k) + (long long)h * p.n_k * D;
  const float* Vh = static_cast<const float*>(p.v) + (long long)h * p.n_k * D;
  const int qi = tid / LPQ, sl = tid % LPQ;
  const bool valid = qi < nrows;
  float q[32], o[32];
  const float* qrow = static_cast<const float*>(p.q) +
                      ((long long)h * p.n_q + r0 + (valid ? qi : 0)) * D + 32 * sl;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    q[i] = valid ? qrow[i] : 0.f;
    o[i] = 0.f;
  }
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const int ntiles = (L + 31) / 32;
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    for (int e = tid; e < 32 * (D / 4); e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      const int pos = t * 32 + r;
      float4 kv = make_float4(0, 0, 0, 0), vv = make_float4(0, 0, 0, 0);
      if (pos < L) {
        const int c = find_cell(sm.cpos, nc, pos);
        const long long row = sm.cstart[c] + (pos - sm.cpos[c]);
        kv = *reinterpret_cast<const float4*>(Kh + row * D + 4 * c4);
        vv = *reinterpret_cast<const float4*>(Vh + row * D + 4 * c4);
      }
      *reinterpret_cast<float4*>(&sm.k[r][4 * c4]) = kv;
      *reinterpret_cast<float4*>(&sm.v[r][4 * c4]) = vv;
    }
    __syncthreads();
    const int tail = L - t * 32;
    float s[32];
    float mloc = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) acc = fmaf(q[i], sm.k[j][32 * sl + i], acc);
#pragma unroll
      for (int o2 = 1; o2 < LPQ; o2 <<= 1) acc += __shfl_xor(acc, o2);
      s[j] = j < tail ? acc * p.scale_log2 : -__builtin_huge_valf();
      mloc = fmaxf(mloc, s[j]);
    }
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < 32; ++i) o[i] *= alpha;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      const float e = exp2f(s[j] - m_new);
      l_run += e;
#pragma unroll
      for (int i = 0; i < 32; ++i) o[i] = fmaf(e, sm.v[j][32 * sl + i], o[i]);
    }
  }
  if (!valid) return;
  const float inv = 1.f / l_run;
  float* orow = p.o + ((long long)h * p.n_q + r0 + qi) * D + 32 * sl;
#pragma unroll
  for (int i = 0; i < 32; i += 4)
    *reinterpret_cast<float4*>(orow + i) =
        make_float4(o[i] * inv, o[i + 1] * inv, o[i + 2] * inv, o[i + 3] * inv);
  if (sl == 0 && p.lse) p.lse[(long long)h * p.n_q + r0 + qi] = (m_run + __log2f(l_run)) * kLn2;
}

int rows_per_item(const sparsepr_dims* d) {
  if (d->dtype == SPARSEPR_BF16) return 128;
  return 256 / (d->head_dim / 32);
}

}  // namespace

size_t attn_ws_bytes(const sparsepr_dims* d) {
  Carver cv(nullptr);
  cv.take<int32_t>(size_t(d->heads) * d->c_q + 1);
  cv.take<uint32_t>(size_t(d->heads));
  return cv.used;
}

}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_sparse_attn(const sparsepr_dims* dims, const int32_t* offsets_q,
                                        const int32_t* offsets_kv, const int32_t* cell_rowptr,
                                        const int32_t* cell_col, const void* q_g, const void* k_g,
                                        const void* v_g, float softmax_scale, float* o_sp,
                                        float* lse, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!offsets_q || !offsets_kv || !cell_rowptr || !cell_col || !q_g || !k_g || !v_g || !o_sp)
    return SPARSEPR_ERR_INVALID;
  const size_t need = attn_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  Carver cv(ws);
  int32_t* tiles = cv.take<int32_t>(size_t(dims->heads) * dims->c_q + 1);
  uint32_t* vmax = cv.take<uint32_t>(size_t(dims->heads));
  const int tq = rows_per_item(dims);
  tile_table_kernel<<<1, 1024, 0, stream>>>(offsets_q, dims->heads, dims->c_q, tq, tiles, vmax);
  SPR_LAUNCH_CHECK();
  if (dims->dtype == SPARSEPR_BF16) {
    dim3 g((dims->n_k + kVmaxRows - 1) / kVmaxRows, dims->heads);
    vmax_kernel<<<g, 256, 0, stream>>>(static_cast<const uint16_t*>(v_g), dims->n_k,
                                       dims->head_dim, vmax);
    SPR_LAUNCH_CHECK();
  }
  // upper bound of work items: sum_a ceil(n_a / tq) <= N_q / tq + C_q per head
  long long bound = (long long)dims->heads * ((dims->n_q + tq - 1) / tq + dims->c_q);
  bound = (bound + 7) & ~7LL;
  if (bound > 0x7fffffffLL) return SPARSEPR_ERR_UNSUPPORTED;
  AttnArgs a;
  a.off_q = offsets_q;
  a.off_k = offsets_kv;
  a.rowptr = cell_rowptr;
  a.col = cell_col;
  a.q = q_g;
  a.k = k_g;
  a.v = v_g;
  a.o = o_sp;
  a.lse = lse;
  a.tiles = tiles;
  a.vmax = vmax;
  a.H = dims->heads;
  a.n_q = dims->n_q;
  a.n_k = dims->n_k;
  a.c_q = dims->c_q;
  a.c_k = dims->c_k;
  a.scale_log2 = softmax_scale * kLog2e;
  a.grid_blocks = int(bound);
  if (dims->dtype == SPARSEPR_BF16) {
    if (dims->head_dim == 128) attn_bf16_kernel<128><<<int(bound), 256, 0, stream>>>(a);
    else attn_bf16_kernel<64><<<int(bound), 256, 0, stream>>>(a);
  } else {
    if (dims->head_dim == 128) attn_f32_kernel<128><<<int(bound), 256, 0, stream>>>(a);
    else attn_f32_kernel<64><<<int(bound), 256, 0, stream>>>(a);
  }
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}
