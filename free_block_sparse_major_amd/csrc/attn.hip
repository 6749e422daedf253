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
// (one query per lane).  K and V tiles are double buffered in LDS and loaded
// one tile ahead directly from global memory; V^T fragments come from
// hardware transposing LDS reads, so V stays row-major.
// PV runs on fp16 MFMA: P (in [0, 1]) is rounded to fp16 and V arrives as
// fp16 after an exact power-of-two scale per head (the layout call chooses
// it from the head's largest |v|, so every normal bf16 value converts without
// rounding); O is scaled back at the end.  Rounding P to bf16 instead costs
// ~1.5e-3 relative error on O, which the fitted correction then amplifies
// past 2e-3.

#include "common.h"
#include "lds_dma.h"
#include "mfma_tiles.h"

#include <mutex>

namespace spr {
namespace {


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
  const int2* items;     // launch order of the work items (h * c_q + a, tile), or null
  const int32_t* v_shift;  // [H] v_g holds fp16(v * 2^-v_shift) (bf16 path)
  int H, n_q, n_k, c_q, c_k;
  float scale_log2;      // softmax_scale * log2(e)
  int grid_blocks;       // launched blocks (multiple of 8)
  // fused correction (the attention writes the corrected output in token
  // order instead of O_sp): out = o + (o A) Psi^T + g * o + c
  const int32_t* perm_q;     // [H][N_q] group-major row -> token
  const float* corr_a;       // [H][D][rank]
  const float* corr_psi_t;   // [H][rank][D]
  const float* corr_c;       // [H][D]
  const float* corr_g;       // [H][D] or null
  void* out;
  long long out_sh, out_st;  // element strides of out
  int out_bf16, rank;
  int splits;            // fp32 kernel: key-stream splits per item (1: no partials)
  float* part_o;         // [splits][H * n_q][D] unnormalised partial outputs
  float* part_ml;        // [splits][H * n_q][2] (max * scale_log2, sum) per partial
};

// tiles[h*c_q + a] = sum over earlier (h, a) of ceil(n_a / tq); tiles[H*c_q] = total.
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ off_q, int H,
                                                         int c_q, int tq,
                                                         int32_t* __restrict__ tiles) {
  __shared__ long long red[16];
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

// Longest-first order of the work items.  Block b orders the query groups
// of head b (the last block those of the last two heads together) by
// descending cost L_a * min(n_a, tq), L_a the length of the group's key
// stream, ties by group index; the items of a group stay consecutive (tile
// order) and heads keep their order, so the items in flight still cover
// about one head's K/V, and the list ends with the shortest items of the last
// two heads (largest-first list scheduling evens out the finishing times).
// Launches with few items per compute unit (all_heads = 1, one block) order
// the groups of all heads together instead: there every unit runs only one
// or two items, and a per-head order would still pair long items with long
// ones (key streams at the CogVideoX-like shape range over 1.4k-9.6k keys).
// The list is indexed by block id.  Blocks are dealt to the 8 XCDs round-robin,
// so XCD x runs positions x, x + 8, ...; positions 8..15 of every complete
// 16-position window are reversed, so that no XCD always takes the larger
// item of each consecutive 8 (the XCDs' shares of the sorted costs balance).
constexpr int kOrderMax = 2 * SPARSEPR_MAX_GROUPS;
__global__ __launch_bounds__(1024) void item_order_kernel(
    const int32_t* __restrict__ off_q, const int32_t* __restrict__ off_k,
    const int32_t* __restrict__ rowptr, const int32_t* __restrict__ col, int H, int c_q, int c_k,
    int tq, const int32_t* __restrict__ tiles, int2* __restrict__ items, int all_heads) {
  __shared__ unsigned long long key[kOrderMax];
  __shared__ int32_t len_g[kOrderMax];
  __shared__ int32_t okl[SPARSEPR_MAX_GROUPS + 1], rpl[SPARSEPR_MAX_GROUPS + 1];
  __shared__ long long red[16];
  const int h0 = all_heads ? 0 : int(blockIdx.x);
  const int nh = all_heads ? H : ((H >= 2 && h0 == H - 2) ? 2 : 1);   // nh * c_q <= kOrderMax
  const int nent = nh * c_q;
  for (int e = threadIdx.x; e < kOrderMax; e += blockDim.x) len_g[e] = 0;
  // key-stream length of every group: 16 lanes per group sum the K/V group
  // sizes of its cells (contiguous in the cell table) and reduce
  const int lane = threadIdx.x & 15, wv = threadIdx.x >> 4, nwv = blockDim.x >> 4;
  if (all_heads) {
    // every group of every head at once, reading the tables in global memory
    // (a per-head pass would wait for its loads once per head): LPE lanes per
    // group, as many as the block holds, at most 16
    __syncthreads();
    int lpe = 16;
    while (lpe > 1 && lpe * nent > int(blockDim.x)) lpe >>= 1;
    const int sub = threadIdx.x % lpe, grp = threadIdx.x / lpe, ngrp = blockDim.x / lpe;
    for (int e = grp; e < nent; e += ngrp) {
      const int h = e / c_q, a = e - (e / c_q) * c_q;
      const int32_t* rp = rowptr + (long long)h * (c_q + 1);
      const int32_t* cl = col + (long long)h * c_q * c_k;
      const int32_t* ok = off_k + (long long)h * (c_k + 1);
      const int c0 = rp[a], c1 = rp[a + 1];
      int sum = 0;
      for (int i = c0 + sub; i < c1; i += 4 * lpe) {
        int b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = i + lpe * u < c1 ? cl[i + lpe * u] : -1;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (b[u] >= 0) sum += ok[b[u] + 1] - ok[b[u]];
      }
      for (int o = lpe >> 1; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (sub == 0) len_g[e] = sum;
    }
  }
  for (int hh = 0; hh < (all_heads ? 0 : nh); ++hh) {
    const int h = h0 + hh;
    __syncthreads();
    for (int i = threadIdx.x; i <= c_k; i += blockDim.x) okl[i] = off_k[(long long)h * (c_k + 1) + i];
    for (int i = threadIdx.x; i <= c_q; i += blockDim.x) rpl[i] = rowptr[(long long)h * (c_q + 1) + i];
    __syncthreads();
    const int32_t* cl = col + (long long)h * c_q * c_k;
    for (int a = wv; a < c_q; a += nwv) {
      const int c0 = rpl[a], c1 = rpl[a + 1];
      int sum = 0;
      for (int i = c0 + lane; i < c1; i += 4 * 16) {
        int b[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) b[u] = i + 16 * u < c1 ? cl[i + 16 * u] : -1;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (b[u] >= 0) sum += okl[b[u] + 1] - okl[b[u]];
      }
#pragma unroll
      for (int o = 8; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
      if (lane == 0) len_g[hh * c_q + a] = sum;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kOrderMax; e += blockDim.x) {
    unsigned long long v = 0;   // padding sorts last
    if (e < nent) {
      const int h = h0 + e / c_q, a = e % c_q;
      const int32_t* oq = off_q + (long long)h * (c_q + 1);
      const int n = oq[a + 1] - oq[a];
      // empty group: no items, sorts after the others
      const long long cost = n > 0 ? (long long)len_g[e] * (long long)(n < tq ? n : tq) : -1;
      v = ((unsigned long long)(cost + 2) << 12) | (unsigned long long)(4095 - e);
    }
    key[e] = v;
  }
  __syncthreads();
  // bitonic sort of the first N >= nent entries (the rest is padding), descending
  int N = 64;
  while (N < nent) N <<= 1;
  for (int k = 2; k <= N; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int pr = threadIdx.x; pr < N / 2; pr += blockDim.x) {
        const int i = (pr / j) * 2 * j + (pr % j), l = i + j;
        const unsigned long long x = key[i], y = key[l];
        const bool desc = (i & k) == 0;
        if (desc ? (x < y) : (x > y)) {
          key[i] = y;
          key[l] = x;
        }
      }
      __syncthreads();
    }
  }
  // items per sorted entry, scanned in sorted order (two entries per thread)
  auto entry_tiles = [&](int r, int& ent) {
    ent = 4095 - int(key[r] & 4095ull);
    if (ent >= nent) return 0;
    const int h = h0 + ent / c_q, a = ent % c_q;
    const int32_t* oq = off_q + (long long)h * (c_q + 1);
    const int n = oq[a + 1] - oq[a];
    return (n + tq - 1) / tq;
  };
  const int per = kOrderMax / blockDim.x;
  int ent[kOrderMax / 1024 > 0 ? kOrderMax / 1024 : 1];
  int cnt[kOrderMax / 1024 > 0 ? kOrderMax / 1024 : 1];
  long long s = 0;
  for (int j = 0; j < per; ++j) {
    cnt[j] = entry_tiles(per * threadIdx.x + j, ent[j]);
    s += cnt[j];
  }
  long long tot;
  long long run = block_exclusive_scan(s, red, &tot) + tiles[(long long)h0 * c_q];
  const long long total = tiles[(long long)H * c_q];
  const long long full = total / 16 * 16;   // positions in complete 16-windows
  for (int j = 0; j < per; ++j) {
    if (cnt[j] > 0) {
      const int h = h0 + ent[j] / c_q, a = ent[j] % c_q;
      for (int t = 0; t < cnt[j]; ++t) {
        long long pos = run + t;
        if (pos < full && (pos & 8)) pos = (pos & ~7ll) + 7 - (pos & 7);
        items[pos] = make_int2(h * c_q + a, t);
      }
    }
    run += cnt[j];
  }
}

// Maps a launched block to (h, a, tile-in-group).  With the ordered list (the
// entry points with a workspace) the block id indexes it.  Otherwise (the
// entry point without one) items go in (h, a, tile) order: blocks are dealt
// to the 8 XCDs round-robin by id, and the remap hands each XCD runs of kXcdRun
// consecutive work items (tiles of one query group, same K/V stream, share
// that XCD's L2) while the 8 XCDs interleave run by run, so the blocks in
// flight across the GPU cover about one head: its K/V (tens of MB) stays in
// the last-level cache instead of eight heads competing for it.
constexpr int kXcdRun = 8;
SPR_DEV bool locate_item(const AttnArgs& p, int& h, int& a, int& kt) {
  const int bid = blockIdx.x;
  const int total = p.tiles[p.H * p.c_q];
  if (p.items) {
    // ordered list, indexed by block id (blocks past the end exit)
    if (bid >= total) return false;
    const int2 it = p.items[bid];
    h = it.x / p.c_q;
    a = it.x - h * p.c_q;
    kt = it.y;
    return true;
  }
  const int x = bid & 7, j = bid >> 3;
  const int lid = (j / kXcdRun) * (8 * kXcdRun) + x * kXcdRun + (j % kXcdRun);
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
// stream length L.  NT threads, <= 1024 cells.
template <int NT>
SPR_DEV int load_cells(const AttnArgs& p, int h, int a, int32_t* cstart, int32_t* cpos,
                       long long* red) {
  constexpr int PER = (SPARSEPR_MAX_GROUPS + NT - 1) / NT;
  const int32_t* rp = p.rowptr + (long long)h * (p.c_q + 1);
  const int c0 = rp[a], nc = rp[a + 1] - c0;
  const int32_t* cl = p.col + (long long)h * p.c_q * p.c_k + c0;
  const int32_t* ok = p.off_k + (long long)h * (p.c_k + 1);
  int len[PER];
  long long s = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    int i = PER * threadIdx.x + j;
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
  for (int j = 0; j < PER; ++j) {
    int i = PER * threadIdx.x + j;
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
// LDS tiles (per stage): K as 64 rows x D bf16, V as 64 rows x D fp16, both
// row-major in 16-byte chunks.  Tiles arrive straight from global memory
// (global_load_lds, 16 bytes per lane): lane l of a wave writes LDS bytes
// base + 16 l, so the XOR swizzle is applied by choosing which source chunk
// each lane fetches.
//   K chunk swizzle: physical = logical ^ (row & (CPR-1)); the QK^T A-operand
//   read (32 rows, one chunk) then hits distinct banks.
//   V chunk swizzle: physical = logical ^ swzV(row), a 64-byte-window rotation
//   that spreads the 8 rows touched by one transposed read over the banks.
// The PV A operand (V^T, 32 d x 16 keys) is read with ds_read_b64_tr_b16:
// inside each 16-lane group, source lane r points at 4 values
// V[k0 + r/4][d0 + 4(r%4) ..+3]; lane i then receives V[k0 + j][d0 + i] for
// j = 0..3, i.e. 4 consecutive keys of its own column.
struct SmemCells {
  int32_t cstart[SPARSEPR_MAX_GROUPS];
  int32_t cpos[SPARSEPR_MAX_GROUPS + 1];
  long long red[16];
};

template <int B>
struct Stage {
  static constexpr int value = B;
};



// Lazy rescale: P is formed against the running reference max and the row is
// rescaled to a new reference only when a lane's sum of its P values in the
// block exceeds this cap (every P above it, and any overflow to inf, implies
// that).  P therefore stays at or below 2^8, well inside fp16.
constexpr float kPSumCap = 256.f;

// Maximum rank of the correction fused into the attention epilogue.
constexpr int kFusedRank = 16;

// ---------------------------------------------------------------------------
// Correction in the attention epilogue, on bf16 MFMA with hi/lo operand
// splits (x = hi + lo, both bf16; products hi*hi + hi*lo + lo*hi accumulated
// in fp32: about 2^-16 relative per product, against 2^-8 for plain bf16).
//   u^T (ranks x rows) = A^T (ranks x D) O^T (D x rows)   [K = D, in 16-dim steps]
//   out^T = O^T + g * O^T + c + Psi (D x ranks) u^T        [K = 16 ranks]
// The O^T accumulator of the attention is the B operand of the first product
// as it stands: in 16-dim step s (d block s / 2, half t = s % 2) lane (n, g)
// supplies registers 8 t .. 8 t + 7 of its block, i.e. dims
//   dim(s, g, i) = 32 (s / 2) + 16 t + 8 (i / 4) + 4 g + i % 4,
// and the A^T tile lane (rank rho, g) supplies A[dim(s, g, i)][rho] (zero for
// rho >= 16).  The result u^T holds in lane (n, g) the ranks
//   rho(g, i) = 8 (i / 4) + 4 g + i % 4,  i = 0..7
// in registers 0..7 (8..15 are ranks 16..31, zero), which is the B operand of
// the second product with that rank order; the Psi tile lane (dim, g)
// supplies Psi^T[rho(g, i)][dim].  The second product's C layout is the O^T
// layout, so the accumulator starts at o + g * o + c.
// LDS (uint4 = 8 bf16):
//   [0, 4D)      A^T: ((s * 2 + g) * 16 + rho) * 2 + {hi, lo}
//   [4D, 8D)     Psi: ((db * 64) + lane) * 2 + {hi, lo}
//   [8D, 8D+D/2) c[D] then g[D] as floats
// ---------------------------------------------------------------------------
SPR_DEV uint32_t bf16_hi_bits(float x) { return __float_as_uint(x) >> 16; }  // truncation
SPR_DEV float bf16_hi_float(float x) { return __uint_as_float(__float_as_uint(x) & 0xffff0000u); }

// 8 floats -> (hi, lo) bf16 octets
SPR_DEV void split8(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float x0 = x[2 * k], x1 = x[2 * k + 1];
    h[k] = bf16_hi_bits(x0) | (bf16_hi_bits(x1) << 16);
    l[k] = uint32_t(f32_to_bf16_rne(x0 - bf16_hi_float(x0))) |
           (uint32_t(f32_to_bf16_rne(x1 - bf16_hi_float(x1))) << 16);
  }
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

template <int D, int NT>
SPR_DEV void stage_correction(const AttnArgs& p, int h, uint4* cs) {
  const float* A = p.corr_a + (long long)h * D * p.rank;
  const float* Pt = p.corr_psi_t + (long long)h * p.rank * D;
  const int rank = p.rank;
  // A^T tiles: D / 16 steps x 2 lane halves x 16 ranks
  for (int e = threadIdx.x; e < 2 * D; e += NT) {
    const int rho = e & 15, g = (e >> 4) & 1, st = e >> 5;
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int dim = 32 * (st >> 1) + 16 * (st & 1) + 8 * (i >> 2) + 4 * g + (i & 3);
      x[i] = rho < rank ? A[dim * rank + rho] : 0.f;
    }
    split8(x, cs[2 * e], cs[2 * e + 1]);
  }
  // Psi tiles: D / 32 blocks x 64 lanes
  for (int e = threadIdx.x; e < 2 * D; e += NT) {
    const int ln = e & 63, db = e >> 6, g = ln >> 5, dim = 32 * db + (ln & 31);
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int rho = 8 * (i >> 2) + 4 * g + (i & 3);
      x[i] = rho < rank ? Pt[rho * D + dim] : 0.f;
    }
    split8(x, cs[4 * D + 2 * e], cs[4 * D + 2 * e + 1]);
  }
  float* cg = reinterpret_cast<float*>(cs + 8 * D);
  for (int j = threadIdx.x; j < D; j += NT) {
    cg[j] = p.corr_c[(long long)h * D + j];
    cg[D + j] = p.corr_g ? p.corr_g[(long long)h * D + j] : 0.f;
  }
}

template <int D>
SPR_DEV void fused_epilogue_mfma(const AttnArgs& p, const uint4* cs, const f32x16_t* oacc,
                                 float inv, int lane, bool store, long long obase) {
  constexpr int NDB = D / 32;
  const int g = lane >> 5, rl = lane & 31;
  const bool rank_lane = rl < 16;
  f32x16_t uacc = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = oacc[st >> 1][8 * (st & 1) + i] * inv;
    uint4 bh, bl;
    split8(x, bh, bl);
    uint4 ah = make_uint4(0, 0, 0, 0), al = ah;
    if (rank_lane) {
      const int e = (st * 2 + g) * 16 + rl;
      ah = cs[2 * e];
      al = cs[2 * e + 1];
    }
    const bf16x8_t Ah = __builtin_bit_cast(bf16x8_t, ah), Al = __builtin_bit_cast(bf16x8_t, al);
    const bf16x8_t Bh = __builtin_bit_cast(bf16x8_t, bh), Bl = __builtin_bit_cast(bf16x8_t, bl);
    uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bh, uacc, 0, 0, 0);
    uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ah, Bl, uacc, 0, 0, 0);
    uacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Al, Bh, uacc, 0, 0, 0);
  }
  float uv[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) uv[i] = uacc[i];
  uint4 uh, ul;
  split8(uv, uh, ul);
  const bf16x8_t Uh = __builtin_bit_cast(bf16x8_t, uh), Ul = __builtin_bit_cast(bf16x8_t, ul);
  const float* cvec = reinterpret_cast<const float*>(cs + 8 * D);
  const float* gvec = cvec + D;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = 32 * db + 8 * (r >> 2) + 4 * g + (r & 3);
      const float o = oacc[db][r] * inv;
      acc[r] = fmaf(gvec[j], o, o + cvec[j]);
    }
    const int e = db * 64 + lane;
    const bf16x8_t Ph = __builtin_bit_cast(bf16x8_t, cs[4 * D + 2 * e]);
    const bf16x8_t Pl = __builtin_bit_cast(bf16x8_t, cs[4 * D + 2 * e + 1]);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ph, Uh, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Ph, Ul, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Pl, Uh, acc, 0, 0, 0);
    if (!store) continue;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int j0 = 32 * db + 8 * i4 + 4 * g;
      if (p.out_bf16) {
        uint2 pk;
        pk.x = uint32_t(f32_to_bf16_rne(acc[4 * i4])) |
               (uint32_t(f32_to_bf16_rne(acc[4 * i4 + 1])) << 16);
        pk.y = uint32_t(f32_to_bf16_rne(acc[4 * i4 + 2])) |
               (uint32_t(f32_to_bf16_rne(acc[4 * i4 + 3])) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + obase + j0) = pk;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + obase + j0) =
            make_float4(acc[4 * i4], acc[4 * i4 + 1], acc[4 * i4 + 2], acc[4 * i4 + 3]);
      }
    }
  }
}

template <int D, int W, bool FUSED>
__global__ __launch_bounds__(64 * W, W <= 4 ? 2 : 1) void attn_bf16_kernel(AttnArgs p) {
  constexpr int NT = 64 * W;          // threads
  constexpr int ROWS = 32 * W;        // query rows per work item
  constexpr int CPR = D / 8;          // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;       // rows per 1 KB wave load
  constexpr int KT = W >= 8 ? 128 : 64;  // keys per LDS tile
  constexpr int NL = KT / RPI;        // wave loads per tensor per tile
  constexpr int NI = (NL + W - 1) / W;  // wave loads per tensor per tile and wave (at most)
  constexpr int NS = D / 16;          // k-steps of QK^T
  constexpr int NDB = D / 32;         // 32-wide d blocks of the output
  constexpr int RB = D * 2;           // row bytes (bf16 K, fp16 V)
  // separate objects per stage: lets the compiler see that loads into one
  // stage never alias reads of the other (no blanket wait before LDS reads)
  __shared__ uint4 k_s0[KT / 8 * D], k_s1[KT / 8 * D];   // KT rows x D bf16
  __shared__ uint4 v_s0[KT / 8 * D], v_s1[KT / 8 * D];   // KT rows x D fp16
  __shared__ SmemCells sm;
  // fused correction operands, staged as bf16 hi/lo pairs in MFMA operand
  // order (see fused_epilogue_mfma): A^T tiles, Psi tiles, then c and g
  __shared__ uint4 corr_s[FUSED ? 8 * D + D / 2 : 1];

  int h, a, kt;
  if (!locate_item(p, h, a, kt)) return;
  if constexpr (FUSED) stage_correction<D, NT>(p, h, corr_s);
  // wave index as a scalar: everything derived from it (LDS destinations of the
  // tile loads, row ranges) stays in SGPRs
  const int tid = threadIdx.x, wid = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63,
            n = lane & 31, g = lane >> 5;
  const int32_t* oq = p.off_q + (long long)h * (p.c_q + 1);
  const int r0 = oq[a] + kt * ROWS;
  const int nrows = min(ROWS, oq[a + 1] - r0);
  const int L = load_cells<NT>(p, h, a, sm.cstart, sm.cpos, sm.red);
  const int ntiles = (L + KT - 1) / KT;
  // cell table -> (next boundary, row delta): row(pos) = pos + delta of its cell
  const int nc = p.rowptr[(long long)h * (p.c_q + 1) + a + 1] -
                 p.rowptr[(long long)h * (p.c_q + 1) + a];
  for (int i = tid; i < nc; i += NT) sm.cstart[i] -= sm.cpos[i];
  __syncthreads();

  const uint32_t head_bytes = uint32_t(p.n_k) * RB;
  const v4i32_t krs =
      head_rsrc(static_cast<const char*>(p.k) + (long long)h * p.n_k * RB, head_bytes);
  const v4i32_t vrs =
      head_rsrc(static_cast<const char*>(p.v) + (long long)h * p.n_k * RB, head_bytes);
  const int sv = p.v_shift[h];

  // query fragments: lane holds row n, dims 16s + 8g .. +8
  // Row chunk (32 query rows) and key blocks of this wave.  Wave w sits on
  // SIMD w % 4.  With 9 or 10 busy chunks in a 12-wave item, two SIMDs would
  // carry three busy waves and two SIMDs only two; instead the idle waves take
  // a share of the 32-key blocks of chunks 8 and 9 (disjoint per wave, the
  // same rows), so every SIMD carries the same work per tile, and the partial
  // softmax states are merged at the end.
  const int nb = (nrows + 31) / 32;
  int chunk = wid;
  uint32_t kmask = (1u << (KT / 32)) - 1u;
  int merge_slot = -1;   // helpers: slot of their partial state
  if constexpr (W >= 12 && KT == 128) {
    if (nb == 9 && wid >= 8) {
      chunk = 8;
      kmask = 1u << (wid - 8);
      merge_slot = wid - 9;
    } else if (nb == 10 && wid >= 8) {
      chunk = 8 + (wid & 1);
      kmask = wid < 10 ? 0x5u : 0xau;
      merge_slot = wid - 10;
    }
  }
  const int qloc = chunk * 32 + n;
  const bool wave_active = chunk * 32 < nrows;
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
  // Q fragments complete here (vmcnt(0)); otherwise the first use inside the
  // loop would wait on the whole vector-memory queue, tile prefetch included
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // loader: wave load i of wave w covers tile rows RPI*(w + i*W) .. +RPI.
  // tc (wave-uniform) is a cell with cpos[tc] <= the tile's first stream
  // position.  One LDS read fetches the next four cell ends (lanes 0-3) and
  // the row deltas of cells tc..tc+3 (lanes 4-7); they are broadcast to
  // scalars.  A wave load whose RPI rows lie in one cell (the common case) is
  // a scalar base plus a per-lane offset fixed for the whole kernel (with W a
  // multiple of 4, a wave's load rows have the same residue mod 16, so the
  // chunk swizzles below do not change from load to load).  A load that
  // straddles a cell end or the stream's end takes the per-lane path: each
  // lane counts the window boundaries at or below its position (walking on
  // past the window if needed).
  static_assert(W % 4 == 0, "per-lane load offsets assume W % 4 == 0");
  int tc = 0;
  const int lrow0 = lane / CPR, lpc0 = lane % CPR;
  const int lrow_w = wid * RPI + lrow0;                       // a load row of this wave
  const uint32_t voff_k = uint32_t(lrow0 * RB + ((lpc0 ^ (lrow_w & (CPR - 1))) * 16));
  const uint32_t voff_v = uint32_t(lrow0 * RB + ((lpc0 ^ swz_v<D>(lrow_w)) * 16));
  auto issue_tile = [&](auto stage, int t) __attribute__((always_inline)) {
    constexpr int B = decltype(stage)::value;
    uint4* kbase = B == 0 ? k_s0 : k_s1;
    uint4* vbase = B == 0 ? v_s0 : v_s1;
    const int t0 = t * KT;
    int wv;
    {
      const int j = lane & 3;
      wv = (lane & 4) ? sm.cstart[min(tc + j, nc - 1)] : sm.cpos[min(tc + 1 + j, nc)];
    }
    int e[4], dl[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = __builtin_amdgcn_readlane(wv, j);
      dl[j] = __builtin_amdgcn_readlane(wv, 4 + j);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int blk = wid + i * W;                        // wave-uniform
      if (NL % W != 0 && blk >= NL) break;
      uint4* kdst = kbase + blk * RPI * CPR;
      uint4* vdst = vbase + blk * RPI * CPR;
      const uint32_t lk = __builtin_amdgcn_readfirstlane(lds_addr_of(kdst));
      const uint32_t lv = __builtin_amdgcn_readfirstlane(lds_addr_of(vdst));
      const int p0 = t0 + blk * RPI;                       // first stream position
      // the first window cell ending after p0 (cell ends increase): its end and
      // row delta, chosen by scalar compare-and-select (e[3] if none does)
      int en = e[3], d0 = dl[3];
      if (p0 < e[2]) en = e[2], d0 = dl[2];
      if (p0 < e[1]) en = e[1], d0 = dl[1];
      if (p0 < e[0]) en = e[0], d0 = dl[0];
      if (p0 + RPI <= en) {
        // all rows in that cell (en <= L, so none past the stream's end)
        const uint32_t soff = uint32_t(p0 + d0) * RB;
        lds_dma16_s(krs, lk, voff_k, soff);
        lds_dma16_s(vrs, lv, voff_v, soff);
      } else {
        // lane-derived terms recomputed here rather than held across the loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int lrow = ln / CPR, lpc = ln % CPR;
        const int row = blk * RPI + lrow;                  // tile row of this lane
        int pos = t0 + row;
        pos = pos < L ? pos : L - 1;                       // tail rows: any valid row
        const int k = int(e[0] <= pos) + int(e[1] <= pos) + int(e[2] <= pos) + int(e[3] <= pos);
        int delta = k == 0 ? dl[0] : (k == 1 ? dl[1] : (k == 2 ? dl[2] : dl[3]));
        if (k == 4) {
          int c = tc + 4;
          while (pos >= sm.cpos[c + 1]) ++c;
          delta = sm.cstart[c];
        }
        const uint32_t roff = uint32_t(pos + delta) * RB;
        const int kc = lpc ^ (row & (CPR - 1));
        const int vc = lpc ^ swz_v<D>(row);
        lds_dma16(krs, lk, roff + kc * 16);
        lds_dma16(vrs, lv, roff + vc * 16);
      }
    }
    // cells that end at or before the next tile's first position
    const int t1 = t0 + KT;
    tc += int(e[0] <= t1) + int(e[1] <= t1) + int(e[2] <= t1) + int(e[3] <= t1);
    tc = __builtin_amdgcn_readfirstlane(min(tc, nc - 1));
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16_t{};
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  const float c2 = p.scale_log2;
  float mc_run = -__builtin_huge_valf();     // m_run * c2
  const f16x2_t ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};

  // transposed-read addressing (fixed per lane): group G, index i in group
  const int G = lane >> 4, gi = lane & 15, gg = G >> 1;
  // LDS -> MFMA software pipelines.  Fragments are read DEPTH MFMAs ahead
  // into a rotating buffer; scheduling fences keep the compiler from
  // regrouping the reads (it would otherwise wait on each read right before
  // its MFMA and expose the full LDS latency every time).
  // Fragment addresses are a per-lane base XOR a k-step term plus constant
  // offsets: with the swizzles above, chunk(s) = chunk(0) ^ 2s for K and
  // chunk(db) = chunk(0) ^ 4db for V.  The bases pass through an empty asm
  // statement per call so the compiler recomputes the XORs (one VALU op per
  // read) instead of hoisting a register per k-step out of the tile loop.
  // K fragment (A operand of S^T = K Q^T): key row kr0 + 32 j + n, dims 16 s + 8 g ..
  const int kbase0 = n * (CPR * 16) + ((g ^ (n & (CPR - 1))) * 16);
  // V^T fragment (A operand of O^T = V^T P^T), 16-key step u, d block db:
  // keys 16u + 4gg + gi/4 (first 4 slots) and +8 (last 4 slots)
  const int vrow0 = 4 * gg + (gi >> 2);
  const int vbase0 = vrow0 * (CPR * 16) +
                     ((2 * (G & 1) + ((gi & 3) >> 1)) ^ swz_v<D>(vrow0)) * 16 + (gi & 1) * 8;
  auto vfrag = [&](const uint4* vb, int vb0, int u, int db) __attribute__((always_inline)) {
    const char* b1 = reinterpret_cast<const char*>(vb) + ((vb0 ^ (64 * db)) + u * 16 * CPR * 16);
    const v4i16_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)b1);
    const v4i16_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(b1 + 8 * CPR * 16));
    return __builtin_bit_cast(
        f16x8_t, (short __attribute__((ext_vector_type(8)))){lo[0], lo[1], lo[2], lo[3], hi[0],
                                                              hi[1], hi[2], hi[3]});
  };
  // S^T for NB 32-key blocks (key rows kr0 + 32 j + n)
  auto qk_pipe = [&](const uint4* kb_, int kr0, auto nb_c, auto depth_c,
                     f32x16_t* sacc) __attribute__((always_inline)) {
    constexpr int NB = decltype(nb_c)::value, DEPTH = decltype(depth_c)::value;
    int kb0 = kbase0;
    asm volatile("" : "+v"(kb0));
    const char* kc = reinterpret_cast<const char*>(kb_) + kr0 * CPR * 16;
    auto kfrag = [&](int j, int s_) __attribute__((always_inline)) {
      return *reinterpret_cast<const bf16x8_t*>(kc + ((kb0 ^ (32 * s_)) + j * 32 * CPR * 16));
    };
    bf16x8_t buf[DEPTH][NB];
#pragma unroll
    for (int d0 = 0; d0 < DEPTH; ++d0)
#pragma unroll
      for (int j = 0; j < NB; ++j) buf[d0][j] = kfrag(j, d0);
#pragma unroll
    for (int s_ = 0; s_ < NS; ++s_) {
#pragma unroll
      for (int j = 0; j < NB; ++j)
        sacc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(buf[s_ % DEPTH][j], qf[s_], sacc[j], 0,
                                                          0, 0);
      if (s_ + DEPTH < NS) {
#pragma unroll
        for (int j = 0; j < NB; ++j) buf[s_ % DEPTH][j] = kfrag(j, s_ + DEPTH);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // O^T += V^T P^T over NU 16-key steps starting at u0 (P fragment pf[u - u0])
  auto pv_pipe = [&](const uint4* vb, int u0, auto nu_c, auto depth_c,
                     const f16x8_t* pf) __attribute__((always_inline)) {
    constexpr int NU = decltype(nu_c)::value, DEPTH = decltype(depth_c)::value;
    constexpr int NF = NU * NDB;
    int vb0 = vbase0;
    asm volatile("" : "+v"(vb0));
    f16x8_t buf[DEPTH];
#pragma unroll
    for (int f = 0; f < DEPTH; ++f) buf[f] = vfrag(vb, vb0, u0 + f / NDB, f % NDB);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      oacc[f % NDB] =
          __builtin_amdgcn_mfma_f32_32x32x16_f16(buf[f % DEPTH], pf[f / NDB], oacc[f % NDB], 0, 0, 0);
      if (f + DEPTH < NF) buf[f % DEPTH] = vfrag(vb, vb0, u0 + (f + DEPTH) / NDB, (f + DEPTH) % NDB);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // one 64-key sub-tile (rows 64 q ..) of the stage; the next tile's loads
  // are issued behind the QK^T MFMAs of sub-tile 0
  auto compute = [&](auto stage, int t, int q) __attribute__((always_inline)) {
    constexpr int B = decltype(stage)::value;
    const uint4* kb_ = (B == 0 ? k_s0 : k_s1) + 64 * q * CPR;
    const uint4* vb = (B == 0 ? v_s0 : v_s1) + 64 * q * CPR;
    // S^T = K Q^T for the two 32-key blocks, fragments read one step ahead
    f32x16_t sacc0 = f32x16_t{}, sacc1 = f32x16_t{};
    const int r_a = n, r_b = 32 + n;
    bf16x8_t a0 = __builtin_bit_cast(bf16x8_t, kb_[r_a * CPR + ((g) ^ (r_a & (CPR - 1)))]);
    bf16x8_t a1 = __builtin_bit_cast(bf16x8_t, kb_[r_b * CPR + ((g) ^ (r_b & (CPR - 1)))]);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      bf16x8_t n0 = a0, n1 = a1;
      if (s + 1 < NS) {
        n0 = __builtin_bit_cast(bf16x8_t, kb_[r_a * CPR + ((2 * s + 2 + g) ^ (r_a & (CPR - 1)))]);
        n1 = __builtin_bit_cast(bf16x8_t, kb_[r_b * CPR + ((2 * s + 2 + g) ^ (r_b & (CPR - 1)))]);
      }
      sacc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], sacc0, 0, 0, 0);
      sacc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], sacc1, 0, 0, 0);
      a0 = n0;
      a1 = n1;
    }
    // next tile's loads go out while the QK^T MFMAs drain
    if (q == 0 && t + 1 < ntiles) issue_tile(Stage<1 - B>{}, t + 1);
    const int tail = L - t * KT - 64 * q;   // valid keys in this sub-tile (may exceed 64)
    if (tail < 64) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int kk = 8 * (i >> 2) + 4 * g + (i & 3);
        if (kk >= tail) sacc0[i] = -__builtin_huge_valf();
        if (kk + 32 >= tail) sacc1[i] = -__builtin_huge_valf();
      }
    }
    // P against the reference max, and this lane's share of the row sum (of
    // the rounded P, the values the PV product uses)
    f16x8_t pf[4];
    float lsum;
    auto form_p = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        pf[i >> 3][i & 7] = static_cast<_Float16>(
            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc0[i], c2, -mc_run)));
        pf[2 + (i >> 3)][i & 7] = static_cast<_Float16>(
            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc1[i], c2, -mc_run)));
      }
      lsum = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int j = 0; j < 8; j += 2)
          lsum = __builtin_amdgcn_fdot2(f16x2_t{pf[u][j], pf[u][j + 1]}, ones, lsum, false);
    };
    form_p();
    // rescale (rare): the row's new reference is the larger of the old one and
    // the block's max over both lanes of the row; O and l follow, P is formed again
    if (__ballot(!(lsum <= kPSumCap))) {
      float mloc = -__builtin_huge_valf();
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, fmaxf(sacc0[i], sacc1[i]));
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      m_run = m_new;
      mc_run = m_run * c2;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      form_p();
    }
    l_run += lsum;
    // u outer, d blocks inner: NDB independent accumulation chains interleave
    const int vb0 = vbase0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vfrag(vb, vb0, u, db), pf[u], oacc[db], 0,
                                                          0, 0);
  };

  // Register-lean variant for large items: the 64-key tile is processed as
  // two 32-key halves (one score block, half the P fragments live at once).
  auto compute_half = [&](const uint4* kb_, const uint4* vb, int kbi, int tail) __attribute__((always_inline)) {
    f32x16_t sacc1[1] = {f32x16_t{}};
    qk_pipe(kb_, 32 * kbi, std::integral_constant<int, 1>{}, std::integral_constant<int, 4>{},
            sacc1);
    f32x16_t sacc = sacc1[0];
    if (tail < 32 * kbi + 32) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (32 * kbi + 8 * (i >> 2) + 4 * g + (i & 3) >= tail) sacc[i] = -__builtin_huge_valf();
    }
    f16x8_t pf[2];
    float lsum;
    auto form_p = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        pf[i >> 3][i & 7] = static_cast<_Float16>(
            __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[i], c2, -mc_run)));
      lsum = 0.f;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 8; j += 2)
          lsum = __builtin_amdgcn_fdot2(f16x2_t{pf[u][j], pf[u][j + 1]}, ones, lsum, false);
    };
    form_p();
    if (__ballot(!(lsum <= kPSumCap))) {
      float mloc = -__builtin_huge_valf();
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, sacc[i]);
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
      m_run = m_new;
      mc_run = m_run * c2;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      form_p();
    }
    l_run += lsum;
    pv_pipe(vb, 2 * kbi, std::integral_constant<int, 2>{}, std::integral_constant<int, 4>{}, pf);
  };
  auto compute_lean = [&](auto stage, int t) __attribute__((always_inline)) {
    constexpr int B = decltype(stage)::value;
    const uint4* kb_ = B == 0 ? k_s0 : k_s1;
    const uint4* vb = B == 0 ? v_s0 : v_s1;
    const int tail = L - t * KT;
    if (kmask & 1u) compute_half(kb_, vb, 0, tail);
    if (t + 1 < ntiles) issue_tile(Stage<1 - B>{}, t + 1);
#pragma unroll
    for (int hq = 1; hq < KT / 32; ++hq)
      if (((kmask >> hq) & 1u) && tail > 32 * hq) compute_half(kb_, vb, hq, tail);
  };

  // Two-stage pipeline with one barrier per tile: after the barrier of step
  // t every wave has finished tile t-1, so the stage it used is refilled with
  // tile t+1 (issued from inside compute, behind the QK^T MFMAs) while tile t
  // is computed.  Raw s_barrier: __syncthreads() would
  // also drain the loads in flight.
  auto step = [&](auto stage, int t) __attribute__((always_inline)) {
    constexpr int B = decltype(stage)::value;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (wave_active) {
      if constexpr (W >= 12) {
        compute_lean(stage, t);
      } else {
        compute(stage, t, 0);
        if constexpr (KT == 128) {
          if (L - t * KT > 64) compute(stage, t, 1);
        }
      }
    } else if (t + 1 < ntiles) {
      issue_tile(Stage<1 - B>{}, t + 1);
    }
  };
  if (ntiles > 0) issue_tile(Stage<0>{}, 0);
  for (int t = 0; t < ntiles; t += 2) {
    step(Stage<0>{}, t);
    if (t + 1 < ntiles) step(Stage<1>{}, t + 1);
  }

  if constexpr (W >= 12 && KT == 128) {
    if (nb == 9 || nb == 10) {
      // helpers park (O, m, l) in the free K/V stages, one slot each, value
      // j of lane l at j * 64 + l; the owner of the chunk folds them in
      constexpr int NV = NDB * 16 + 2;
      static_assert(NV * 64 * 4 <= KT / 8 * D * 16, "merge slot fits a stage");
      auto slot = [&](int i) -> float* {
        return reinterpret_cast<float*>(i == 0 ? k_s0 : (i == 1 ? k_s1 : v_s0));
      };
      __syncthreads();
      if (merge_slot >= 0) {
        float* sl = slot(merge_slot);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) sl[(db * 16 + r) * 64 + lane] = oacc[db][r];
        sl[(NDB * 16) * 64 + lane] = m_run;
        sl[(NDB * 16 + 1) * 64 + lane] = l_run;
      }
      __syncthreads();
      if (merge_slot >= 0) return;
      if (chunk == 8 || chunk == 9) {
        const int first = nb == 9 ? 0 : (chunk - 8);
        const int count = nb == 9 ? 3 : 1;
        for (int si = first; si < first + count; ++si) {
          const float* sl = slot(si);
          const float mh = sl[(NDB * 16) * 64 + lane], lh = sl[(NDB * 16 + 1) * 64 + lane];
          const float mn = fmaxf(m_run, mh);
          const float a0 = m_run == -__builtin_huge_valf()
                               ? 0.f
                               : __builtin_amdgcn_exp2f((m_run - mn) * c2);
          const float a1 =
              mh == -__builtin_huge_valf() ? 0.f : __builtin_amdgcn_exp2f((mh - mn) * c2);
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              oacc[db][r] = oacc[db][r] * a0 + sl[(db * 16 + r) * 64 + lane] * a1;
          l_run = l_run * a0 + lh * a1;
          m_run = mn;
        }
      }
    }
  }

  if constexpr (FUSED) {
    // the epilogue's MFMAs take operands from every lane: the whole wave runs
    // them (rows past the end with o = 0) and only valid rows store
    if (!wave_active) return;
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = row_valid ? __builtin_ldexpf(1.f, sv) / l_tot : 0.f;
    const int tok = row_valid ? p.perm_q[(long long)h * p.n_q + r0 + qloc] : 0;
    fused_epilogue_mfma<D>(p, corr_s, oacc, inv, lane, row_valid,
                           (long long)h * p.out_sh + (long long)tok * p.out_st);
    if (g == 0 && p.lse && row_valid)
      p.lse[(long long)h * p.n_q + r0 + qloc] = (m_run * c2 + __log2f(l_tot)) * kLn2;
    return;
  }
  if (!row_valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = __builtin_ldexpf(1.f, sv) / l_tot;
  {
    float* orow = p.o + ((long long)h * p.n_q + r0 + qloc) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        float4 v = make_float4(oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv,
                               oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * i4 + 4 * g) = v;
      }
  }
  if (g == 0 && p.lse)
    p.lse[(long long)h * p.n_q + r0 + qloc] = (m_run * c2 + __log2f(l_tot)) * kLn2;
}

// ---------------------------------------------------------------------------
// fp32 kernel on fp32 MFMA (v_mfma_f32_32x32x2_f32: exact products, fp32
// accumulation): 4 waves of 32 query rows, 32-key LDS tiles.
// S^T = K Q^T: A = K (lane l: key l % 32, dim 2 s + l / 32), B = Q^T (lane l:
// query l % 32, same dims), held in registers.  The result lane l holds
// query l % 32 and keys 8 (r / 4) + 4 (l / 32) + r % 4 (r < 16).  PV takes
// the keys in the order the lanes hold them: k-step u pairs key
// kap(u, h) = 8 (u / 4) + 4 h + u % 4 of lane half h, so the B operand of
// O^T = V^T P^T is register u of P as it stands and the A operand is
// V[kap(u, l / 32)][32 db + l % 32].  Softmax is an fp32 online softmax over
// exact fp32 P (no rounding of P before the product).
// ---------------------------------------------------------------------------
template <int D>
struct SmemF32 {
  float kv[2][32][D + 1];   // K tile, V tile (rows padded: K is read by key)
  int32_t cstart[SPARSEPR_MAX_GROUPS];
  int32_t cpos[SPARSEPR_MAX_GROUPS + 1];
  long long red[4];
};

typedef float f32x16v_t __attribute__((ext_vector_type(16)));

template <int D>
__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs p) {
  constexpr int NS = D / 2;     // k-steps of S^T
  constexpr int NDB = D / 32;   // 32-dim blocks of O^T
  constexpr int TQ = 128;       // query rows per item
  __shared__ SmemF32<D> sm;
  int h, a, kt;
  if (!locate_item(p, h, a, kt)) return;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, n = lane & 31, hf = lane >> 5;
  const int32_t* oq = p.off_q + (long long)h * (p.c_q + 1);
  const int r0 = oq[a] + kt * TQ;
  const int nrows = min(TQ, oq[a + 1] - r0);
  const int nc = p.rowptr[(long long)h * (p.c_q + 1) + a + 1] -
                 p.rowptr[(long long)h * (p.c_q + 1) + a];
  const int L = load_cells<256>(p, h, a, sm.cstart, sm.cpos, sm.red);
  const float* Kh = static_cast<const float*>(p.k) + (long long)h * p.n_k * D;
  const float* Vh = static_cast<const float*>(p.v) + (long long)h * p.n_k * D;
  const int qloc = wid * 32 + n;
  const bool wave_active = wid * 32 < nrows;
  const bool row_valid = qloc < nrows;
  // Q^T fragments: dims 2 s + hf of this lane's query
  float qf[NS];
  {
    const float* qrow = static_cast<const float*>(p.q) +
                        ((long long)h * p.n_q + r0 + (row_valid ? qloc : 0)) * D;
#pragma unroll
    for (int s = 0; s < NS; ++s) qf[s] = row_valid ? qrow[2 * s + hf] : 0.f;
  }
  f32x16v_t oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16v_t{};
  const float c2 = p.scale_log2;
  float m_run = -__builtin_huge_valf(), l_run = 0.f;
  // split blockIdx.y of p.splits takes a contiguous range of the item's tiles
  const int ntiles_all = (L + 31) / 32;
  const int per = (ntiles_all + p.splits - 1) / p.splits;
  const int t_lo = min(ntiles_all, int(blockIdx.y) * per);
  const int ntiles = min(ntiles_all, t_lo + per);
  for (int t = t_lo; t < ntiles; ++t) {
    __syncthreads();
    // 32 keys x D of K and of V: thread e moves one float4 of each
    for (int e = tid; e < 32 * (D / 4); e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      const int pos = t * 32 + r;
      float4 kv4 = make_float4(0, 0, 0, 0), vv4 = make_float4(0, 0, 0, 0);
      if (pos < L) {
        const int c = find_cell(sm.cpos, nc, pos);
        const long long row = sm.cstart[c] + (pos - sm.cpos[c]);
        kv4 = *reinterpret_cast<const float4*>(Kh + row * D + 4 * c4);
        vv4 = *reinterpret_cast<const float4*>(Vh + row * D + 4 * c4);
      }
      float* kd = &sm.kv[0][r][4 * c4];
      float* vd = &sm.kv[1][r][4 * c4];
      kd[0] = kv4.x; kd[1] = kv4.y; kd[2] = kv4.z; kd[3] = kv4.w;
      vd[0] = vv4.x; vd[1] = vv4.y; vd[2] = vv4.z; vd[3] = vv4.w;
    }
    __syncthreads();
    if (!wave_active) continue;
    // S^T for the 32 keys of the tile
    f32x16v_t sacc = f32x16v_t{};
#pragma unroll
    for (int s = 0; s < NS; ++s)
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(sm.kv[0][n][2 * s + hf], qf[s], sacc, 0, 0, 0);
    const int tail = L - t * 32;
    float mloc = -__builtin_huge_valf();
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * hf + (r & 3);
      if (key >= tail) sacc[r] = -__builtin_huge_valf();
      mloc = fmaxf(mloc, sacc[r]);
    }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * c2);
    m_run = m_new;
    const float mc = m_new * c2;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c2, -mc));
      lsum += sacc[r];
    }
    l_run = l_run * alpha + lsum;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
    // O^T += V^T P^T, keys in the lanes' own order
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int key = 8 * (u >> 2) + 4 * hf + (u & 3);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sm.kv[1][key][32 * db + n], sacc[u],
                                                        oacc[db], 0, 0, 0);
    }
  }
  if (!row_valid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const long long grow = (long long)h * p.n_q + r0 + qloc;
  if (p.splits > 1) {
    // unnormalised partial and its (max, sum); a split without keys leaves
    // (-inf, 0) and zeros
    const long long prow = (long long)blockIdx.y * p.H * p.n_q + grow;
    float* po = p.part_o + prow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4)
        *reinterpret_cast<float4*>(po + 32 * db + 8 * i4 + 4 * hf) =
            make_float4(oacc[db][4 * i4 + 0], oacc[db][4 * i4 + 1], oacc[db][4 * i4 + 2],
                        oacc[db][4 * i4 + 3]);
    if (hf == 0) {
      p.part_ml[2 * prow] = m_run == -__builtin_huge_valf() ? m_run : m_run * c2;
      p.part_ml[2 * prow + 1] = l_tot;
    }
    return;
  }
  const float inv = 1.f / l_tot;
  // O^T lane l: query l % 32, dims 32 db + 8 (r / 4) + 4 (l / 32) + r % 4
  float* orow = p.o + grow * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      float4 v = make_float4(oacc[db][4 * i4 + 0] * inv, oacc[db][4 * i4 + 1] * inv,
                             oacc[db][4 * i4 + 2] * inv, oacc[db][4 * i4 + 3] * inv);
      *reinterpret_cast<float4*>(orow + 32 * db + 8 * i4 + 4 * hf) = v;
    }
  if (hf == 0 && p.lse) p.lse[grow] = (m_run * c2 + __log2f(l_tot)) * kLn2;
}

// Split partials of the fp32 kernel combined per row: weights 2^(m_s - M)
// with M the largest partial maximum (log2 units), then O = sum w_s O_s /
// sum w_s l_s.  D / 4 threads per row, four dims each.
template <int D>
__global__ __launch_bounds__(256) void attn_split_merge_kernel(const float* __restrict__ part_o,
                                                               const float* __restrict__ part_ml,
                                                               int splits, long long rows,
                                                               float* __restrict__ o,
                                                               float* __restrict__ lse) {
  constexpr int TPR = D / 4;
  const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c4 = threadIdx.x % TPR;
  if (row >= rows) return;
  float M = -__builtin_huge_valf();
  for (int s = 0; s < splits; ++s) M = fmaxf(M, part_ml[2 * (s * rows + row)]);
  float l = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s = 0; s < splits; ++s) {
    const float ms = part_ml[2 * (s * rows + row)];
    if (ms == -__builtin_huge_valf()) continue;
    const float wgt = __builtin_amdgcn_exp2f(ms - M);
    l = fmaf(wgt, part_ml[2 * (s * rows + row) + 1], l);
    const float4 v = reinterpret_cast<const float4*>(part_o + (s * rows + row) * D)[c4];
    acc.x = fmaf(wgt, v.x, acc.x);
    acc.y = fmaf(wgt, v.y, acc.y);
    acc.z = fmaf(wgt, v.z, acc.z);
    acc.w = fmaf(wgt, v.w, acc.w);
  }
  const float inv = 1.f / l;
  reinterpret_cast<float4*>(o + row * D)[c4] =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (c4 == 0 && lse) lse[row] = (M + __log2f(l)) * kLn2;
}

// Waves (32 query rows each) per bf16 work item: 4 (two blocks per CU), 8 or
// 12 (one block per CU).  All waves of an item share every K/V tile it loads,
// so a larger item streams its group's K/V fewer times, but rows past the
// group's end leave wave slots idle.  With q = ceil(mean group size / 32)
// busy waves per group, the choice maximises q / (W * ceil(q / W)) and takes
// the largest W on ties.  A call whose items would then number fewer than
// the 256 compute units keeps W = 4: there the grid itself is short and more,
// smaller blocks balance better.
int bf16_waves(const sparsepr_dims* d) {
  const long long groups = (long long)d->heads * d->c_q;
  const int q = int((d->n_q + 32LL * d->c_q - 1) / (32LL * d->c_q));
  int best = 4;
  double best_eff = 0.0;
  for (int w : {4, 8, 12}) {
    const double eff = double(q) / (double(w) * double((q + w - 1) / w));
    if (eff >= best_eff - 1e-12) {
      best = w;
      best_eff = eff;
    }
  }
  if (groups * ((q + best - 1) / best) < 256) return 4;
  return best;
}

int rows_per_item(const sparsepr_dims* d) {
  if (d->dtype == SPARSEPR_BF16) return 32 * bf16_waves(d);
  return 128;   // fp32: 4 waves of 32 query rows
}

template <int D, bool FUSED = false>
void launch_bf16(const AttnArgs& a, int blocks, int waves, hipStream_t s) {
  switch (waves) {
    case 4: attn_bf16_kernel<D, 4, FUSED><<<blocks, 256, 0, s>>>(a); break;
    case 8: attn_bf16_kernel<D, 8, FUSED><<<blocks, 512, 0, s>>>(a); break;
    default: attn_bf16_kernel<D, 12, FUSED><<<blocks, 768, 0, s>>>(a); break;
  }
}

}  // namespace

// fp32 calls with few work items split every item's key stream over up to
// 8 blocks (partials merged afterwards), so the grid reaches about two
// blocks per compute unit.
int f32_splits(const sparsepr_dims* d) {
  if (d->dtype != SPARSEPR_F32) return 1;
  const long long items = (long long)d->heads * ((d->n_q + 127) / 128);
  long long s = 512 / (items > 0 ? items : 1);
  return int(s < 1 ? 1 : (s > 8 ? 8 : s));
}

// The fused call runs the correction in the attention epilogue for bf16
// inputs with rank <= kFusedRank; otherwise it computes O_sp into its
// workspace and runs the correction kernel.
bool fused_epilogue(const sparsepr_dims* d, int rank) {
  return d->dtype == SPARSEPR_BF16 && rank <= kFusedRank;
}

size_t attn_ws_bytes(const sparsepr_dims* d);

size_t attn_correct_ws_bytes(const sparsepr_dims* d, int rank) {
  size_t nb = (attn_ws_bytes(d) + 255) & ~size_t(255);
  if (!fused_epilogue(d, rank)) nb += size_t(d->heads) * d->n_q * d->head_dim * sizeof(float);
  return nb;
}

// work items of a launch: sum_a ceil(n_a / tq) <= N_q / tq + C_q per head
long long item_bound(const sparsepr_dims* d) {
  const int tq = rows_per_item(d);
  return (long long)d->heads * ((d->n_q + tq - 1) / tq + d->c_q);
}

size_t attn_ws_bytes(const sparsepr_dims* d) {
  Carver cv(nullptr);
  cv.take<int32_t>(size_t(d->heads) * d->c_q + 1);
  cv.take<int2>(size_t(item_bound(d)));
  const int sp = f32_splits(d);
  if (sp > 1) {
    cv.take<float>(size_t(sp) * d->heads * d->n_q * d->head_dim);
    cv.take<float>(size_t(sp) * d->heads * d->n_q * 2);
  }
  return cv.used;
}

}  // namespace spr

using namespace spr;

namespace {

int32_t check_attn_args(const sparsepr_dims* dims, const int32_t* offsets_q,
                        const int32_t* offsets_kv, const int32_t* cell_rowptr,
                        const int32_t* cell_col, const void* q_g, const void* k_g,
                        const void* v_g, const int32_t* v_shift, const float* o_sp) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!offsets_q || !offsets_kv || !cell_rowptr || !cell_col || !q_g || !k_g || !v_g ||
      !v_shift || !o_sp)
    return SPARSEPR_ERR_INVALID;
  return SPARSEPR_OK;
}

// The work-item table (H*C_q + 1 int32, rewritten in full by every call)
// and the attention launch, shared by both entry points.
int32_t launch_attn(const sparsepr_dims* dims, const int32_t* offsets_q,
                    const int32_t* offsets_kv, const int32_t* cell_rowptr,
                    const int32_t* cell_col, const void* q_g, const void* k_g, const void* v_g,
                    const int32_t* v_shift, float softmax_scale, float* o_sp, float* lse,
                    int32_t* tiles, int2* items, int splits, float* part_o, float* part_ml,
                    hipStream_t stream, const AttnArgs* fuse = nullptr) {
  const int tq = rows_per_item(dims);
  tile_table_kernel<<<1, 1024, 0, stream>>>(offsets_q, dims->heads, dims->c_q, tq, tiles);
  SPR_LAUNCH_CHECK();
  // With many items per compute unit (8 or more on average, by the bound) the
  // list is ordered per head (L2 reuse within a head); with fewer, all heads
  // are ordered together in one block when their groups fit its sort, and the
  // items otherwise go in their natural order.
  if (items) {
    const bool many = item_bound(dims) >= 8LL * 256;
    if (many) {
      const unsigned nblk = unsigned(dims->heads >= 2 ? dims->heads - 1 : 1);
      item_order_kernel<<<nblk, 1024, 0, stream>>>(offsets_q, offsets_kv, cell_rowptr, cell_col,
                                                   dims->heads, dims->c_q, dims->c_k, tq, tiles,
                                                   items, 0);
    } else if ((long long)dims->heads * dims->c_q <= kOrderMax) {
      item_order_kernel<<<1, 1024, 0, stream>>>(offsets_q, offsets_kv, cell_rowptr, cell_col,
                                                dims->heads, dims->c_q, dims->c_k, tq, tiles,
                                                items, 1);
    } else {
      items = nullptr;
    }
    if (items) SPR_LAUNCH_CHECK();
  }
  long long bound = item_bound(dims);
  bound = (bound + 8 * kXcdRun - 1) / (8 * kXcdRun) * (8 * kXcdRun);
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
  a.items = items;
  a.v_shift = v_shift;
  a.H = dims->heads;
  a.n_q = dims->n_q;
  a.n_k = dims->n_k;
  a.c_q = dims->c_q;
  a.c_k = dims->c_k;
  a.scale_log2 = softmax_scale * kLog2e;
  a.grid_blocks = int(bound);
  a.splits = splits;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.perm_q = nullptr;
  a.corr_a = a.corr_psi_t = a.corr_c = a.corr_g = nullptr;
  a.out = nullptr;
  a.out_sh = a.out_st = 0;
  a.out_bf16 = a.rank = 0;
  if (fuse) {
    a.perm_q = fuse->perm_q;
    a.corr_a = fuse->corr_a;
    a.corr_psi_t = fuse->corr_psi_t;
    a.corr_c = fuse->corr_c;
    a.corr_g = fuse->corr_g;
    a.out = fuse->out;
    a.out_sh = fuse->out_sh;
    a.out_st = fuse->out_st;
    a.out_bf16 = fuse->out_bf16;
    a.rank = fuse->rank;
  }
  if (dims->dtype == SPARSEPR_BF16) {
    const int w = bf16_waves(dims);
    if (fuse) {
      if (dims->head_dim == 128) launch_bf16<128, true>(a, int(bound), w, stream);
      else launch_bf16<64, true>(a, int(bound), w, stream);
    } else {
      if (dims->head_dim == 128) launch_bf16<128>(a, int(bound), w, stream);
      else launch_bf16<64>(a, int(bound), w, stream);
    }
  } else {
    const dim3 grid{unsigned(bound), unsigned(splits), 1u};
    if (dims->head_dim == 128) attn_f32_kernel<128><<<grid, 256, 0, stream>>>(a);
    else attn_f32_kernel<64><<<grid, 256, 0, stream>>>(a);
    SPR_LAUNCH_CHECK();
    if (splits > 1) {
      const long long rows = (long long)dims->heads * dims->n_q;
      const int rpb = 256 / (dims->head_dim / 4);
      const unsigned mb = unsigned((rows + rpb - 1) / rpb);
      if (dims->head_dim == 128)
        attn_split_merge_kernel<128><<<mb, 256, 0, stream>>>(part_o, part_ml, splits, rows, o_sp,
                                                             lse);
      else
        attn_split_merge_kernel<64><<<mb, 256, 0, stream>>>(part_o, part_ml, splits, rows, o_sp,
                                                            lse);
    }
  }
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}

// Scratch of the entry point that allocates nothing: the work-item table in
// a fixed device array.  In host code `scratch` names a host-side stand-in;
// its device address on each GPU comes from hipGetSymbolAddress, taken once
// per device with that device current, and only that address is passed on.
constexpr int kNoAllocTableEntries = 65537;   // H * C_q + 1 <= 65537 (256 KiB)
static __device__ __align__(256) int32_t scratch[kNoAllocTableEntries];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {};

int32_t* scratch_on_current_device(int32_t* status) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *status = SPARSEPR_ERR_HIP;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      *status = SPARSEPR_ERR_HIP;
      return nullptr;
    }
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *status = SPARSEPR_OK;
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int32_t sparsepr_sparse_attn(const sparsepr_dims* dims, const int32_t* offsets_q,
                                        const int32_t* offsets_kv, const int32_t* cell_rowptr,
                                        const int32_t* cell_col, const void* q_g, const void* k_g,
                                        const void* v_g, const int32_t* v_shift,
                                        float softmax_scale, float* o_sp,
                                        float* lse, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  int32_t st = check_attn_args(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g,
                               v_shift, o_sp);
  if (st != SPARSEPR_OK) return st;
  const size_t need = attn_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  Carver cv(ws);
  int32_t* tiles = cv.take<int32_t>(size_t(dims->heads) * dims->c_q + 1);
  int2* items = cv.take<int2>(size_t(item_bound(dims)));
  const int sp = f32_splits(dims);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (sp > 1) {
    part_o = cv.take<float>(size_t(sp) * dims->heads * dims->n_q * dims->head_dim);
    part_ml = cv.take<float>(size_t(sp) * dims->heads * dims->n_q * 2);
  }
  return launch_attn(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g, v_shift,
                     softmax_scale, o_sp, lse, tiles, items, sp, part_o, part_ml, stream);
}

extern "C" int32_t sparsepr_sparse_attn_noalloc(const sparsepr_dims* dims,
                                                const int32_t* offsets_q,
                                                const int32_t* offsets_kv,
                                                const int32_t* cell_rowptr,
                                                const int32_t* cell_col, const void* q_g,
                                                const void* k_g, const void* v_g,
                                                const int32_t* v_shift, float softmax_scale,
                                                float* o_sp, float* lse, hipStream_t stream) {
  int32_t st = check_attn_args(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g,
                               v_shift, o_sp);
  if (st != SPARSEPR_OK) return st;
  if (int64_t(dims->heads) * dims->c_q + 1 > kNoAllocTableEntries) return SPARSEPR_ERR_UNSUPPORTED;
  int32_t* tiles = scratch_on_current_device(&st);
  if (st != SPARSEPR_OK) return st;
  // no partial buffers: fp32 calls run unsplit here
  return launch_attn(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g, v_shift,
                     softmax_scale, o_sp, lse, tiles, nullptr, 1, nullptr, nullptr, stream);
}

extern "C" int32_t sparsepr_sparse_attn_correct(
    const sparsepr_dims* dims, int32_t m, int32_t rank, const int32_t* offsets_q,
    const int32_t* offsets_kv, const int32_t* cell_rowptr, const int32_t* cell_col,
    const void* q_g, const void* k_g, const void* v_g, const int32_t* v_shift,
    float softmax_scale, const int32_t* perm_q, const int32_t* probe_tokens,
    const float* o_probe_dense, const float* corr_a, const float* corr_psi_t,
    const float* corr_c, const float* corr_g, void* out, int32_t out_dtype,
    int64_t out_stride_head, int64_t out_stride_tok, float* lse, void* ws, size_t ws_bytes,
    hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!offsets_q || !offsets_kv || !cell_rowptr || !cell_col || !q_g || !k_g || !v_g ||
      !v_shift || !perm_q || !probe_tokens || !o_probe_dense || !corr_a || !corr_psi_t ||
      !corr_c || !out)
    return SPARSEPR_ERR_INVALID;
  if (m < 1 || m > SPARSEPR_MAX_PROBES || rank < 0 || rank > SPARSEPR_MAX_RANK)
    return SPARSEPR_ERR_INVALID;
  if (out_dtype != SPARSEPR_BF16 && out_dtype != SPARSEPR_F32) return SPARSEPR_ERR_UNSUPPORTED;
  if (check_out_strides(dims, out_dtype, out_stride_head, out_stride_tok) != SPARSEPR_OK)
    return SPARSEPR_ERR_INVALID;
  if (!ws || ws_bytes < attn_correct_ws_bytes(dims, rank)) return SPARSEPR_ERR_WORKSPACE;
  Carver cv(ws);
  int32_t* tiles = cv.take<int32_t>(size_t(dims->heads) * dims->c_q + 1);
  int2* items = cv.take<int2>(size_t(item_bound(dims)));
  const int sp = f32_splits(dims);
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (sp > 1) {
    part_o = cv.take<float>(size_t(sp) * dims->heads * dims->n_q * dims->head_dim);
    part_ml = cv.take<float>(size_t(sp) * dims->heads * dims->n_q * 2);
  }
  if (fused_epilogue(dims, rank)) {
    AttnArgs fz;
    fz.perm_q = perm_q;
    fz.corr_a = corr_a;
    fz.corr_psi_t = corr_psi_t;
    fz.corr_c = corr_c;
    fz.corr_g = corr_g;
    fz.out = out;
    fz.out_sh = out_stride_head;
    fz.out_st = out_stride_tok;
    fz.out_bf16 = out_dtype == SPARSEPR_BF16;
    fz.rank = rank;
    st = launch_attn(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g, v_shift,
                     softmax_scale, nullptr, lse, tiles, items, sp, part_o, part_ml, stream,
                     &fz);
    if (st != SPARSEPR_OK) return st;
    return launch_probe_overwrite(dims, m, probe_tokens, o_probe_dense, out,
                                  out_dtype == SPARSEPR_BF16, out_stride_head, out_stride_tok,
                                  stream);
  }
  // correction as its own kernel, O_sp in the workspace
  size_t off = (attn_ws_bytes(dims) + 255) & ~size_t(255);
  float* o_sp = reinterpret_cast<float*>(static_cast<char*>(ws) + off);
  st = launch_attn(dims, offsets_q, offsets_kv, cell_rowptr, cell_col, q_g, k_g, v_g, v_shift,
                   softmax_scale, o_sp, lse, tiles, items, sp, part_o, part_ml, stream);
  if (st != SPARSEPR_OK) return st;
  return sparsepr_correct_ex(dims, m, rank, perm_q, o_sp, probe_tokens, o_probe_dense, corr_a,
                             corr_psi_t, corr_c, corr_g, out, out_dtype, out_stride_head,
                             out_stride_tok, nullptr, 0, stream);
}
