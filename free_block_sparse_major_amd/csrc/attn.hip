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
  const int32_t* v_shift;  // [H] v_g holds fp16(v * 2^-v_shift) (bf16 path)
  int H, n_q, n_k, c_q, c_k;
  float scale_log2;      // softmax_scale * log2(e)
  int grid_blocks;       // launched blocks (multiple of 8)
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

// Maps a launched block to (h, a, tile-in-group).  Blocks are dealt to the 8
// XCDs round-robin by id.  The remap hands each XCD runs of kXcdRun
// consecutive work items (tiles of one query group, same K/V stream, share
// that XCD's L2) while the 8 XCDs interleave run by run, so the blocks in
// flight across the GPU cover about one head: its K/V (tens of MB) stays in
// the last-level cache instead of eight heads competing for it.
constexpr int kXcdRun = 8;
SPR_DEV bool locate_item(const AttnArgs& p, int& h, int& a, int& kt) {
  const int bid = blockIdx.x;
  const int x = bid & 7, j = bid >> 3;
  const int lid = (j / kXcdRun) * (8 * kXcdRun) + x * kXcdRun + (j % kXcdRun);
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

typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

template <int D>
SPR_DEV int swz_v(int row) {
  return D == 128 ? 4 * (row & 3) : 4 * ((row >> 1) & 1);
}

typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));


// Lazy rescale: P is formed against the running reference max and the row is
// rescaled to a new reference only when a lane's sum of its P values in the
// block exceeds this cap (every P above it, and any overflow to inf, implies
// that).  P therefore stays at or below 2^8, well inside fp16.
constexpr float kPSumCap = 256.f;

template <int D, int W>
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

  int h, a, kt;
  if (!locate_item(p, h, a, kt)) return;
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
      const int k0 = int(e[0] <= p0) + int(e[1] <= p0) + int(e[2] <= p0) + int(e[3] <= p0);
      const int en = k0 == 0 ? e[0] : (k0 == 1 ? e[1] : (k0 == 2 ? e[2] : e[3]));
      if (p0 + RPI <= en) {
        // all rows in cell tc + k0 (en <= L, so none past the stream's end)
        const int d0 = k0 == 0 ? dl[0] : (k0 == 1 ? dl[1] : (k0 == 2 ? dl[2] : dl[3]));
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
  if (g == 0 && p.lse)
    p.lse[(long long)h * p.n_q + r0 + qloc] = (m_run * c2 + __log2f(l_tot)) * kLn2;
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
  const int L = load_cells<256>(p, h, a, sm.cstart, sm.cpos, sm.red);
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

// Waves (32 query rows each) per bf16 work item: 4 (two blocks per CU), 8 or
// 12 (one block per CU).  All waves of an item share every K/V tile it loads,
// so a larger item streams its group's K/V fewer times, but rows past the
// group's end leave wave slots idle.  With q = ceil(mean group size / 32)
// busy waves per group, the choice maximises q / (W * ceil(q / W)) and takes
// the largest W on ties.  Calls with few groups per CU keep W = 4: there the
// grid itself is short and more, smaller blocks balance better.
int bf16_waves(const sparsepr_dims* d) {
  const long long groups = (long long)d->heads * d->c_q;
  if (groups < 4LL * 256) return 4;
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
  return best;
}

int rows_per_item(const sparsepr_dims* d) {
  if (d->dtype == SPARSEPR_BF16) return 32 * bf16_waves(d);
  return 256 / (d->head_dim / 32);
}

template <int D>
void launch_bf16(const AttnArgs& a, int blocks, int waves, hipStream_t s) {
  switch (waves) {
    case 4: attn_bf16_kernel<D, 4><<<blocks, 256, 0, s>>>(a); break;
    case 8: attn_bf16_kernel<D, 8><<<blocks, 512, 0, s>>>(a); break;
    default: attn_bf16_kernel<D, 12><<<blocks, 768, 0, s>>>(a); break;
  }
}

}  // namespace

size_t attn_ws_bytes(const sparsepr_dims* d) {
  Carver cv(nullptr);
  cv.take<int32_t>(size_t(d->heads) * d->c_q + 1);
  return cv.used;
}

}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_sparse_attn(const sparsepr_dims* dims, const int32_t* offsets_q,
                                        const int32_t* offsets_kv, const int32_t* cell_rowptr,
                                        const int32_t* cell_col, const void* q_g, const void* k_g,
                                        const void* v_g, const int32_t* v_shift,
                                        float softmax_scale, float* o_sp,
                                        float* lse, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!offsets_q || !offsets_kv || !cell_rowptr || !cell_col || !q_g || !k_g || !v_g ||
      !v_shift || !o_sp)
    return SPARSEPR_ERR_INVALID;
  const size_t need = attn_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  Carver cv(ws);
  int32_t* tiles = cv.take<int32_t>(size_t(dims->heads) * dims->c_q + 1);
  const int tq = rows_per_item(dims);
  tile_table_kernel<<<1, 1024, 0, stream>>>(offsets_q, dims->heads, dims->c_q, tq, tiles);
  SPR_LAUNCH_CHECK();
  // upper bound of work items: sum_a ceil(n_a / tq) <= N_q / tq + C_q per head
  long long bound = (long long)dims->heads * ((dims->n_q + tq - 1) / tq + dims->c_q);
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
  a.v_shift = v_shift;
  a.H = dims->heads;
  a.n_q = dims->n_q;
  a.n_k = dims->n_k;
  a.c_q = dims->c_q;
  a.c_k = dims->c_k;
  a.scale_log2 = softmax_scale * kLog2e;
  a.grid_blocks = int(bound);
  if (dims->dtype == SPARSEPR_BF16) {
    const int w = bf16_waves(dims);
    if (dims->head_dim == 128) launch_bf16<128>(a, int(bound), w, stream);
    else launch_bf16<64>(a, int(bound), w, stream);
  } else {
    if (dims->head_dim == 128) attn_f32_kernel<128><<<int(bound), 256, 0, stream>>>(a);
    else attn_f32_kernel<64><<<int(bound), 256, 0, stream>>>(a);
  }
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}
