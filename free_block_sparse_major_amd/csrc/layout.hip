// S1-S3: group-major layout of Q, K, V.
//
// SparsePR paper, §3 problem setup: queries and keys are partitioned into
// groups, each value follows its key.  The review of the paper (method
// summary, step (3)) permutes Q, K, V to a group-major layout before the
// variable-length block-sparse kernel.  Inside a group tokens keep their
// ascending token order, so the layout is a stable counting sort of the labels.
//
// Kernels (per tensor kind, per head):
//   hist     per 1024-token tile: label histogram            -> counts[tile][c]
//   scan     exclusive scan of counts in (label, tile) order  -> bases, offsets
//   scatter  per tile: bitonic sort of (label, index), rank   -> perm
//   gather   row copy q_g[j] = q[perm[j]] with 16-byte accesses (HBM bound)
//   centroid fp64 sum of each group's rows / group size

#include "common.h"

namespace spr {
namespace {

constexpr int kTile = 1024;       // tokens per histogram / scatter tile
constexpr int kThreads = 256;

struct KindArgs {
  const int32_t* labels;  // [H][N]
  int32_t* perm;          // [H][N]
  int32_t* offsets;       // [H][C+1]
  int32_t* counts;        // [H][ntiles][C] (workspace)
  int n, c, ntiles;
};

// Labels outside [0, C) are a caller error (sparsepr_debug_check reports
// them); they are sorted as the nearest valid group, so perm stays a
// permutation and every later kernel indexes in bounds.
SPR_DEV int clamp_label(int l, int c) { return l < 0 ? 0 : (l >= c ? c - 1 : l); }

__global__ __launch_bounds__(kThreads) void hist_kernel(KindArgs qa, KindArgs ka, uint32_t* vmax,
                                                       int heads) {
  const KindArgs& A = blockIdx.z == 0 ? qa : ka;
  const int tile = blockIdx.x, h = blockIdx.y;
  if (vmax && tile == 0 && h == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < heads; i += kThreads) vmax[i] = 0u;
  if (tile >= A.ntiles) return;
  __shared__ int32_t hist[SPARSEPR_MAX_GROUPS];
  for (int i = threadIdx.x; i < A.c; i += kThreads) hist[i] = 0;
  __syncthreads();
  const int32_t* lab = A.labels + int64_t(h) * A.n;
  const int t0 = tile * kTile;
  for (int i = threadIdx.x; i < kTile; i += kThreads) {
    int t = t0 + i;
    if (t < A.n) atomicAdd(&hist[clamp_label(lab[t], A.c)], 1);
  }
  __syncthreads();
  int32_t* cnt = A.counts + int64_t(h) * A.c * A.ntiles;
  for (int c = threadIdx.x; c < A.c; c += kThreads) cnt[int64_t(tile) * A.c + c] = hist[c];
}

// One block per (head, kind): exclusive scan of counts[tile][c] in (c, tile)
// order, in place.  Thread c sums its label over the tiles (each tile's row
// of counts is read by consecutive threads), a block scan over the labels
// gives each label's base, and thread c walks its tiles again writing the
// running bases.  offsets[c] = base of (c, tile 0), offsets[C] = N.
__global__ __launch_bounds__(1024) void scan_kernel(KindArgs qa, KindArgs ka) {
  const KindArgs& A = blockIdx.y == 0 ? qa : ka;
  const int h = blockIdx.x;
  __shared__ long long red[1024 / 64];
  int32_t* cnt = A.counts + int64_t(h) * A.c * A.ntiles;
  const int c = threadIdx.x;   // C <= SPARSEPR_MAX_GROUPS = 1024 = blockDim.x
  constexpr int U = 8;         // tiles loaded before their counts are used
  long long tot = 0;
  if (c < A.c) {
    for (int t0 = 0; t0 < A.ntiles; t0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = t0 + u < A.ntiles ? cnt[int64_t(t0 + u) * A.c + c] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u) tot += v[u];
    }
  }
  long long all;
  const long long base = block_exclusive_scan(tot, red, &all);
  if (c < A.c) {
    long long run = base;
    for (int t0 = 0; t0 < A.ntiles; t0 += U) {
      int v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = t0 + u < A.ntiles ? cnt[int64_t(t0 + u) * A.c + c] : 0;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (t0 + u < A.ntiles) {
          cnt[int64_t(t0 + u) * A.c + c] = int32_t(run);
          run += v[u];
        }
    }
    A.offsets[int64_t(h) * (A.c + 1) + c] = int32_t(base);
  }
  if (threadIdx.x == 0) A.offsets[int64_t(h) * (A.c + 1) + A.c] = A.n;
}

// Per tile: the stable rank of every token among the tile's earlier tokens of
// its label, added to the scanned base of (label, tile).  The tile's 1024
// tokens are 16 rows of 64 in token order and wave w takes rows 4w .. 4w+3.
// Within a row the lanes holding the same label are found with one ballot per
// label bit (multi-split), and a lane's rank in the row is the number of them
// below it; earlier rows of the wave count through the wave's running label
// histogram, earlier waves through a prefix of the waves' histograms.
__global__ __launch_bounds__(kThreads) void scatter_kernel(KindArgs qa, KindArgs ka) {
  const KindArgs& A = blockIdx.z == 0 ? qa : ka;
  const int tile = blockIdx.x, h = blockIdx.y;
  if (tile >= A.ntiles) return;
  constexpr int NW = kThreads / 64;           // waves
  constexpr int RPW = kTile / 64 / NW;        // rows of 64 tokens per wave
  static_assert(RPW * 64 * NW == kTile, "rows cover the tile");
  __shared__ int32_t whist[NW][SPARSEPR_MAX_GROUPS];
  const int wid = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int32_t* lab = A.labels + int64_t(h) * A.n;
  const int t0 = tile * kTile;
  for (int i = threadIdx.x; i < NW * A.c; i += kThreads) whist[i / A.c][i % A.c] = 0;
  int l[RPW];
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int t = t0 + (wid * RPW + r) * 64 + lane;
    l[r] = t < A.n ? clamp_label(lab[t], A.c) : -1;
  }
  __syncthreads();
#pragma unroll
  for (int r = 0; r < RPW; ++r)
    if (l[r] >= 0) atomicAdd(&whist[wid][l[r]], 1);
  __syncthreads();
  // per label, exclusive prefix over the waves (in place)
  for (int c = threadIdx.x; c < A.c; c += kThreads) {
    int run = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int v = whist[w][c];
      whist[w][c] = run;
      run += v;
    }
  }
  __syncthreads();
  const int nbits = A.c > 1 ? 32 - __clz(A.c - 1) : 0;   // label bits
  const uint64_t below = (1ull << lane) - 1ull;
  const int32_t* cnt = A.counts + int64_t(h) * A.c * A.ntiles;
  int32_t* perm = A.perm + int64_t(h) * A.n;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int lr = l[r];
    const bool valid = lr >= 0;
    uint64_t same = __ballot(valid);
    for (int bt = 0; bt < nbits; ++bt) {
      const bool bit = (lr >> bt) & 1;
      const uint64_t ones = __ballot(valid && bit);
      same &= bit ? ones : ~ones;
    }
    if (valid) {
      const int rank = whist[wid][lr] + __popcll(same & below);
      perm[cnt[int64_t(tile) * A.c + lr] + rank] = t0 + (wid * RPW + r) * 64 + lane;
      // the highest lane of each label adds the row's count (one writer per
      // label, after every lane of the row has read the running count)
      if ((same >> lane) == 1ull) whist[wid][lr] += __popcll(same);
    }
  }
}

// Row gather with 16-byte accesses.  grid.z: 0 = q, 1 = k, 2 = v.
struct GatherArgs {
  const char* src[3];
  char* dst[3];
  const int32_t* perm[3];
  int64_t stride_head[3], stride_tok[3];  // elements
  int n[3];
  int row_bytes;   // d * element size (multiple of 16)
  int esize;
  const uint32_t* vmax;  // bf16 inputs: per-head largest |v| bit pattern (else null)
  int32_t* v_shift;      // [H] output: v_g = fp16(v * 2^-v_shift)
};

// Exponent shift that puts a head's largest |v| in [2^14, 2^15): every bf16
// value down to 2^-28 of that maximum converts to fp16 without rounding.
SPR_DEV int v_shift_of(uint32_t vmax_bits) {
  const int E = int((vmax_bits >> 7) & 0xffu);
  int s = (E == 0 ? -127 : E - 127) - 14;
  return s < -100 ? -100 : (s > 100 ? 100 : s);
}

// Largest |v| of every head of the caller's bf16 values (sign cleared; positive
// bf16 bit patterns order like their values).  vmax must be zero on entry.
constexpr int kVmaxRows = 1024;
__global__ __launch_bounds__(kThreads) void vmax_kernel(const uint16_t* __restrict__ v, int n,
                                                       int d, int64_t stride_head,
                                                       int64_t stride_tok,
                                                       uint32_t* __restrict__ vmax) {
  const int h = blockIdx.y;
  const int r0 = blockIdx.x * kVmaxRows;
  if (r0 >= n) return;
  const int rows = min(kVmaxRows, n - r0);
  const int chunks = d / 8;
  __shared__ uint32_t red[kThreads / 64];
  uint32_t mx = 0;
  // eight 16-byte loads in flight per thread before their values are used
  constexpr int U = 8;
  const int total = rows * chunks;
  for (int i0 = threadIdx.x; i0 < total; i0 += U * kThreads) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + u * kThreads;
      const int r = i / chunks, c = i - r * chunks;
      w[u] = i < total ? *reinterpret_cast<const uint4*>(v + h * stride_head +
                                                         (r0 + r) * stride_tok + c * 8)
                       : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t ws[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) mx = max(mx, max(ws[j] & 0x7fffu, (ws[j] >> 16) & 0x7fffu));
    }
  }
  mx = block_max(mx, red);
  if (threadIdx.x == 0) atomicMax(&vmax[h], mx);
}

// fp64 sums of one 16-byte chunk of a row (8 bf16 or 4 fp32 values)
template <typename T>
SPR_DEV void add_chunk(double* acc, const uint4& w);
template <>
SPR_DEV void add_chunk<uint16_t>(double* acc, const uint4& w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc[2 * j] += double(__uint_as_float(ws[j] << 16));
    acc[2 * j + 1] += double(__uint_as_float(ws[j] & 0xffff0000u));
  }
}
template <>
SPR_DEV void add_chunk<float>(double* acc, const uint4& w) {
  acc[0] += double(__uint_as_float(w.x));
  acc[1] += double(__uint_as_float(w.y));
  acc[2] += double(__uint_as_float(w.z));
  acc[3] += double(__uint_as_float(w.w));
}

// Gather fused with the fp64 centroids, one block per group: kind 0 copies
// the query rows of group a (q -> q_g) and kind 1 the key and value rows of
// K/V group a (k -> k_g, v -> v_g in fp16 after the head's shift).  The rows
// of a group are the group-major rows off[a] .. off[a + 1]; thread (ch, ph)
// copies chunk ch of rows off[a] + ph + i * phases and adds them in that
// order, and the phase partials are combined in a fixed order, so every
// centroid is the same sum as a separate pass over the gathered rows.
template <typename T>
__global__ __launch_bounds__(kThreads) void gather_group_kernel(GatherArgs g,
                                                                const int32_t* __restrict__ off_q,
                                                                const int32_t* __restrict__ off_k,
                                                                double* __restrict__ cen_q,
                                                                double* __restrict__ cen_k,
                                                                int c_q, int c_k, int d) {
  constexpr int EPC = 16 / sizeof(T);
  const int kind = blockIdx.z, h = blockIdx.y, a = blockIdx.x;
  const int C = kind == 0 ? c_q : c_k;
  if (a >= C) return;
  const int n = g.n[kind];
  const int32_t* off = (kind == 0 ? off_q : off_k) + int64_t(h) * (C + 1);
  double* cen = (kind == 0 ? cen_q : cen_k) + (int64_t(h) * C + a) * d;
  const int32_t* perm = g.perm[kind] + int64_t(h) * n;
  const char* src = g.src[kind] + int64_t(h) * g.stride_head[kind] * g.esize;
  char* dst = g.dst[kind] + int64_t(h) * n * g.row_bytes;
  const int64_t st = g.stride_tok[kind] * g.esize;
  const bool with_v = kind == 1;
  const char* vsrc = g.src[2] + int64_t(h) * g.stride_head[2] * g.esize;
  char* vdst = g.dst[2] + int64_t(h) * n * g.row_bytes;
  const int64_t vst = g.stride_tok[2] * g.esize;
  const bool conv = g.vmax != nullptr;
  float sc = 1.f;
  if (with_v) {
    const int sh = conv ? v_shift_of(g.vmax[h]) : 0;
    sc = __builtin_ldexpf(1.f, -sh);
    if (a == 0 && threadIdx.x == 0 && g.v_shift) g.v_shift[h] = sh;
  }
  __shared__ double part[kThreads * 8];
  const int cpr = d / EPC;
  const int phases = kThreads / cpr;
  const int ch = threadIdx.x % cpr, ph = threadIdx.x / cpr;
  const int lo = off[a], hi = off[a + 1];
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  auto put_v = [&](int row, uint4 w) __attribute__((always_inline)) {
    if (conv) {
      uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const _Float16 l16 = static_cast<_Float16>(__uint_as_float(ws[j] << 16) * sc);
        const _Float16 h16 = static_cast<_Float16>(__uint_as_float(ws[j] & 0xffff0000u) * sc);
        ws[j] = uint32_t(__builtin_bit_cast(uint16_t, l16)) |
                (uint32_t(__builtin_bit_cast(uint16_t, h16)) << 16);
      }
      w = make_uint4(ws[0], ws[1], ws[2], ws[3]);
    }
    *reinterpret_cast<uint4*>(vdst + int64_t(row) * g.row_bytes + ch * 16) = w;
  };
  int r = lo + ph;
  for (; r + 3 * phases < hi; r += 4 * phases) {
    uint4 w[4], wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tok = perm[r + u * phases];
      w[u] = *reinterpret_cast<const uint4*>(src + tok * st + ch * 16);
      if (with_v) wv[u] = *reinterpret_cast<const uint4*>(vsrc + tok * vst + ch * 16);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *reinterpret_cast<uint4*>(dst + int64_t(r + u * phases) * g.row_bytes + ch * 16) = w[u];
      add_chunk<T>(acc, w[u]);
      if (with_v) put_v(r + u * phases, wv[u]);
    }
  }
  for (; r < hi; r += phases) {
    const int tok = perm[r];
    const uint4 w = *reinterpret_cast<const uint4*>(src + tok * st + ch * 16);
    *reinterpret_cast<uint4*>(dst + int64_t(r) * g.row_bytes + ch * 16) = w;
    add_chunk<T>(acc, w);
    if (with_v) put_v(r, *reinterpret_cast<const uint4*>(vsrc + tok * vst + ch * 16));
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[threadIdx.x * 8 + e] = acc[e];
  __syncthreads();
  for (int j = threadIdx.x; j < d; j += kThreads) {
    const int c = j / EPC, e = j % EPC;
    double t = 0.0;
    for (int p2 = 0; p2 < phases; ++p2) t += part[(p2 * cpr + c) * 8 + e];
    cen[j] = hi > lo ? t / double(hi - lo) : 0.0;
  }
}

}  // namespace

size_t layout_ws_bytes(const sparsepr_dims* d) {
  Carver cv(nullptr);
  int tq = (d->n_q + kTile - 1) / kTile, tk = (d->n_k + kTile - 1) / kTile;
  cv.take<int32_t>(size_t(d->heads) * d->c_q * tq);
  cv.take<int32_t>(size_t(d->heads) * d->c_k * tk);
  cv.take<uint32_t>(size_t(d->heads));
  return cv.used;
}

// Stable counting sort of labels[H][n] in [0, c) (the layout's own sort):
// perm[h][j] = token of group-major row j, offsets[h][c+1].  ws holds the
// per-tile counts.
size_t group_sort_ws_bytes(int heads, int n, int c) {
  const int ntiles = (n + kTile - 1) / kTile;
  return (size_t(heads) * c * ntiles * sizeof(int32_t) + 255) & ~size_t(255);
}

int32_t group_sort(const int32_t* labels, int heads, int n, int c, int32_t* perm,
                   int32_t* offsets, void* ws, hipStream_t stream) {
  const int ntiles = (n + kTile - 1) / kTile;
  KindArgs a{labels, perm, offsets, static_cast<int32_t*>(ws), n, c, ntiles};
  hist_kernel<<<dim3(ntiles, heads, 1), kThreads, 0, stream>>>(a, a, nullptr, heads);
  SPR_LAUNCH_CHECK();
  scan_kernel<<<dim3(heads, 1), 1024, 0, stream>>>(a, a);
  SPR_LAUNCH_CHECK();
  scatter_kernel<<<dim3(ntiles, heads, 1), kThreads, 0, stream>>>(a, a);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}

}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_partition_layout(const sparsepr_dims* dims, const int32_t* labels_q,
                                             const int32_t* labels_kv, const void* q, const void* k,
                                             const void* v, int32_t* perm_q, int32_t* offsets_q,
                                             int32_t* perm_kv, int32_t* offsets_kv, void* q_g,
                                             void* k_g, void* v_g, int32_t* v_shift,
                                             double* centroid_q, double* centroid_k, void* ws,
                                             size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!labels_q || !labels_kv || !q || !k || !v || !perm_q || !offsets_q || !perm_kv ||
      !offsets_kv || !q_g || !k_g || !v_g || !v_shift || !centroid_q || !centroid_k)
    return SPARSEPR_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(q_g) || !aligned16(k_g) ||
      !aligned16(v_g))
    return SPARSEPR_ERR_INVALID;
  const size_t need = layout_ws_bytes(dims);
  if (need > 0 && (!ws || ws_bytes < need)) return SPARSEPR_ERR_WORKSPACE;
  const int H = dims->heads, d = dims->head_dim;
  Carver cv(ws);
  KindArgs qa{labels_q, perm_q, offsets_q, nullptr, dims->n_q, dims->c_q,
              (dims->n_q + kTile - 1) / kTile};
  KindArgs ka{labels_kv, perm_kv, offsets_kv, nullptr, dims->n_k, dims->c_k,
              (dims->n_k + kTile - 1) / kTile};
  qa.counts = cv.take<int32_t>(size_t(H) * qa.c * qa.ntiles);
  ka.counts = cv.take<int32_t>(size_t(H) * ka.c * ka.ntiles);
  uint32_t* vmax = cv.take<uint32_t>(size_t(H));
  const bool bf16 = dims->dtype == SPARSEPR_BF16;
  const int maxt = qa.ntiles > ka.ntiles ? qa.ntiles : ka.ntiles;

  hist_kernel<<<dim3(maxt, H, 2), kThreads, 0, stream>>>(qa, ka, bf16 ? vmax : nullptr, H);
  SPR_LAUNCH_CHECK();
  scan_kernel<<<dim3(H, 2), 1024, 0, stream>>>(qa, ka);
  SPR_LAUNCH_CHECK();
  scatter_kernel<<<dim3(maxt, H, 2), kThreads, 0, stream>>>(qa, ka);
  SPR_LAUNCH_CHECK();

  const int es = int(elem_bytes(dims->dtype));
  GatherArgs g;
  g.src[0] = static_cast<const char*>(q);
  g.src[1] = static_cast<const char*>(k);
  g.src[2] = static_cast<const char*>(v);
  g.dst[0] = static_cast<char*>(q_g);
  g.dst[1] = static_cast<char*>(k_g);
  g.dst[2] = static_cast<char*>(v_g);
  g.perm[0] = perm_q;
  g.perm[1] = perm_kv;
  g.perm[2] = perm_kv;
  g.stride_head[0] = dims->q_stride_head;
  g.stride_tok[0] = dims->q_stride_tok;
  g.stride_head[1] = g.stride_head[2] = dims->kv_stride_head;
  g.stride_tok[1] = g.stride_tok[2] = dims->kv_stride_tok;
  g.n[0] = dims->n_q;
  g.n[1] = g.n[2] = dims->n_k;
  g.row_bytes = d * es;
  g.esize = es;
  g.vmax = bf16 ? vmax : nullptr;
  g.v_shift = v_shift;
  if (bf16) {
    vmax_kernel<<<dim3((dims->n_k + kVmaxRows - 1) / kVmaxRows, H), kThreads, 0, stream>>>(
        static_cast<const uint16_t*>(v), dims->n_k, d, dims->kv_stride_head, dims->kv_stride_tok,
        vmax);
    SPR_LAUNCH_CHECK();
  }
  const int maxc = dims->c_q > dims->c_k ? dims->c_q : dims->c_k;
  if (dims->dtype == SPARSEPR_BF16)
    gather_group_kernel<uint16_t><<<dim3(maxc, H, 2), kThreads, 0, stream>>>(
        g, offsets_q, offsets_kv, centroid_q, centroid_k, dims->c_q, dims->c_k, d);
  else
    gather_group_kernel<float><<<dim3(maxc, H, 2), kThreads, 0, stream>>>(
        g, offsets_q, offsets_kv, centroid_q, centroid_k, dims->c_q, dims->c_k, d);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}
