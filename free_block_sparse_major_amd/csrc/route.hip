// S3-S4: cell routing under a routed pair budget.
//
// SparsePR paper §4.3: every selected cell G_a x G_b costs |G_a||G_b| exact
// interactions and the router keeps the shortest prefix of ranked cells that
// reaches the pair budget (probe cost reserved by the caller).  The score is
// the centroid logit s_ab = qbar_a . kbar_b / sqrt(d) (the value-aware score
// the paper uses is not printed on its pages); every non-empty query group
// first keeps its best cell, then cells follow in (s desc, a asc, b asc)
// order.
//
// The greedy walk is equivalent to: find the crossing cell e* -- the first
// cell (in that order) at which forced pairs + running pairs reach the
// budget -- and select every candidate ordered at or before e*.  e* is found
// without sorting: a 4096-bucket weighted histogram over the score range
// narrows the search to one bucket, repeated until at most kCap candidates
// remain, which are ranked by brute force in LDS.  Pair counts are int64.
//
// Work split: row_stats_kernel takes each query group's forced cell and its
// candidate weight and score range (one wave per group); select_kernel (one
// block per head) reduces them and searches the crossing cell; count_kernel
// and emit_kernel then apply the selection row by row and write the CSR.

#include "common.h"

namespace spr {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kBuckets = 4096;
constexpr int kCap = 2048;

typedef double f64x4_t __attribute__((ext_vector_type(4)));

// scores[h][a][b] = dot(cq[h][a], ck[h][b]) / sqrt_d in fp64, on
// v_mfma_f64_16x16x4_f64: a block of 4 waves computes a 64 x 64 tile, wave w
// rows 16 w .. 16 w + 15 and four 16-column blocks; centroid rows pass
// through LDS 32 dimensions at a time.  Operand lane l holds row (A) or
// column (B) l % 16 at k = l / 16; result lane l holds column l % 16 of rows
// l / 16 + 4 i, i < 4.  Products accumulate in fp64, in a different order
// than a sequential dot product (within fp64 rounding).
// VEC: both centroid arrays 16-byte aligned (chosen on the host), so rows
// move in 16-byte pairs; otherwise one double at a time.
template <bool VEC>
__global__ __launch_bounds__(256) void score_mfma_kernel(const double* __restrict__ cq,
                                                         const double* __restrict__ ck,
                                                         double* __restrict__ scores, int c_q,
                                                         int c_k, int d, double sqrt_d) {
  const int a0 = blockIdx.x * 64, b0 = blockIdx.y * 64, h = blockIdx.z;
  const int tid = threadIdx.x, wid = tid >> 6, lane = tid & 63, r = lane & 15, kq = lane >> 4;
  __shared__ double As[64][33];
  __shared__ double Bs[64][33];
  const double* Q = cq + int64_t(h) * c_q * d;
  const double* K = ck + int64_t(h) * c_k * d;
  f64x4_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  for (int d0 = 0; d0 < d; d0 += 32) {
    if constexpr (!VEC) {
      __syncthreads();
      for (int i = tid; i < 64 * 32; i += 256) {
        const int rr = i >> 5, c = i & 31;
        As[rr][c] = a0 + rr < c_q ? Q[int64_t(a0 + rr) * d + d0 + c] : 0.0;
        Bs[rr][c] = b0 + rr < c_k ? K[int64_t(b0 + rr) * d + d0 + c] : 0.0;
      }
      __syncthreads();
    } else {
    // 16-byte loads, all eight of a thread in flight before the first store
    // (rows are d = 64 or 128 doubles, so with an aligned base every pair is)
    double2 qa[4], kb[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, rr = i >> 4, c = 2 * (i & 15);
      qa[u] = a0 + rr < c_q
                  ? *reinterpret_cast<const double2*>(Q + int64_t(a0 + rr) * d + d0 + c)
                  : double2{0.0, 0.0};
      kb[u] = b0 + rr < c_k
                  ? *reinterpret_cast<const double2*>(K + int64_t(b0 + rr) * d + d0 + c)
                  : double2{0.0, 0.0};
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = tid + 256 * u, rr = i >> 4, c = 2 * (i & 15);
      As[rr][c] = qa[u].x;
      As[rr][c + 1] = qa[u].y;
      Bs[rr][c] = kb[u].x;
      Bs[rr][c + 1] = kb[u].y;
    }
    __syncthreads();
    }
#pragma unroll
    for (int kk = 0; kk < 32; kk += 4) {
      const double av = As[16 * wid + r][kk + kq];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[j] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, Bs[16 * j + r][kk + kq], acc[j], 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int b = b0 + 16 * j + r;
    if (b >= c_k) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = a0 + 16 * wid + kq + 4 * i;
      if (a < c_q) scores[(int64_t(h) * c_q + a) * c_k + b] = acc[j][i] / sqrt_d;
    }
  }
}

enum { kModeNone = 0, kModeAll = 1, kModeThresh = 2, kModeFailed = 3 };
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kMaxRowChunks = SPARSEPR_MAX_GROUPS / 64;

// Per-head outcome of the crossing search: every cell with (s, a c_k + b)
// ordered at or before (es, ei) is selected (mode kModeThresh), every
// candidate (kModeAll) or none besides the forced cells (kModeNone).
// kModeFailed: the search found no crossing cell, which finite scores never
// cause (see select_kernel); the head keeps its forced cells only and its
// routed pair count is reported as -1.
struct SelState {
  double es;
  int32_t ei;
  int32_t mode;
};

// Pass 1, one wave per query group a: forced cell (best score over the
// non-empty K/V groups, ties -> smaller b; -1 for an empty group), forced
// pairs, candidate weight (the other non-empty cells) and candidate score range.
__global__ __launch_bounds__(256) void row_stats_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ off_k, int c_q, int c_k, int32_t* __restrict__ forced,
    long long* __restrict__ row_f, long long* __restrict__ row_w, double* __restrict__ row_min,
    double* __restrict__ row_max) {
  const int h = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= c_q) return;
  const int32_t* oq = off_q + int64_t(h) * (c_q + 1);
  const int32_t* ok = off_k + int64_t(h) * (c_k + 1);
  const long long o = int64_t(h) * c_q + a;
  const int n_a = oq[a + 1] - oq[a];
  if (n_a == 0) {
    if (lane == 0) {
      forced[o] = -1;
      row_f[o] = 0;
      row_w[o] = 0;
      row_min[o] = __builtin_huge_val();
      row_max[o] = -__builtin_huge_val();
    }
    return;
  }
  const double* S = scores + (int64_t(h) * c_q + a) * c_k;
  const int nbk = (c_k + 63) / 64;
  double sv[kMaxRowChunks];
  int mbv[kMaxRowChunks];
  double best = 0.0;
  int bb = -1;
  // every load first (scores and group sizes are independent), then the
  // candidate tests, so the loads of a row are in flight together
#pragma unroll
  for (int k = 0; k < kMaxRowChunks; ++k) {
    const int b = 64 * k + lane;
    const bool in = k < nbk && b < c_k;
    sv[k] = in ? S[b] : 0.0;
    mbv[k] = in ? ok[b + 1] - ok[b] : 0;
  }
#pragma unroll
  for (int k = 0; k < kMaxRowChunks; ++k) {
    const int b = 64 * k + lane;
    if (mbv[k] > 0 && (bb < 0 || sv[k] > best)) { best = sv[k]; bb = b; }
  }
#pragma unroll
  for (int sh = 32; sh > 0; sh >>= 1) {
    const double s2 = __shfl_xor(best, sh);
    const int b2 = __shfl_xor(bb, sh);
    if (b2 >= 0 && (bb < 0 || s2 > best || (s2 == best && b2 < bb))) { best = s2; bb = b2; }
  }
  long long wpart = 0;
  double lmin = __builtin_huge_val(), lmax = -__builtin_huge_val();
#pragma unroll
  for (int k = 0; k < kMaxRowChunks; ++k) {
    const int b = 64 * k + lane;
    if (k < nbk && b < c_k && b != bb && mbv[k] > 0) {
      wpart += (long long)n_a * mbv[k];
      lmin = sv[k] < lmin ? sv[k] : lmin;
      lmax = sv[k] > lmax ? sv[k] : lmax;
    }
  }
  wpart = wave_sum(wpart);
#pragma unroll
  for (int sh = 32; sh > 0; sh >>= 1) {
    lmin = fmin(lmin, __shfl_xor(lmin, sh));
    lmax = fmax(lmax, __shfl_xor(lmax, sh));
  }
  if (lane == 0) {
    forced[o] = bb;
    row_f[o] = bb >= 0 ? (long long)n_a * (ok[bb + 1] - ok[bb]) : 0;
    row_w[o] = wpart;
    row_min[o] = lmin;
    row_max[o] = lmax;
  }
}

// One block per head: the crossing search.  Every pass walks the cell matrix
// row by row (one wave per query group, lanes over K/V groups), so row
// quantities are wave-uniform and the score reads are coalesced.
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ off_k, int c_q, int c_k, long long budget,
    const int32_t* __restrict__ forced_g, const long long* __restrict__ row_f,
    const long long* __restrict__ row_w, const double* __restrict__ row_min,
    const double* __restrict__ row_max, SelState* __restrict__ state) {
  const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  __shared__ int32_t na[SPARSEPR_MAX_GROUPS], mb[SPARSEPR_MAX_GROUPS];
  __shared__ int32_t forced[SPARSEPR_MAX_GROUPS];
  __shared__ unsigned long long hist_w[kBuckets];
  __shared__ uint32_t hist_c[kBuckets];
  __shared__ double cand_s[kCap];
  __shared__ int32_t cand_i[kCap];
  __shared__ long long red[kSelWaves];
  __shared__ double redd[kSelWaves];
  __shared__ int32_t slot;
  __shared__ long long sh_tp;
  __shared__ int32_t sh_j;
  __shared__ uint32_t sh_cnt;
  __shared__ double sh_es;
  __shared__ int32_t sh_ei;

  const int32_t* oq = off_q + int64_t(h) * (c_q + 1);
  const int32_t* ok = off_k + int64_t(h) * (c_k + 1);
  const long long ro = int64_t(h) * c_q;
  long long fpart = 0, wpart = 0;
  double lmin = __builtin_huge_val(), lmax = -__builtin_huge_val();
  for (int i = tid; i < c_q; i += kSelThreads) {
    na[i] = oq[i + 1] - oq[i];
    forced[i] = forced_g[ro + i];
    fpart += row_f[ro + i];
    wpart += row_w[ro + i];
    lmin = fmin(lmin, row_min[ro + i]);
    lmax = fmax(lmax, row_max[ro + i]);
  }
  for (int i = tid; i < c_k; i += kSelThreads) mb[i] = ok[i + 1] - ok[i];
  if (tid == 0) { sh_es = 0.0; sh_ei = -1; }
  const long long F = block_sum(fpart, red);
  const long long W = block_sum(wpart, red);
  double lo = block_min(lmin, redd);
  double hi = block_max(lmax, redd);
  const double* S = scores + int64_t(h) * c_q * c_k;
  const int nbk = (c_k + 63) / 64;

  // candidate cells (non-empty, not forced) of the rows this wave walks; a
  // row's scores are loaded together before its candidates are visited
  auto for_cands = [&](auto&& fn) {
    for (int a = wid; a < c_q; a += kSelWaves) {
      const int n_a = na[a];
      if (n_a == 0) continue;
      const int fb = forced[a];
      double sv[kMaxRowChunks];
#pragma unroll
      for (int k = 0; k < kMaxRowChunks; ++k) {
        const int b = 64 * k + lane;
        sv[k] = k < nbk && b < c_k ? S[int64_t(a) * c_k + b] : 0.0;
      }
#pragma unroll
      for (int k = 0; k < kMaxRowChunks; ++k) {
        const int b = 64 * k + lane;
        if (k < nbk && b < c_k && b != fb) {
          const int m = mb[b];
          if (m > 0) fn(sv[k], (long long)n_a * m, a * c_k + b);
        }
      }
    }
  };

  int mode = kModeNone;
  double es = 0.0;
  int ei = -1;
  const long long T = budget - F;
  if (T > 0) {
    if (W <= T) {
      mode = kModeAll;
    } else {
      mode = kModeThresh;
      long long Tp = T;  // weight still to take inside [lo, hi] (everything above is taken)
      // Termination: each round either ends (a tie range or at most kCap
      // candidates) or replaces [lo, hi] by the exact score range of one of
      // kBuckets = 2^12 equal-width buckets.  The range of finite fp64
      // scores is below 2^1025 and distinct scores differ by at least
      // 2^-1074, so at most 175 rounds are ever needed; a non-finite score
      // (NaN or Inf inputs) can leave the crossing unresolved, which is
      // reported.
      bool found = false;
      for (int round = 0; round < 256; ++round) {
        if (lo == hi) {
          // every remaining candidate has the same score: index order decides
          const int cells = c_q * c_k;
          const int per = (cells + kSelThreads - 1) / kSelThreads;
          const int i0 = tid * per, i1 = min(cells, i0 + per);
          auto cand_at = [&](int idx, long long& w) -> bool {
            const int a = idx / c_k, b = idx - a * c_k;
            if (na[a] == 0 || mb[b] == 0 || b == forced[a] || S[idx] != lo) return false;
            w = (long long)na[a] * mb[b];
            return true;
          };
          long long part = 0;
          for (int idx = i0; idx < i1; ++idx) {
            long long w;
            if (cand_at(idx, w)) part += w;
          }
          long long tot;
          long long run = block_exclusive_scan(part, red, &tot);
          for (int idx = i0; idx < i1; ++idx) {
            long long w;
            if (cand_at(idx, w)) {
              if (run < Tp && Tp <= run + w) { sh_es = lo; sh_ei = idx; }
              run += w;
            }
          }
          __syncthreads();
          es = sh_es;
          ei = sh_ei;
          found = true;
          break;
        }
        // weighted histogram of the candidates in [lo, hi]; bucket() is
        // monotone in the score, so equal scores share a bucket
        const double scale = double(kBuckets) / (hi - lo);
        auto bucket = [&](double sc) -> int {
          const int bk = int((sc - lo) * scale);
          return bk < 0 ? 0 : (bk < kBuckets ? bk : kBuckets - 1);
        };
        for (int i = tid; i < kBuckets; i += kSelThreads) { hist_w[i] = 0; hist_c[i] = 0; }
        __syncthreads();
        for_cands([&](double sc, long long w, int) {
          if (sc >= lo && sc <= hi) {
            const int bk = bucket(sc);
            atomicAdd(&hist_w[bk], (unsigned long long)w);
            atomicAdd(&hist_c[bk], 1u);
          }
        });
        __syncthreads();
        // crossing bucket: scanning down from the top, the first bucket at
        // which the accumulated weight reaches Tp
        {
          constexpr int BPT = kBuckets / kSelThreads;
          long long loc = 0;
#pragma unroll
          for (int j = 0; j < BPT; ++j) loc += (long long)hist_w[BPT * tid + j];
          long long tot;
          const long long pre = block_exclusive_scan(loc, red, &tot);
          long long acc = tot - pre - loc;  // weight of the buckets above this thread's
#pragma unroll
          for (int j = BPT - 1; j >= 0; --j) {
            const int bk = BPT * tid + j;
            const long long w = (long long)hist_w[bk];
            if (acc < Tp && Tp <= acc + w) {
              sh_j = bk;
              sh_tp = Tp - acc;
              sh_cnt = hist_c[bk];
            }
            acc += w;
          }
        }
        __syncthreads();
        const int jb = sh_j;
        Tp = sh_tp;
        const uint32_t cnt = sh_cnt;
        if (cnt <= kCap) {
          if (tid == 0) slot = 0;
          __syncthreads();
          for_cands([&](double sc, long long, int idx) {
            if (sc >= lo && sc <= hi && bucket(sc) == jb) {
              const int p = atomicAdd(&slot, 1);
              cand_s[p] = sc;
              cand_i[p] = idx;
            }
          });
          __syncthreads();
          const int n = slot;
          for (int i = tid; i < n; i += kSelThreads) {
            const double si = cand_s[i];
            const int ii = cand_i[i];
            long long pre = 0;
            for (int j = 0; j < n; ++j) {
              const double sj = cand_s[j];
              const int ij = cand_i[j];
              if (sj > si || (sj == si && ij < ii)) {
                const int aj = ij / c_k;
                pre += (long long)na[aj] * mb[ij - aj * c_k];
              }
            }
            const int ai = ii / c_k;
            const long long w = (long long)na[ai] * mb[ii - ai * c_k];
            if (pre < Tp && Tp <= pre + w) { sh_es = si; sh_ei = ii; }
          }
          __syncthreads();
          es = sh_es;
          ei = sh_ei;
          found = true;
          break;
        }
        // narrow to the exact score range of the crossing bucket
        double bmin = __builtin_huge_val(), bmax = -__builtin_huge_val();
        for_cands([&](double sc, long long, int) {
          if (sc >= lo && sc <= hi && bucket(sc) == jb) {
            bmin = sc < bmin ? sc : bmin;
            bmax = sc > bmax ? sc : bmax;
          }
        });
        const double nlo = block_min(bmin, redd);
        const double nhi = block_max(bmax, redd);
        lo = nlo;
        hi = nhi;
        if (!(lo <= hi)) break;   // NaN bounds: no crossing can be found
      }
      if (!found || ei < 0) mode = kModeFailed;
    }
  }

  if (tid == 0) state[h] = SelState{es, ei, mode};
}

// Whether cell (a, b) of head h is selected (the forced cell, or ordered at
// or before the crossing cell).
SPR_DEV bool cell_selected(const SelState& st, int n_a, int m_b, int fb, int a, int b, int c_k,
                           const double* S) {
  if (n_a == 0 || m_b == 0) return false;
  if (b == fb) return true;
  if (st.mode == kModeAll) return true;
  if (st.mode == kModeNone || st.mode == kModeFailed) return false;
  const double sc = S[int64_t(a) * c_k + b];
  const int idx = a * c_k + b;
  return sc > st.es || (sc == st.es && idx <= st.ei);
}

// Selected cells and pairs of each query group (one wave per group).
__global__ __launch_bounds__(256) void count_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ off_k, int c_q, int c_k, const int32_t* __restrict__ forced,
    const SelState* __restrict__ state, int32_t* __restrict__ row_cnt,
    long long* __restrict__ row_p) {
  const int h = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= c_q) return;
  const int32_t* oq = off_q + int64_t(h) * (c_q + 1);
  const int32_t* ok = off_k + int64_t(h) * (c_k + 1);
  const SelState st = state[h];
  const int n_a = oq[a + 1] - oq[a], fb = forced[int64_t(h) * c_q + a];
  const double* S = scores + int64_t(h) * c_q * c_k;
  int cnt = 0;
  long long pp = 0;
  for (int b0 = 0; b0 < c_k; b0 += 64) {
    const int b = b0 + lane;
    const int m_b = b < c_k ? ok[b + 1] - ok[b] : 0;
    const bool f = b < c_k && cell_selected(st, n_a, m_b, fb, a, b, c_k, S);
    cnt += __popcll(__ballot(f));
    if (f) pp += (long long)n_a * m_b;
  }
  pp = wave_sum(pp);
  if (lane == 0) {
    row_cnt[int64_t(h) * c_q + a] = cnt;
    row_p[int64_t(h) * c_q + a] = pp;
  }
}

// CSR rows (b ascending) and row pointers; the last group's wave also writes
// the end pointer and the head's routed pairs.  One wave per group.
__global__ __launch_bounds__(256) void emit_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ off_k, int c_q, int c_k, const int32_t* __restrict__ forced,
    const SelState* __restrict__ state, const int32_t* __restrict__ row_cnt,
    const long long* __restrict__ row_p, int32_t* __restrict__ rowptr,
    int32_t* __restrict__ col, long long* __restrict__ routed) {
  const int h = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (a >= c_q) return;
  const int32_t* oq = off_q + int64_t(h) * (c_q + 1);
  const int32_t* ok = off_k + int64_t(h) * (c_k + 1);
  const int32_t* rc = row_cnt + int64_t(h) * c_q;
  long long pre = 0;
  for (int i = lane; i < a; i += 64) pre += rc[i];
  pre = wave_sum(pre);
  int32_t* rp = rowptr + int64_t(h) * (c_q + 1);
  if (lane == 0) rp[a] = int32_t(pre);
  if (a == c_q - 1) {
    long long pt = 0;
    const long long* rpp = row_p + int64_t(h) * c_q;
    for (int i = lane; i < c_q; i += 64) pt += rpp[i];
    pt = wave_sum(pt);
    if (lane == 0) {
      rp[c_q] = int32_t(pre + rc[a]);
      routed[h] = state[h].mode == kModeFailed ? -1LL : pt;
    }
  }
  const SelState st = state[h];
  const int n_a = oq[a + 1] - oq[a], fb = forced[int64_t(h) * c_q + a];
  const double* S = scores + int64_t(h) * c_q * c_k;
  int32_t* cl = col + int64_t(h) * c_q * c_k;
  int pos = int(pre);
  for (int b0 = 0; b0 < c_k; b0 += 64) {
    const int b = b0 + lane;
    const int m_b = b < c_k ? ok[b + 1] - ok[b] : 0;
    const bool f = b < c_k && cell_selected(st, n_a, m_b, fb, a, b, c_k, S);
    const unsigned long long m = __ballot(f);
    if (f) cl[pos + __popcll(m & ((1ull << lane) - 1ull))] = b;
    pos += __popcll(m);
  }
}

// ---------------------------------------------------------------------------
// Per-group rule ([paper] §4.3): each query group ranks the non-empty K/V
// groups by decreasing score (ties -> smaller b) and keeps the shortest
// prefix whose key-token count reaches the common per-query budget (at
// least its top cell).  One block per (a, h) sorts its row of scores in LDS
// (bitonic, (ordered score, b) keys), scans the group sizes in that order
// and writes its selected b ascending into a per-row slot; a per-head scan
// gives the CSR row pointers and a copy pass compacts the rows.
// ---------------------------------------------------------------------------
// fp64 -> uint64 whose ascending order is the descending order of the score
SPR_DEV unsigned long long desc_key(double s) {
  unsigned long long u = __double_as_longlong(s);
  u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);   // ascending order of s
  return ~u;
}

__global__ __launch_bounds__(256) void group_route_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ off_q,
    const int32_t* __restrict__ off_k, int c_q, int c_k, long long key_budget,
    int32_t* __restrict__ slots, int32_t* __restrict__ counts, long long* __restrict__ pairs) {
  const int a = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  constexpr int N = SPARSEPR_MAX_GROUPS;
  __shared__ unsigned long long key[N];
  __shared__ int32_t idx[N];
  __shared__ int32_t take[N];
  __shared__ long long red[4];
  const int32_t* oq = off_q + (long long)h * (c_q + 1);
  const int32_t* ok = off_k + (long long)h * (c_k + 1);
  const long long na = oq[a + 1] - oq[a];
  const long long row = (long long)h * c_q + a;
  if (na == 0) {
    if (tid == 0) {
      counts[row] = 0;
      pairs[row] = 0;
    }
    return;
  }
  int np2 = 1;
  while (np2 < c_k) np2 <<= 1;
  const double* S = scores + row * c_k;
  for (int b = tid; b < np2; b += 256) {
    const bool ne = b < c_k && ok[b + 1] > ok[b];
    key[b] = ne ? desc_key(S[b]) : ~0ull;   // empty / padding sort last
    idx[b] = b;
    take[b] = 0;
  }
  __syncthreads();
  for (int size = 2; size <= np2; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = tid; p < np2 / 2; p += 256) {
        const int i = 2 * p - (p & (stride - 1)), j = i + stride;
        const bool up = (i & size) == 0;
        const unsigned long long ki = key[i], kj = key[j];
        const int ii = idx[i], ij = idx[j];
        const bool gt = ki > kj || (ki == kj && ii > ij);
        if (gt == up) {
          key[i] = kj;
          key[j] = ki;
          idx[i] = ij;
          idx[j] = ii;
        }
      }
      __syncthreads();
    }
  }
  // inclusive prefix of group sizes in sorted order (4 entries per thread)
  long long v[4], loc = 0;
  const int base = 4 * tid;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = base + u;
    v[u] = (i < np2 && key[i] != ~0ull) ? (long long)(ok[idx[i] + 1] - ok[idx[i]]) : 0;
    loc += v[u];
  }
  long long tot;
  long long run = block_exclusive_scan(loc, red, &tot);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = base + u;
    // selected: non-empty and the prefix before it is still below the budget
    // (the top cell always)
    if (i < np2 && key[i] != ~0ull && (i == 0 || run < key_budget)) take[idx[i]] = 1;
    run += v[u];
  }
  __syncthreads();
  // selected b ascending into the row's slot, and the row's pair count
  long long cnt = 0, keys = 0;
  int t4[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int b = base + u;
    t4[u] = b < c_k ? take[b] : 0;
    cnt += t4[u];
    keys += t4[u] ? (long long)(ok[b + 1] - ok[b]) : 0;
  }
  long long ntot;
  long long pos = block_exclusive_scan(cnt, red, &ntot);
  const long long ksum = block_sum(keys, red);
  int32_t* out = slots + row * c_k;
#pragma unroll
  for (int u = 0; u < 4; ++u)
    if (t4[u]) out[pos++] = base + u;
  if (tid == 0) {
    counts[row] = int32_t(ntot);
    pairs[row] = na * ksum;
  }
}

// per head: row pointers (exclusive scan of the counts) and the pair total
__global__ __launch_bounds__(1024) void group_rowptr_kernel(const int32_t* __restrict__ counts,
                                                            const long long* __restrict__ pairs,
                                                            int c_q, int32_t* __restrict__ rowptr,
                                                            long long* __restrict__ routed) {
  const int h = blockIdx.x, tid = threadIdx.x;
  __shared__ long long red[16];
  const long long c = tid < c_q ? counts[(long long)h * c_q + tid] : 0;
  const long long p = tid < c_q ? pairs[(long long)h * c_q + tid] : 0;
  long long tot;
  const long long ex = block_exclusive_scan(c, red, &tot);
  if (tid < c_q) rowptr[(long long)h * (c_q + 1) + tid] = int32_t(ex);
  if (tid == 0) rowptr[(long long)h * (c_q + 1) + c_q] = int32_t(tot);
  const long long ps = block_sum(p, red);
  if (tid == 0) routed[h] = ps;
}

__global__ __launch_bounds__(256) void group_copy_kernel(const int32_t* __restrict__ slots,
                                                         const int32_t* __restrict__ counts,
                                                         const int32_t* __restrict__ rowptr,
                                                         int c_q, int c_k,
                                                         int32_t* __restrict__ col) {
  const int a = blockIdx.x, h = blockIdx.y;
  const long long row = (long long)h * c_q + a;
  const int n = counts[row], dst = rowptr[(long long)h * (c_q + 1) + a];
  for (int i = threadIdx.x; i < n; i += 256)
    col[(long long)h * c_q * c_k + dst + i] = slots[row * c_k + i];
}

}  // namespace

size_t route_ex_ws_bytes(const sparsepr_dims* d) {
  Carver cv(nullptr);
  cv.take<double>(size_t(d->heads) * d->c_q * d->c_k);
  cv.take<int32_t>(size_t(d->heads) * d->c_q * d->c_k);
  cv.take<int32_t>(size_t(d->heads) * d->c_q);
  cv.take<long long>(size_t(d->heads) * d->c_q);
  return cv.used;
}

// global rule: scores, then per-row statistics, the per-head search outcome
// and the per-row counts
struct SelWs {
  double* scores;
  int32_t *forced, *row_cnt;
  long long *row_f, *row_w, *row_p;
  double *row_min, *row_max;
  SelState* state;
};

SelWs carve_sel(void* base, const sparsepr_dims* d, size_t* used) {
  Carver cv(base);
  const size_t H = d->heads, R = H * d->c_q;
  SelWs w;
  w.scores = cv.take<double>(R * d->c_k);
  w.forced = cv.take<int32_t>(R);
  w.row_cnt = cv.take<int32_t>(R);
  w.row_f = cv.take<long long>(R);
  w.row_w = cv.take<long long>(R);
  w.row_p = cv.take<long long>(R);
  w.row_min = cv.take<double>(R);
  w.row_max = cv.take<double>(R);
  w.state = cv.take<SelState>(H);
  if (used) *used = cv.used;
  return w;
}

size_t route_ws_bytes(const sparsepr_dims* d) {
  size_t used = 0;
  carve_sel(nullptr, d, &used);
  return used;
}

}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_route_cells_ex(const sparsepr_dims* dims, int32_t rule,
                                           const int32_t* offsets_q, const int32_t* offsets_kv,
                                           const double* centroid_q, const double* centroid_k,
                                           int64_t budget, int32_t* cell_rowptr,
                                           int32_t* cell_col, int64_t* routed_pairs, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  if (rule == SPARSEPR_ROUTE_GLOBAL)
    return sparsepr_route_cells(dims, offsets_q, offsets_kv, centroid_q, centroid_k, budget,
                                cell_rowptr, cell_col, routed_pairs, ws, ws_bytes, stream);
  if (rule != SPARSEPR_ROUTE_PER_GROUP) return SPARSEPR_ERR_INVALID;
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!offsets_q || !offsets_kv || !centroid_q || !centroid_k || !cell_rowptr || !cell_col ||
      !routed_pairs)
    return SPARSEPR_ERR_INVALID;
  const size_t need = route_ex_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  const int H = dims->heads, d = dims->head_dim;
  Carver cv(ws);
  double* scores = cv.take<double>(size_t(H) * dims->c_q * dims->c_k);
  int32_t* slots = cv.take<int32_t>(size_t(H) * dims->c_q * dims->c_k);
  int32_t* counts = cv.take<int32_t>(size_t(H) * dims->c_q);
  long long* pairs = cv.take<long long>(size_t(H) * dims->c_q);
  dim3 g1((dims->c_q + 63) / 64, (dims->c_k + 63) / 64, H);
  if (aligned16(centroid_q) && aligned16(centroid_k))
    score_mfma_kernel<true><<<g1, 256, 0, stream>>>(centroid_q, centroid_k, scores, dims->c_q,
                                                    dims->c_k, d, __builtin_sqrt(double(d)));
  else
    score_mfma_kernel<false><<<g1, 256, 0, stream>>>(centroid_q, centroid_k, scores, dims->c_q,
                                                     dims->c_k, d, __builtin_sqrt(double(d)));
  SPR_LAUNCH_CHECK();
  group_route_kernel<<<dim3(dims->c_q, H), 256, 0, stream>>>(scores, offsets_q, offsets_kv,
                                                             dims->c_q, dims->c_k,
                                                             (long long)budget, slots, counts,
                                                             pairs);
  SPR_LAUNCH_CHECK();
  group_rowptr_kernel<<<H, 1024, 0, stream>>>(counts, pairs, dims->c_q, cell_rowptr,
                                              (long long*)routed_pairs);
  SPR_LAUNCH_CHECK();
  group_copy_kernel<<<dim3(dims->c_q, H), 256, 0, stream>>>(slots, counts, cell_rowptr, dims->c_q,
                                                            dims->c_k, cell_col);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}

extern "C" int32_t sparsepr_route_cells(const sparsepr_dims* dims, const int32_t* offsets_q,
                                        const int32_t* offsets_kv, const double* centroid_q,
                                        const double* centroid_k, int64_t routed_pair_budget,
                                        int32_t* cell_rowptr, int32_t* cell_col,
                                        int64_t* routed_pairs, void* ws, size_t ws_bytes,
                                        hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!offsets_q || !offsets_kv || !centroid_q || !centroid_k || !cell_rowptr || !cell_col ||
      !routed_pairs)
    return SPARSEPR_ERR_INVALID;
  const size_t need = route_ws_bytes(dims);
  if (!ws || ws_bytes < need) return SPARSEPR_ERR_WORKSPACE;
  const SelWs w = carve_sel(ws, dims, nullptr);
  const int H = dims->heads, d = dims->head_dim, c_q = dims->c_q, c_k = dims->c_k;
  dim3 g1((c_q + 63) / 64, (c_k + 63) / 64, H);
  if (aligned16(centroid_q) && aligned16(centroid_k))
    score_mfma_kernel<true><<<g1, 256, 0, stream>>>(centroid_q, centroid_k, w.scores, c_q, c_k,
                                                    d, __builtin_sqrt(double(d)));
  else
    score_mfma_kernel<false><<<g1, 256, 0, stream>>>(centroid_q, centroid_k, w.scores, c_q, c_k,
                                                     d, __builtin_sqrt(double(d)));
  SPR_LAUNCH_CHECK();
  const dim3 gr((c_q + 3) / 4, H);
  row_stats_kernel<<<gr, 256, 0, stream>>>(w.scores, offsets_q, offsets_kv, c_q, c_k, w.forced,
                                           w.row_f, w.row_w, w.row_min, w.row_max);
  SPR_LAUNCH_CHECK();
  select_kernel<<<H, kSelThreads, 0, stream>>>(w.scores, offsets_q, offsets_kv, c_q, c_k,
                                               (long long)routed_pair_budget, w.forced, w.row_f,
                                               w.row_w, w.row_min, w.row_max, w.state);
  SPR_LAUNCH_CHECK();
  count_kernel<<<gr, 256, 0, stream>>>(w.scores, offsets_q, offsets_kv, c_q, c_k, w.forced,
                                       w.state, w.row_cnt, w.row_p);
  SPR_LAUNCH_CHECK();
  emit_kernel<<<gr, 256, 0, stream>>>(w.scores, offsets_q, offsets_kv, c_q, c_k, w.forced,
                                      w.state, w.row_cnt, w.row_p, cell_rowptr, cell_col,
                                      (long long*)routed_pairs);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}
