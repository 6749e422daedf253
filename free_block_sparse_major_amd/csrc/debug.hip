// Read-only validation of a call's integer data: labels, group layout, cell
// table, routed pair counts and probes.
//
// The quantities checked are those of the SparsePR paper's problem setup
// (§3: the query and key index sets are partitioned into groups, a cell
// G_a x G_b is selected or not) and of its probe step (App. A.2, Algorithm
// A.1: distinct probe rows).  The kernels only read the arrays they check
// and set bits of one error word with vector atomics.  A value read from an
// array is used as an index only after it has been checked to lie inside
// the documented extent of the array it indexes; a value that fails the
// check is reported and never dereferenced.

#include "common.h"

namespace spr {
namespace {

struct DbgArgs {
  const int32_t* labels[2];    // q, kv (may be null)
  const int32_t* offsets[2];   // q, kv (may be null)
  const int32_t* perm[2];      // q, kv (may be null)
  const int32_t* rowptr;       // [H][C_q+1] (may be null)
  const int32_t* col;          // [H][C_q*C_k]
  const long long* routed;     // [H] (may be null)
  const int32_t* probe_rows;   // [H][m] (may be null)
  const int32_t* probe_tokens; // [H][m] (may be null)
  uint32_t* err;
  int H, n[2], c[2], m;
};

__global__ void dbg_zero_kernel(uint32_t* err) {
  if (threadIdx.x == 0) err[0] = 0u;
}

SPR_DEV void flag(uint32_t* err, uint32_t bit) { atomicOr(err, bit); }

// labels in [0, C): grid (tiles of 1024 tokens, H, kind)
__global__ __launch_bounds__(256) void dbg_labels_kernel(DbgArgs p) {
  const int kind = blockIdx.z, h = blockIdx.y;
  const int32_t* lab = p.labels[kind];
  if (!lab) return;
  const int n = p.n[kind], c = p.c[kind];
  bool bad = false;
  for (int i = blockIdx.x * 1024 + threadIdx.x; i < min(n, (blockIdx.x + 1) * 1024); i += 256) {
    const int l = lab[(long long)h * n + i];
    bad |= l < 0 || l >= c;
  }
  if (__ballot(bad) && (threadIdx.x & 63) == 0) flag(p.err, SPARSEPR_DBG_LABELS);
}

// One wave per (group a, head, kind): offsets[a] .. offsets[a+1] inside
// [0, N] and non-decreasing (offsets[0] = 0, offsets[C] = N), then the rows
// of the group: perm in [0, N), strictly ascending, and the label of each
// token equal to a (so perm is the stable counting sort of the labels).
__global__ __launch_bounds__(256) void dbg_groups_kernel(DbgArgs p) {
  const int kind = blockIdx.z, h = blockIdx.y;
  const int a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int32_t* off = p.offsets[kind];
  const int n = p.n[kind], c = p.c[kind];
  if (!off || a >= c) return;
  const int32_t* o = off + (long long)h * (c + 1);
  const int lo = o[a], hi = o[a + 1];
  bool ok = lo >= 0 && hi <= n && lo <= hi;
  if (a == 0) ok = ok && lo == 0;
  if (a == c - 1) ok = ok && hi == n;
  if (!ok) {
    if (lane == 0) flag(p.err, SPARSEPR_DBG_OFFSETS);
    return;
  }
  const int32_t* perm = p.perm[kind];
  if (!perm) return;
  const int32_t* pr = perm + (long long)h * n;
  const int32_t* lab = p.labels[kind] ? p.labels[kind] + (long long)h * n : nullptr;
  bool bad = false;
  for (int j = lo + lane; j < hi; j += 64) {
    const int t = pr[j];
    if (t < 0 || t >= n) {
      bad = true;
      continue;
    }
    if (j > lo) {
      const int tp = pr[j - 1];
      bad |= !(tp < t);
    }
    if (lab) bad |= lab[t] != a;
  }
  if (__ballot(bad) && lane == 0) flag(p.err, SPARSEPR_DBG_PERM);
}

// One wave per (query group a, head): row pointers (rowptr[0] = 0,
// non-decreasing, at most C_q*C_k), then the row's columns: inside [0, C_k),
// strictly ascending, only non-empty K/V groups, and at least one cell for a
// non-empty query group, none for an empty one.
__global__ __launch_bounds__(256) void dbg_cells_kernel(DbgArgs p) {
  const int h = blockIdx.y, a = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int c_q = p.c[0], c_k = p.c[1];
  if (a >= c_q) return;
  if (a == 0 && lane == 0 && p.routed && p.routed[h] < 0) flag(p.err, SPARSEPR_DBG_ROUTE);
  const int32_t* rp = p.rowptr + (long long)h * (c_q + 1);
  const long long cells = (long long)c_q * c_k;
  const int r0 = rp[a], r1 = rp[a + 1];
  bool ok = r0 >= 0 && r0 <= r1 && r1 <= cells;
  if (a == 0) ok = ok && r0 == 0;
  if (!ok) {
    if (lane == 0) flag(p.err, SPARSEPR_DBG_ROWPTR);
    return;
  }
  const int32_t* oq = p.offsets[0] ? p.offsets[0] + (long long)h * (c_q + 1) : nullptr;
  const int32_t* ok_ = p.offsets[1] ? p.offsets[1] + (long long)h * (c_k + 1) : nullptr;
  bool bad = false;
  if (oq) {
    // offsets are checked by dbg_groups_kernel; here they only decide emptiness
    const int na = oq[a + 1] - oq[a];
    bad |= (na > 0) != (r1 > r0);
  }
  const int32_t* col = p.col + (long long)h * cells;
  for (int j = r0 + lane; j < r1; j += 64) {
    const int b = col[j];
    if (b < 0 || b >= c_k) {
      bad = true;
      continue;
    }
    if (j > r0) bad |= !(col[j - 1] < b);
    if (ok_) bad |= ok_[b + 1] <= ok_[b];
  }
  if (__ballot(bad) && lane == 0) flag(p.err, SPARSEPR_DBG_CELLS);
}

// One wave per head: probes.  The first min(m, N_q) rows lie in [0, N_q)
// and are distinct, the rest are -1; each token is perm_q of its row.
__global__ __launch_bounds__(64) void dbg_probes_kernel(DbgArgs p) {
  const int h = blockIdx.x, i = threadIdx.x;
  const int n = p.n[0], m = p.m, me = min(m, n);
  const int32_t* pr = p.probe_rows + (long long)h * m;
  const int32_t* pt = p.probe_tokens ? p.probe_tokens + (long long)h * m : nullptr;
  const int32_t* perm = p.perm[0] ? p.perm[0] + (long long)h * n : nullptr;
  bool bad = false;
  if (i < m) {
    const int r = pr[i];
    if (i >= me) {
      bad = r != -1 || (pt && pt[i] != -1);
    } else if (r < 0 || r >= n) {
      bad = true;
    } else {
      for (int j = 0; j < i; ++j) bad |= pr[j] == r;
      if (pt && perm) bad |= pt[i] != perm[r];
    }
  }
  if (__ballot(bad) && i == 0) flag(p.err, SPARSEPR_DBG_PROBES);
}

}  // namespace
}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_debug_check(const sparsepr_dims* dims, int32_t m,
                                        const int32_t* labels_q, const int32_t* labels_kv,
                                        const int32_t* offsets_q, const int32_t* offsets_kv,
                                        const int32_t* perm_q, const int32_t* perm_kv,
                                        const int32_t* cell_rowptr, const int32_t* cell_col,
                                        const int64_t* routed_pairs, const int32_t* probe_rows,
                                        const int32_t* probe_tokens, uint32_t* error_word,
                                        hipStream_t stream) {
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (!error_word) return SPARSEPR_ERR_INVALID;
  if ((cell_rowptr == nullptr) != (cell_col == nullptr)) return SPARSEPR_ERR_INVALID;
  if (probe_rows && (m < 1 || m > SPARSEPR_MAX_PROBES)) return SPARSEPR_ERR_INVALID;
  DbgArgs a;
  a.labels[0] = labels_q;
  a.labels[1] = labels_kv;
  a.offsets[0] = offsets_q;
  a.offsets[1] = offsets_kv;
  a.perm[0] = perm_q;
  a.perm[1] = perm_kv;
  a.rowptr = cell_rowptr;
  a.col = cell_col;
  a.routed = reinterpret_cast<const long long*>(routed_pairs);
  a.probe_rows = probe_rows;
  a.probe_tokens = probe_tokens;
  a.err = error_word;
  a.H = dims->heads;
  a.n[0] = dims->n_q;
  a.n[1] = dims->n_k;
  a.c[0] = dims->c_q;
  a.c[1] = dims->c_k;
  a.m = m;
  const int H = dims->heads;
  dbg_zero_kernel<<<1, 64, 0, stream>>>(error_word);
  SPR_LAUNCH_CHECK();
  if (labels_q || labels_kv) {
    const int nmax = dims->n_q > dims->n_k ? dims->n_q : dims->n_k;
    dbg_labels_kernel<<<dim3((nmax + 1023) / 1024, H, 2), 256, 0, stream>>>(a);
    SPR_LAUNCH_CHECK();
  }
  if (offsets_q || offsets_kv) {
    const int cmax = dims->c_q > dims->c_k ? dims->c_q : dims->c_k;
    dbg_groups_kernel<<<dim3((cmax + 3) / 4, H, 2), 256, 0, stream>>>(a);
    SPR_LAUNCH_CHECK();
  }
  if (cell_rowptr) {
    dbg_cells_kernel<<<dim3((dims->c_q + 3) / 4, H), 256, 0, stream>>>(a);
    SPR_LAUNCH_CHECK();
  }
  if (probe_rows) {
    dbg_probes_kernel<<<H, 64, 0, stream>>>(a);
    SPR_LAUNCH_CHECK();
  }
  return SPARSEPR_OK;
}
