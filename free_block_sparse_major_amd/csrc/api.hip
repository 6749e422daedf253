// Status strings, shape validation and workspace sizes of the C ABI.
#include "common.h"

namespace spr {

size_t layout_ws_bytes(const sparsepr_dims* d);
size_t route_ws_bytes(const sparsepr_dims* d);
size_t route_ex_ws_bytes(const sparsepr_dims* d);
size_t attn_ws_bytes(const sparsepr_dims* d);
size_t probe_ws_bytes(const sparsepr_dims* d, int32_t m, int32_t rank);
size_t probe_feat_ws_bytes(const sparsepr_dims* d, int32_t m, int32_t rank);
size_t rcp_ws_bytes(const sparsepr_dims* d);

int32_t check_dims(const sparsepr_dims* d) {
  if (!d) return SPARSEPR_ERR_INVALID;
  if (d->heads < 1 || d->n_q < 1 || d->n_k < 1 || d->c_q < 1 || d->c_k < 1 || d->reserved != 0)
    return SPARSEPR_ERR_INVALID;
  if (d->head_dim != 64 && d->head_dim != 128) return SPARSEPR_ERR_UNSUPPORTED;
  if (d->dtype != SPARSEPR_BF16 && d->dtype != SPARSEPR_F32) return SPARSEPR_ERR_UNSUPPORTED;
  if (d->c_q > SPARSEPR_MAX_GROUPS || d->c_k > SPARSEPR_MAX_GROUPS) return SPARSEPR_ERR_UNSUPPORTED;
  const int64_t es = int64_t(elem_bytes(d->dtype));
  // rows are moved with 16-byte accesses: strides in elements are multiples
  // of 16 / es (tested without forming stride * es, which may overflow)
  const int64_t align = 16 / es;
  if ((d->q_stride_head % align) || (d->q_stride_tok % align) || (d->kv_stride_head % align) ||
      (d->kv_stride_tok % align))
    return SPARSEPR_ERR_INVALID;
  if (d->q_stride_tok < d->head_dim || d->kv_stride_tok < d->head_dim ||
      d->q_stride_head < 0 || d->kv_stride_head < 0)
    return SPARSEPR_ERR_INVALID;
  // the byte extent of q and of k, v must be addressable with int64 offsets
  auto extent_ok = [&](int64_t sh, int64_t st, int64_t n) {
    const __int128 last = __int128(d->heads - 1) * sh + __int128(n - 1) * st + d->head_dim;
    return last * es <= (__int128(1) << 62);
  };
  if (!extent_ok(d->q_stride_head, d->q_stride_tok, d->n_q) ||
      !extent_ok(d->kv_stride_head, d->kv_stride_tok, d->n_k))
    return SPARSEPR_ERR_INVALID;
  // group-major tensors are indexed with 32-bit rows inside a head
  if (int64_t(d->c_q) * d->c_k > (int64_t(1) << 30)) return SPARSEPR_ERR_UNSUPPORTED;
  // the bf16 kernels address one head's K or V rows through a buffer
  // resource with 32-bit byte offsets (and the fp32 kernels share the limit)
  if (int64_t(d->n_k) * d->head_dim * es >= (int64_t(1) << 32) ||
      int64_t(d->n_q) * d->head_dim * 4 >= (int64_t(1) << 32))
    return SPARSEPR_ERR_UNSUPPORTED;
  return SPARSEPR_OK;
}

int32_t check_out_strides(const sparsepr_dims* d, int32_t out_dtype, int64_t sh, int64_t st) {
  const int64_t es = out_dtype == SPARSEPR_BF16 ? 2 : 4;
  const int64_t align = 16 / es;
  if ((sh % align) || (st % align) || st < d->head_dim || sh < 0) return SPARSEPR_ERR_INVALID;
  const __int128 last = __int128(d->heads - 1) * sh + __int128(d->n_q - 1) * st + d->head_dim;
  if (last * es > (__int128(1) << 62)) return SPARSEPR_ERR_INVALID;
  return SPARSEPR_OK;
}

}  // namespace spr

extern "C" size_t sparsepr_workspace_bytes(int32_t which, const sparsepr_dims* dims, int32_t m,
                                           int32_t rank) {
  if (spr::check_dims(dims) != SPARSEPR_OK) return 0;
  switch (which) {
    case SPARSEPR_CALL_PARTITION_LAYOUT: return spr::layout_ws_bytes(dims);
    case SPARSEPR_CALL_ROUTE_CELLS: return spr::route_ws_bytes(dims);
    case SPARSEPR_CALL_SPARSE_ATTN: return spr::attn_ws_bytes(dims);
    case SPARSEPR_CALL_PROBE_FIT:
      if (m < 1 || m > SPARSEPR_MAX_PROBES || rank < 0 || rank > SPARSEPR_MAX_RANK) return 0;
      return spr::probe_ws_bytes(dims, m, rank);
    case SPARSEPR_CALL_CORRECT: return 0;
    case SPARSEPR_CALL_RCP_PARTITION: return spr::rcp_ws_bytes(dims);
    case SPARSEPR_CALL_ROUTE_CELLS_EX: return spr::route_ex_ws_bytes(dims);
    case SPARSEPR_CALL_SPARSE_ATTN_CORRECT:
      if (rank < 0 || rank > SPARSEPR_MAX_RANK) return 0;
      return spr::attn_correct_ws_bytes(dims, rank);
    case SPARSEPR_CALL_PROBE_FIT_EX:
      if (m < 1 || m > SPARSEPR_MAX_PROBES || rank < 0 || rank > SPARSEPR_MAX_RANK) return 0;
      return spr::probe_feat_ws_bytes(dims, m, rank);
    default: return 0;
  }
}

extern "C" const char* sparsepr_status_string(int32_t status) {
  switch (status) {
    case SPARSEPR_OK: return "ok";
    case SPARSEPR_ERR_INVALID: return "invalid argument";
    case SPARSEPR_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SPARSEPR_ERR_WORKSPACE: return "workspace too small";
    case SPARSEPR_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

extern "C" int32_t sparsepr_version(void) { return 10000; }
