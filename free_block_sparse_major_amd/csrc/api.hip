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
  // rows are moved with 16-byte accesses
  if (((d->q_stride_head * es) & 15) || ((d->q_stride_tok * es) & 15) ||
      ((d->kv_stride_head * es) & 15) || ((d->kv_stride_tok * es) & 15))
    return SPARSEPR_ERR_INVALID;
  if (d->q_stride_tok < d->head_dim || d->kv_stride_tok < d->head_dim ||
      d->q_stride_head < 0 || d->kv_stride_head < 0)
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
