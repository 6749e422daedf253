// S9: corrected output in original token order.
//
// Review of the SparsePR paper, method summary step (5): unprobed rows get
// their sparse output plus the predicted residual, probe rows their exact
// dense output, and the result returns to the original order.  With the
// folded fit, out = o + (o A) Psi^T + c.
//
// HBM-bound: O_sp is read once and the output written once.  One query row
// per lane, held in registers; the 2 * d * rank FMAs per row take A and Psi
// as wave-uniform operands (scalar loads of the per-head factors, which every
// lane shares), so no LDS or cross-lane traffic is needed.

#include "common.h"

namespace spr {
namespace {

struct CorrArgs {
  const int32_t* perm_q;
  const float* o_sp;
  const float* corr_a;
  const float* corr_psi_t;
  const float* corr_c;
  void* out;
  int64_t out_sh, out_st;
  int n_q, rank;
  int out_bf16;
};

template <int D, int RK>
__global__ __launch_bounds__(256) void correct_kernel(const int32_t* __restrict__ perm_q,
                                                      const float* __restrict__ o_sp,
                                                      const float* __restrict__ corr_a,
                                                      const float* __restrict__ corr_psi_t,
                                                      const float* __restrict__ corr_c,
                                                      void* __restrict__ out, int64_t out_sh,
                                                      int64_t out_st, int n_q, int rank,
                                                      int out_bf16) {
  const int h = blockIdx.y;
  const int r = blockIdx.x * 256 + threadIdx.x;
  const bool valid = r < n_q;
  const float* __restrict__ Ah = corr_a + (long long)h * D * rank;      // [D][rank]
  const float* __restrict__ Ph = corr_psi_t + (long long)h * rank * D;  // [rank][D]
  const float* __restrict__ ch = corr_c + (long long)h * D;
  const float* src = o_sp + ((long long)h * n_q + (valid ? r : 0)) * D;
  float o[D];
#pragma unroll
  for (int c = 0; c < D / 4; ++c) {
    const float4 v = *reinterpret_cast<const float4*>(src + 4 * c);
    o[4 * c] = v.x;
    o[4 * c + 1] = v.y;
    o[4 * c + 2] = v.z;
    o[4 * c + 3] = v.w;
  }
  const int tok = valid ? perm_q[(long long)h * n_q + r] : 0;
  // u = o A: i outer, so each step reads one contiguous row A[i][0 .. RK)
  float u[RK];
#pragma unroll
  for (int k = 0; k < RK; ++k) u[k] = 0.f;
  if (rank == RK) {
#pragma unroll
    for (int i = 0; i < D; ++i)
#pragma unroll
      for (int k = 0; k < RK; ++k) u[k] = fmaf(o[i], Ah[i * RK + k], u[k]);
  } else {
    for (int k = 0; k < rank; ++k) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < D; ++i) acc = fmaf(o[i], Ah[i * rank + k], acc);
#pragma unroll
      for (int kk = 0; kk < RK; ++kk)
        if (kk == k) u[kk] = acc;
    }
  }
  // o + c + u Psi^T: k outer, so each step reads one contiguous row Psi^T[k]
#pragma unroll
  for (int i = 0; i < D; ++i) o[i] += ch[i];
#pragma unroll
  for (int k = 0; k < RK; ++k) {
    if (k >= rank) break;
#pragma unroll
    for (int i = 0; i < D; ++i) o[i] = fmaf(u[k], Ph[k * D + i], o[i]);
  }
  if (!valid) return;
  const long long base = (long long)h * out_sh + (long long)tok * out_st;
  if (out_bf16) {
    uint16_t* dst = static_cast<uint16_t*>(out) + base;
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      uint4 w;
      w.x = uint32_t(f32_to_bf16_rne(o[8 * c])) | (uint32_t(f32_to_bf16_rne(o[8 * c + 1])) << 16);
      w.y = uint32_t(f32_to_bf16_rne(o[8 * c + 2])) | (uint32_t(f32_to_bf16_rne(o[8 * c + 3])) << 16);
      w.z = uint32_t(f32_to_bf16_rne(o[8 * c + 4])) | (uint32_t(f32_to_bf16_rne(o[8 * c + 5])) << 16);
      w.w = uint32_t(f32_to_bf16_rne(o[8 * c + 6])) | (uint32_t(f32_to_bf16_rne(o[8 * c + 7])) << 16);
      *reinterpret_cast<uint4*>(dst + 8 * c) = w;
    }
  } else {
    float* dst = static_cast<float*>(out) + base;
#pragma unroll
    for (int c = 0; c < D / 4; ++c)
      *reinterpret_cast<float4*>(dst + 4 * c) =
          make_float4(o[4 * c], o[4 * c + 1], o[4 * c + 2], o[4 * c + 3]);
  }
}

// probe rows take their dense output (after the correction pass on the stream)
__global__ __launch_bounds__(256) void probe_overwrite_kernel(const int32_t* __restrict__ tokens,
                                                              const float* __restrict__ dense,
                                                              int m, int d, void* out,
                                                              int64_t sh, int64_t st,
                                                              int out_bf16) {
  const int h = blockIdx.x;
  for (int e = threadIdx.x; e < m * d; e += 256) {
    const int p = e / d, j = e % d;
    const int tok = tokens[(long long)h * m + p];
    if (tok < 0) continue;
    const float v = dense[((long long)h * m + p) * d + j];
    const long long o = (long long)h * sh + (long long)tok * st + j;
    if (out_bf16) static_cast<uint16_t*>(out)[o] = f32_to_bf16_rne(v);
    else static_cast<float*>(out)[o] = v;
  }
}

template <int D>
void launch_correct(const CorrArgs& a, dim3 grid, hipStream_t s) {
#define SPR_CORR(RK)                                                                          \
  correct_kernel<D, RK><<<grid, 256, 0, s>>>(a.perm_q, a.o_sp, a.corr_a, a.corr_psi_t, a.corr_c, \
                                             a.out, a.out_sh, a.out_st, a.n_q, a.rank, a.out_bf16)
  if (a.rank <= 16) SPR_CORR(16);
  else if (a.rank <= 32) SPR_CORR(32);
  else SPR_CORR(64);
#undef SPR_CORR
}

}  // namespace
}  // namespace spr

using namespace spr;

extern "C" int32_t sparsepr_correct(const sparsepr_dims* dims, int32_t m, int32_t rank,
                                    const int32_t* perm_q, const float* o_sp,
                                    const int32_t* probe_tokens, const float* o_probe_dense,
                                    const float* corr_a, const float* corr_psi_t,
                                    const float* corr_c, void* out, int32_t out_dtype,
                                    int64_t out_stride_head, int64_t out_stride_tok, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  (void)ws;
  (void)ws_bytes;
  int32_t st = check_dims(dims);
  if (st != SPARSEPR_OK) return st;
  if (m < 1 || m > SPARSEPR_MAX_PROBES || rank < 0 || rank > SPARSEPR_MAX_RANK)
    return SPARSEPR_ERR_INVALID;
  if (!perm_q || !o_sp || !probe_tokens || !o_probe_dense || !corr_a || !corr_psi_t || !corr_c ||
      !out)
    return SPARSEPR_ERR_INVALID;
  if (out_dtype != SPARSEPR_BF16 && out_dtype != SPARSEPR_F32) return SPARSEPR_ERR_UNSUPPORTED;
  const int64_t es = out_dtype == SPARSEPR_BF16 ? 2 : 4;
  if (((out_stride_head * es) & 15) || ((out_stride_tok * es) & 15) ||
      out_stride_tok < dims->head_dim || out_stride_head < 0)
    return SPARSEPR_ERR_INVALID;
  CorrArgs a;
  a.perm_q = perm_q;
  a.o_sp = o_sp;
  a.corr_a = corr_a;
  a.corr_psi_t = corr_psi_t;
  a.corr_c = corr_c;
  a.out = out;
  a.out_sh = out_stride_head;
  a.out_st = out_stride_tok;
  a.n_q = dims->n_q;
  a.rank = rank;
  a.out_bf16 = out_dtype == SPARSEPR_BF16;
  dim3 grid((dims->n_q + 255) / 256, dims->heads);
  if (dims->head_dim == 128) launch_correct<128>(a, grid, stream);
  else launch_correct<64>(a, grid, stream);
  SPR_LAUNCH_CHECK();
  probe_overwrite_kernel<<<dims->heads, 256, 0, stream>>>(probe_tokens, o_probe_dense, m,
                                                          dims->head_dim, out, out_stride_head,
                                                          out_stride_tok, a.out_bf16);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}
