// S9: corrected output in original token order.
//
// Review of the SparsePR paper, method summary step (5): unprobed rows get
// their sparse output plus the predicted residual, probe rows their exact
// dense output, and the result returns to the original order.  With the
// folded fit, out = o + (o A) Psi^T + c.
//
// HBM-bound: every block stages 64 group-major rows of O_sp through LDS with
// fully coalesced 16-byte loads, then 4 lanes share a row (D/4 dims each):
// u = o A is reduced across the 4 lanes, the row is rebuilt and written to
// its original token position.  A block walks several row tiles so the
// per-head A, Psi^T and c are loaded once per block.

#include "common.h"

namespace spr {
namespace {

constexpr int kRowsPerTile = 64;
constexpr int kTilesPerBlock = 8;

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
__global__ __launch_bounds__(256) void correct_kernel(CorrArgs a) {
  constexpr int DPL = D / 4;
  const int h = blockIdx.y, tid = threadIdx.x;
  __shared__ float sA[D][RK + 1];
  __shared__ float sP[RK][D + 4];
  __shared__ float sc[D];
  __shared__ float tile[kRowsPerTile][D + 4];
  const float* Ah = a.corr_a + (long long)h * D * a.rank;
  const float* Ph = a.corr_psi_t + (long long)h * a.rank * D;
  for (int e = tid; e < D * RK; e += 256) {
    const int i = e / RK, k = e % RK;
    sA[i][k] = k < a.rank ? Ah[i * a.rank + k] : 0.f;
  }
  for (int e = tid; e < RK * D; e += 256) {
    const int k = e / D, i = e % D;
    sP[k][i] = k < a.rank ? Ph[k * D + i] : 0.f;
  }
  for (int i = tid; i < D; i += 256) sc[i] = a.corr_c[(long long)h * D + i];
  const int r_in = tid >> 2, sl = tid & 3;
  for (int tt = 0; tt < kTilesPerBlock; ++tt) {
    const int row0 = (blockIdx.x * kTilesPerBlock + tt) * kRowsPerTile;
    if (row0 >= a.n_q) break;
    const int rows = min(kRowsPerTile, a.n_q - row0);
    __syncthreads();
    const float* src = a.o_sp + ((long long)h * a.n_q + row0) * D;
    for (int e = tid; e < rows * (D / 4); e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      *reinterpret_cast<float4*>(&tile[r][4 * c4]) =
          *reinterpret_cast<const float4*>(src + (long long)r * D + 4 * c4);
    }
    __syncthreads();
    if (r_in >= rows) continue;
    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] = tile[r_in][sl * DPL + i];
    float u[RK];
#pragma unroll
    for (int k = 0; k < RK; ++k) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < DPL; ++i) s = fmaf(o[i], sA[sl * DPL + i][k], s);
      s += __shfl_xor(s, 1);
      s += __shfl_xor(s, 2);
      u[k] = s;
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float s = o[i] + sc[sl * DPL + i];
#pragma unroll
      for (int k = 0; k < RK; ++k) s = fmaf(u[k], sP[k][sl * DPL + i], s);
      o[i] = s;
    }
    const int tok = a.perm_q[(long long)h * a.n_q + row0 + r_in];
    const long long base = (long long)h * a.out_sh + (long long)tok * a.out_st + sl * DPL;
    if (a.out_bf16) {
      uint16_t* dst = static_cast<uint16_t*>(a.out) + base;
#pragma unroll
      for (int i = 0; i < DPL; i += 8) {
        uint4 w;
        w.x = uint32_t(f32_to_bf16_rne(o[i + 0])) | (uint32_t(f32_to_bf16_rne(o[i + 1])) << 16);
        w.y = uint32_t(f32_to_bf16_rne(o[i + 2])) | (uint32_t(f32_to_bf16_rne(o[i + 3])) << 16);
        w.z = uint32_t(f32_to_bf16_rne(o[i + 4])) | (uint32_t(f32_to_bf16_rne(o[i + 5])) << 16);
        w.w = uint32_t(f32_to_bf16_rne(o[i + 6])) | (uint32_t(f32_to_bf16_rne(o[i + 7])) << 16);
        *reinterpret_cast<uint4*>(dst + i) = w;
      }
    } else {
      float* dst = static_cast<float*>(a.out) + base;
#pragma unroll
      for (int i = 0; i < DPL; i += 4)
        *reinterpret_cast<float4*>(dst + i) = make_float4(o[i], o[i + 1], o[i + 2], o[i + 3]);
    }
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
  if (a.rank <= 16) correct_kernel<D, 16><<<grid, 256, 0, s>>>(a);
  else if (a.rank <= 32) correct_kernel<D, 32><<<grid, 256, 0, s>>>(a);
  else correct_kernel<D, 64><<<grid, 256, 0, s>>>(a);
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
  const int per_block = kRowsPerTile * kTilesPerBlock;
  dim3 grid((dims->n_q + per_block - 1) / per_block, dims->heads);
  if (dims->head_dim == 128) launch_correct<128>(a, grid, stream);
  else launch_correct<64>(a, grid, stream);
  SPR_LAUNCH_CHECK();
  probe_overwrite_kernel<<<dims->heads, 256, 0, stream>>>(probe_tokens, o_probe_dense, m,
                                                          dims->head_dim, out, out_stride_head,
                                                          out_stride_tok, a.out_bf16);
  SPR_LAUNCH_CHECK();
  return SPARSEPR_OK;
}
