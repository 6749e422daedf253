// S9: corrected output in original token order.
//
// Review of the SparsePR paper, method summary step (5): unprobed rows get
// their sparse output plus the predicted residual, probe rows their exact
// dense output, and the result returns to the original order.  With the
// folded fit, out = o + (o A) Psi^T + c.
//
// HBM-bound: O_sp is read once and the output written once; the
// 2 * d * rank FMAs per row run from registers with A and Psi broadcast from
// LDS, loaded once per block of 4 waves x 4 row tiles.

#include "common.h"

namespace spr {
namespace {

constexpr int kRowsPerTile = 64;     // one row per lane of a wave
constexpr int kTilesPerWave = 4;
constexpr int kStagePitch = 36;      // floats per staged row (32 + 4: conflict-free 16B reads)

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

// Each wave owns 64-row tiles, one row per lane held in registers.  Rows
// move between HBM and registers through a per-wave LDS stage in 32-column
// slices: global accesses stay contiguous within each row, while a lane
// reads or writes its own row in LDS.  A and Psi are stored k-contiguous
// ([d][rank]) in LDS and read as broadcasts.  LDS traffic of one wave stays
// inside that wave, whose LDS operations complete in program order.
template <int D, int RK>
__global__ __launch_bounds__(256) void correct_kernel(CorrArgs a) {
  constexpr int NSL = D / 32;                // 32-column slices
  const int h = blockIdx.y, tid = threadIdx.x, wid = tid >> 6, lane = tid & 63;
  __shared__ float4 sA4[D * RK / 4];         // A[i][k]
  __shared__ float4 sP4[D * RK / 4];         // Psi^T transposed: P[i][k]
  __shared__ float sc[D];
  __shared__ float stage[4][kRowsPerTile * kStagePitch];
  float* sA = reinterpret_cast<float*>(sA4);
  float* sP = reinterpret_cast<float*>(sP4);
  const float* Ah = a.corr_a + (long long)h * D * a.rank;
  const float* Ph = a.corr_psi_t + (long long)h * a.rank * D;
  for (int e = tid; e < D * RK; e += 256) {
    const int i = e / RK, k = e % RK;
    sA[e] = k < a.rank ? Ah[i * a.rank + k] : 0.f;
    sP[e] = k < a.rank ? Ph[k * D + i] : 0.f;
  }
  for (int i = tid; i < D; i += 256) sc[i] = a.corr_c[(long long)h * D + i];
  __syncthreads();
  float* st = stage[wid];
  for (int tt = 0; tt < kTilesPerWave; ++tt) {
    const int row0 = ((blockIdx.x * 4 + wid) * kTilesPerWave + tt) * kRowsPerTile;
    if (row0 >= a.n_q) break;
    const int rows = min(kRowsPerTile, a.n_q - row0);
    const float* src = a.o_sp + ((long long)h * a.n_q + row0) * D;
    float o[D];
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
      // slice sl of the 64 rows: 8 16-byte chunks per row, contiguous per row
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int e = it * 64 + lane, r = e >> 3, c = e & 7;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (r < rows) v = *reinterpret_cast<const float4*>(src + (long long)r * D + 32 * sl + 4 * c);
        *reinterpret_cast<float4*>(st + r * kStagePitch + 4 * c) = v;
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float4 v = *reinterpret_cast<const float4*>(st + lane * kStagePitch + 4 * c);
        o[32 * sl + 4 * c + 0] = v.x;
        o[32 * sl + 4 * c + 1] = v.y;
        o[32 * sl + 4 * c + 2] = v.z;
        o[32 * sl + 4 * c + 3] = v.w;
      }
    }
    float u[RK];
#pragma unroll
    for (int k = 0; k < RK; ++k) u[k] = 0.f;
#pragma unroll 4
    for (int i = 0; i < D; ++i) {
#pragma unroll
      for (int k4 = 0; k4 < RK / 4; ++k4) {
        const float4 w = sA4[i * (RK / 4) + k4];
        u[4 * k4 + 0] = fmaf(o[i], w.x, u[4 * k4 + 0]);
        u[4 * k4 + 1] = fmaf(o[i], w.y, u[4 * k4 + 1]);
        u[4 * k4 + 2] = fmaf(o[i], w.z, u[4 * k4 + 2]);
        u[4 * k4 + 3] = fmaf(o[i], w.w, u[4 * k4 + 3]);
      }
    }
#pragma unroll 4
    for (int i = 0; i < D; ++i) {
      float v = o[i] + sc[i];
#pragma unroll
      for (int k4 = 0; k4 < RK / 4; ++k4) {
        const float4 w = sP4[i * (RK / 4) + k4];
        v = fmaf(u[4 * k4 + 0], w.x, v);
        v = fmaf(u[4 * k4 + 1], w.y, v);
        v = fmaf(u[4 * k4 + 2], w.z, v);
        v = fmaf(u[4 * k4 + 3], w.w, v);
      }
      o[i] = v;
    }
    // write back in original token order through the stage
    const int my_tok = lane < rows ? a.perm_q[(long long)h * a.n_q + row0 + lane] : 0;
#pragma unroll
    for (int sl = 0; sl < NSL; ++sl) {
#pragma unroll
      for (int c = 0; c < 8; ++c)
        *reinterpret_cast<float4*>(st + lane * kStagePitch + 4 * c) =
            make_float4(o[32 * sl + 4 * c], o[32 * sl + 4 * c + 1], o[32 * sl + 4 * c + 2],
                        o[32 * sl + 4 * c + 3]);
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int e = it * 64 + lane, r = e >> 3, c = e & 7;
        const int tok = __shfl(my_tok, r);
        const float4 v = *reinterpret_cast<const float4*>(st + r * kStagePitch + 4 * c);
        if (r >= rows) continue;
        const long long base = (long long)h * a.out_sh + (long long)tok * a.out_st + 32 * sl + 4 * c;
        if (a.out_bf16) {
          uint2 w;
          w.x = uint32_t(f32_to_bf16_rne(v.x)) | (uint32_t(f32_to_bf16_rne(v.y)) << 16);
          w.y = uint32_t(f32_to_bf16_rne(v.z)) | (uint32_t(f32_to_bf16_rne(v.w)) << 16);
          *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + base) = w;
        } else {
          *reinterpret_cast<float4*>(static_cast<float*>(a.out) + base) = v;
        }
      }
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
  const int per_block = kRowsPerTile * kTilesPerWave * 4;
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
