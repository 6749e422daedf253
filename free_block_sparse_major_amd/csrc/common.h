// Internal helpers shared by the HIP sources of libsparsepr (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "sparsepr.h"

#define SPR_DEV __device__ __forceinline__

namespace spr {

constexpr int kWave = 64;

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bit level; bf16 values are carried as uint16_t)
// ---------------------------------------------------------------------------
SPR_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

SPR_DEV uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return uint16_t(0x7fc0);  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// ---------------------------------------------------------------------------
// wave / block reductions
// ---------------------------------------------------------------------------
template <typename T>
SPR_DEV T wave_sum(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T>
SPR_DEV T wave_max(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

template <typename T>
SPR_DEV T wave_min(T v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    T w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  return v;
}

// Block-wide sum; `red` must hold blockDim.x/64 entries.  All threads get the
// result.  Deterministic: waves are combined in a fixed order.
template <typename T>
SPR_DEV T block_sum(T v, T* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  T s = T(0);
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

template <typename T>
SPR_DEV T block_max(T v, T* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_max(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  T s = red[0];
  for (int i = 1; i < nw; ++i) s = red[i] > s ? red[i] : s;
  return s;
}

template <typename T>
SPR_DEV T block_min(T v, T* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = wave_min(v);
  __syncthreads();
  if (lane == 0) red[wid] = v;
  __syncthreads();
  T s = red[0];
  for (int i = 1; i < nw; ++i) s = red[i] < s ? red[i] : s;
  return s;
}

// Exclusive scan of one int64 value per thread over the block; returns the
// exclusive prefix, *total receives the block total.  `red` holds nw entries.
SPR_DEV long long block_exclusive_scan(long long v, long long* red, long long* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    long long y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[wid] = x;
  __syncthreads();
  long long base = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    if (i < wid) base += red[i];
    tot += red[i];
  }
  *total = tot;
  return base + x - v;
}

// ---------------------------------------------------------------------------
// workspace carving (host side)
// ---------------------------------------------------------------------------
struct Carver {
  char* base;
  size_t used;
  explicit Carver(void* p) : base(static_cast<char*>(p)), used(0) {}
  template <typename T>
  T* take(size_t count) {
    size_t off = (used + 255) & ~size_t(255);
    used = off + count * sizeof(T);
    return base ? reinterpret_cast<T*>(base + off) : nullptr;
  }
};

inline size_t elem_bytes(int dtype) { return dtype == SPARSEPR_BF16 ? 2 : 4; }

// Validates the shape; returns a status code.
int32_t check_dims(const sparsepr_dims* d);
// Output strides (elements of out_dtype) of a [H][N_q][d] output: 16-byte
// aligned rows, stride_tok >= d, stride_head >= 0, extent addressable with
// int64 offsets.  SPARSEPR_OK or SPARSEPR_ERR_INVALID.
int32_t check_out_strides(const sparsepr_dims* d, int32_t out_dtype, int64_t stride_head,
                          int64_t stride_tok);
// Probe rows take their dense output in the token-order output (S9).
int32_t launch_probe_overwrite(const sparsepr_dims* d, int m, const int32_t* tokens,
                               const float* dense, void* out, int out_bf16, int64_t sh,
                               int64_t st, hipStream_t stream);
// Workspace of sparsepr_sparse_attn_correct.
size_t attn_correct_ws_bytes(const sparsepr_dims* d, int rank);
// rows of q, k and v are read in 16-byte chunks: their base pointers must be
// 16-byte aligned (the strides are checked by check_dims)
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace spr

#define SPR_LAUNCH_CHECK()                          \
  do {                                              \
    if (hipGetLastError() != hipSuccess) return SPARSEPR_ERR_HIP; \
  } while (0)
