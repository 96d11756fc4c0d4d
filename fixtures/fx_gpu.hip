// Device fill of the seeded input generator (see fx_core.h), for tests and benchmarks that need
// gigabytes of synthetic weights resident in HBM.  Draws the same bits as fx_host.c.
// Build with -ffp-contract=off so the gain's multiply and add stay separately rounded.
#include <hip/hip_runtime.h>
#include "fx_core.h"

namespace {

__global__ void k_fill_normal_bf16(uint64_t key, uint64_t offset, uint64_t n, float sigma,
                                   uint16_t* __restrict__ out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = fx_normal_bf16(key, offset + i, sigma);
}

__global__ void k_fill_gain_bf16(uint64_t key, uint64_t n, float sigma, uint16_t* __restrict__ out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = fx_gain_bf16(key, i, sigma);
}

__global__ void k_fill_normal_f32(uint64_t key, uint64_t offset, uint64_t n, float* __restrict__ out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = fx_std_normal(key, offset + i);
}

__global__ void k_fill_tokens(uint64_t key, uint64_t n, uint32_t vocab, int32_t* __restrict__ out) {
  uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    out[i] = fx_token(key, i, vocab);
}

unsigned grid_for(uint64_t n) {
  uint64_t g = (n + 255) / 256;
  if (g > 16384) g = 16384;
  if (g == 0) g = 1;
  return (unsigned)g;
}

}  // namespace

extern "C" {

int fxg_fill_normal_bf16(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, float sigma,
                         uint16_t* out, hipStream_t s) {
  if (n == 0) return 0;
  k_fill_normal_bf16<<<grid_for(n), 256, 0, s>>>(fx_stream_key(seed, stream), offset, n, sigma, out);
  return (int)hipGetLastError();
}

int fxg_fill_gain_bf16(uint64_t seed, uint64_t stream, uint64_t n, float sigma, uint16_t* out,
                       hipStream_t s) {
  if (n == 0) return 0;
  k_fill_gain_bf16<<<grid_for(n), 256, 0, s>>>(fx_stream_key(seed, stream), n, sigma, out);
  return (int)hipGetLastError();
}

int fxg_fill_normal_f32(uint64_t seed, uint64_t stream, uint64_t offset, uint64_t n, float* out,
                        hipStream_t s) {
  if (n == 0) return 0;
  k_fill_normal_f32<<<grid_for(n), 256, 0, s>>>(fx_stream_key(seed, stream), offset, n, out);
  return (int)hipGetLastError();
}

int fxg_fill_tokens(uint64_t seed, uint64_t stream, uint64_t n, uint32_t vocab, int32_t* out,
                    hipStream_t s) {
  if (n == 0) return 0;
  k_fill_tokens<<<grid_for(n), 256, 0, s>>>(fx_stream_key(seed, stream), n, vocab, out);
  return (int)hipGetLastError();
}

}  // extern "C"
