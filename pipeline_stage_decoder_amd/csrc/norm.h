// Row RMS scale shared by the RMSNorm kernel and the decode GEMV prologue, so both reduce in the
// same order: thread t sums x[4t .. 4t+4), x[4t+1024 ..) ... sequentially, then a 64-lane
// butterfly, then the four wave partials ((w0 + w1) + w2) + w3.
//
// The norm output is a bf16 GEMM operand: a 1-ulp difference before that rounding flips the bf16
// value, and one flipped element of h perturbs every output of the next projection enough to flip
// ~1% of the bf16 values rounded after it.  So the sum of squares, the scale and the product
// x * r * g are computed in f64 (a few f64 operations per element of one row) and rounded once to
// f32, then to bf16, which matches a float64 reference's rounding decisions.
#pragma once
#include "common.h"

PSD_DEV double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// r = 1 / sqrt(mean(x^2) + eps) of one row of K f32 values (K % 4 == 0), for a 256-thread block.
// `red` is 4 doubles of LDS.  Every thread returns r.
PSD_DEV double block_rms_scale(const float* __restrict__ x, int K, float eps, double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x * 4; i < K; i += 1024) {
    const float4 v = *(const float4*)(x + i);
    ss = fma((double)v.x, (double)v.x, ss);
    ss = fma((double)v.y, (double)v.y, ss);
    ss = fma((double)v.z, (double)v.z, ss);
    ss = fma((double)v.w, (double)v.w, ss);
  }
  ss = wave_sum_f64(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return 1.0 / sqrt(t / (double)K + (double)eps);
}

// (float)(x * r * g) with the product in f64
PSD_DEV float norm_mul(float x, double r, float g) { return (float)((double)x * r * (double)g); }
