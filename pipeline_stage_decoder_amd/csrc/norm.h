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

// Sum of squares of 4 values in f64, accumulated into ss in element order.
PSD_DEV double sumsq4(const float4& v, double ss) {
  ss = fma((double)v.x, (double)v.x, ss);
  ss = fma((double)v.y, (double)v.y, ss);
  ss = fma((double)v.z, (double)v.z, ss);
  return fma((double)v.w, (double)v.w, ss);
}

// r = 1 / sqrt(t / K + eps) from each thread's partial sum of squares (thread t holding
// x[4t .. 4t+4), x[4t+1024 ..) ...), for a 256-thread block.  `red` is 4 doubles of LDS.
PSD_DEV double block_rms_finish(double ss, int K, float eps, double* red) {
  ss = wave_sum_f64(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  const double t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return 1.0 / sqrt(t / (double)K + (double)eps);
}

// r = 1 / sqrt(mean(x^2) + eps) of one row of K f32 values (K % 4 == 0), for a 256-thread block.
// `red` is 4 doubles of LDS.  Every thread returns r.
PSD_DEV double block_rms_scale(const float* __restrict__ x, int K, float eps, double* red) {
  double ss = 0.0;
  for (int i = threadIdx.x * 4; i < K; i += 1024) ss = sumsq4(*(const float4*)(x + i), ss);
  return block_rms_finish(ss, K, eps, red);
}

// (float)(x * r * g) with the product in f64
PSD_DEV float norm_mul(float x, double r, float g) { return (float)((double)x * r * (double)g); }

// Normalised values x * r * g of elements i .. i+3 of a row, as three bf16 planes (hi, mid, lo) at
// p, p + ps, p + 2 ps (p points at element i of the row in the hi plane).
PSD_DEV void store_norm_planes4(uint16_t* p, size_t ps, const float4& v, double r, const float4& g) {
  const float y0 = norm_mul(v.x, r, g.x), y1 = norm_mul(v.y, r, g.y), y2 = norm_mul(v.z, r, g.z),
              y3 = norm_mul(v.w, r, g.w);
  uint32_t h[2], md[2], l[2];
  split3_pk(y0, y1, h[0], md[0], l[0]);
  split3_pk(y2, y3, h[1], md[1], l[1]);
  *(uint2*)p = make_uint2(h[0], h[1]);
  *(uint2*)(p + ps) = make_uint2(md[0], md[1]);
  *(uint2*)(p + 2 * ps) = make_uint2(l[0], l[1]);
}
