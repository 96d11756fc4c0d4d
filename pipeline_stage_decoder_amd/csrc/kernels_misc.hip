// RMSNorm rows, token embedding, KV import/export and small conversions.
#include "kernels.h"
#include "norm.h"

namespace {

__global__ __launch_bounds__(256) void k_rmsnorm(NormArgs a) {
  __shared__ double red[4];
  const int m = blockIdx.x;
  const float* x = a.x + (size_t)m * a.K;
  const double r = block_rms_scale(x, a.K, a.eps, red);
  for (int i = threadIdx.x * 4; i < a.K; i += 1024) {
    const float4 v = *(const float4*)(x + i);
    const float4 g = *(const float4*)(a.gain + i);
    if (a.out_f32)
      *(float4*)(a.out_f32 + (size_t)m * a.K + i) =
          make_float4(norm_mul(v.x, r, g.x), norm_mul(v.y, r, g.y), norm_mul(v.z, r, g.z), norm_mul(v.w, r, g.w));
    if (a.out_pair) store_norm_planes4(a.out_pair + (size_t)m * a.K + i, a.pair_ps, v, r, g);
  }
}

// The same for rows of exactly PER * 1024 values: each thread loads its PER float4 (and gains) at
// once instead of one per loop trip, then sums their squares in the same order as
// block_rms_scale (i = 4 t + 1024 j, j ascending), so the scale and every output bit are equal.
template <int PER>
__global__ __launch_bounds__(256) void k_rmsnorm_rows(NormArgs a) {
  __shared__ double red[4];
  const int m = blockIdx.x;
  const float* x = a.x + (size_t)m * a.K;
  float4 v[PER], g[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    v[j] = *(const float4*)(x + threadIdx.x * 4 + j * 1024);
    g[j] = *(const float4*)(a.gain + threadIdx.x * 4 + j * 1024);
  }
  double ss = 0.0;
#pragma unroll
  for (int j = 0; j < PER; ++j) ss = sumsq4(v[j], ss);
  const double r = block_rms_finish(ss, a.K, a.eps, red);
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = threadIdx.x * 4 + j * 1024;
    if (a.out_f32)
      *(float4*)(a.out_f32 + (size_t)m * a.K + i) = make_float4(
          norm_mul(v[j].x, r, g[j].x), norm_mul(v[j].y, r, g[j].y), norm_mul(v[j].z, r, g[j].z), norm_mul(v[j].w, r, g[j].w));
    if (a.out_pair) store_norm_planes4(a.out_pair + (size_t)m * a.K + i, a.pair_ps, v[j], r, g[j]);
  }
}

__global__ __launch_bounds__(256) void k_embed(const uint16_t* __restrict__ table, int V, int d,
                                               const int32_t* __restrict__ tokens, float* __restrict__ out,
                                               uint32_t* err) {
  const int i = blockIdx.x;
  const int tok = tokens[i];
  float* o = out + (size_t)i * d;
  if (tok < 0 || tok >= V) {
    for (int j = threadIdx.x; j < d; j += 256) o[j] = 0.0f;
    if (threadIdx.x == 0) atomicAdd(err, 1u);
    return;
  }
  const uint16_t* e = table + (size_t)tok * d;
  for (int j = threadIdx.x * 4; j < d; j += 1024) {
    const uint2 w = *(const uint2*)(e + j);
    *(float4*)(o + j) = make_float4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y));
  }
}

// Embedding rows of a vocabulary slice: the table holds ids [lo, lo + V); other ids contribute a
// zero row.  out = (accumulate ? out : 0) + row, one F32 add per element.  Negative ids are errors.
__global__ __launch_bounds__(256) void k_embed_range(const uint16_t* __restrict__ table, int V, int d, int lo,
                                                     const int32_t* __restrict__ tokens, float* __restrict__ out,
                                                     int accumulate, uint32_t* err) {
  const int i = blockIdx.x;
  const int tok = tokens[i];
  float* o = out + (size_t)i * d;
  if (tok < 0 && threadIdx.x == 0) atomicAdd(err, 1u);
  const bool inside = tok >= lo && tok - lo < V;
  const uint16_t* e = table + (size_t)(inside ? tok - lo : 0) * d;
  for (int j = threadIdx.x * 4; j < d; j += 1024) {
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    if (inside) {
      const uint2 w = *(const uint2*)(e + j);
      r = make_float4(bf_lo(w.x), bf_hi(w.x), bf_lo(w.y), bf_hi(w.y));
    }
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    if (accumulate) a = *(const float4*)(o + j);
    *(float4*)(o + j) = make_float4(a.x + r.x, a.y + r.y, a.z + r.z, a.w + r.w);
  }
}

__global__ void k_bf16_to_f32(const uint16_t* __restrict__ src, float* __restrict__ dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf2f(src[i]);
}

__global__ void k_zero_f32(float* __restrict__ p, size_t n) {
  size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0.0f;
}

// K cache [slot][kvh][ctx_cap][Dh]; V cache [slot][kvh][ctx_cap/8][Dh][8]; element type T.
template <typename T>
__global__ void k_kv_import(T* kc, T* vc, int hkv, int dh, int ctx_cap, int slot, int pos0,
                            const T* __restrict__ k, const T* __restrict__ v) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int pos = pos0 + t;
  const size_t src = ((size_t)t * hkv + h) * dh + d;
  kc[(((size_t)slot * hkv + h) * ctx_cap + pos) * dh + d] = k[src];
  vc[((((size_t)slot * hkv + h) * (ctx_cap >> 3) + (pos >> 3)) * dh + d) * 8 + (pos & 7)] = v[src];
}

template <typename T>
__global__ void k_kv_export(const T* kc, const T* vc, int hkv, int dh, int ctx_cap, int slot, int pos0,
                            T* __restrict__ k, T* __restrict__ v) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int pos = pos0 + t;
  const size_t dst = ((size_t)t * hkv + h) * dh + d;
  k[dst] = kc[(((size_t)slot * hkv + h) * ctx_cap + pos) * dh + d];
  v[dst] = vc[((((size_t)slot * hkv + h) * (ctx_cap >> 3) + (pos >> 3)) * dh + d) * 8 + (pos & 7)];
}

// The F32-grade cache: element d of a K row (V 8-key group) is hi + lo, the row's (group's) bf16 hi
// plane followed by its lo plane.  Import splits F32 values the way the QKV epilogue does; export
// returns hi + lo (exact in F32).
__global__ void k_kv_import_pair(uint16_t* kc, uint16_t* vc, int hkv, int dh, int ctx_cap, int slot, int pos0,
                                 const float* __restrict__ k, const float* __restrict__ v) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int pos = pos0 + t;
  const size_t src = ((size_t)t * hkv + h) * dh + d;
  const size_t kr = (((size_t)slot * hkv + h) * ctx_cap + pos) * 2 * dh;
  const size_t vg = (((size_t)slot * hkv + h) * (ctx_cap >> 3) + (pos >> 3)) * 2 * dh * 8 + (size_t)d * 8 + (pos & 7);
  uint32_t hi, lo;
  split2(k[src], hi, lo);
  kc[kr + d] = (uint16_t)hi;
  kc[kr + dh + d] = (uint16_t)lo;
  split2(v[src], hi, lo);
  vc[vg] = (uint16_t)hi;
  vc[vg + (size_t)dh * 8] = (uint16_t)lo;
}

__global__ void k_kv_export_pair(const uint16_t* kc, const uint16_t* vc, int hkv, int dh, int ctx_cap, int slot,
                                 int pos0, float* __restrict__ k, float* __restrict__ v) {
  const int t = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int pos = pos0 + t;
  const size_t dst = ((size_t)t * hkv + h) * dh + d;
  const size_t kr = (((size_t)slot * hkv + h) * ctx_cap + pos) * 2 * dh;
  const size_t vg = (((size_t)slot * hkv + h) * (ctx_cap >> 3) + (pos >> 3)) * 2 * dh * 8 + (size_t)d * 8 + (pos & 7);
  k[dst] = bf2f(kc[kr + d]) + bf2f(kc[kr + dh + d]);
  v[dst] = bf2f(vc[vg]) + bf2f(vc[vg + (size_t)dh * 8]);
}

// Greedy choice per row: the largest logit, the lowest index among equal ones.  Each thread scans
// a strided subset in ascending index order (a strict > keeps its first maximum), then the
// (value, index) pairs reduce with the same rule.  NaN compares false and never wins.
__global__ __launch_bounds__(256) void k_argmax(const float* __restrict__ logits, int V, int32_t* __restrict__ out) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const float* row = logits + (size_t)blockIdx.x * V;
  float best = -__builtin_huge_valf();
  int bi = 0x7fffffff;
  for (int i = threadIdx.x; i < V; i += 256) {
    const float v = row[i];
    if (v > best) {
      best = v;
      bi = i;
    }
  }
  auto better = [](float v, int i, float bv, int bidx) { return v > bv || (v == bv && i < bidx); };
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const float v = __shfl_xor(best, o, 64);
    const int i = __shfl_xor(bi, o, 64);
    if (better(v, i, best, bi)) {
      best = v;
      bi = i;
    }
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    sv[wave] = best;
    si[wave] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < 4; ++w)
      if (better(sv[w], si[w], best, bi)) {
        best = sv[w];
        bi = si[w];
      }
    out[blockIdx.x] = bi == 0x7fffffff ? 0 : bi;
  }
}

}  // namespace

hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t s) {
  if (a.M <= 0) return hipSuccess;
  if (a.K == 4096) k_rmsnorm_rows<4><<<a.M, 256, 0, s>>>(a);
  else if (a.K == 8192) k_rmsnorm_rows<8><<<a.M, 256, 0, s>>>(a);
  else k_rmsnorm<<<a.M, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_embed(const uint16_t* table, int V, int d, const int32_t* tokens, int n, float* out,
                        uint32_t* err, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_embed<<<n, 256, 0, s>>>(table, V, d, tokens, out, err);
  return hipGetLastError();
}

hipError_t launch_embed_range(const uint16_t* table, int V, int d, int lo, const int32_t* tokens, int n, float* out,
                              int accumulate, uint32_t* err, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_embed_range<<<n, 256, 0, s>>>(table, V, d, lo, tokens, out, accumulate, err);
  return hipGetLastError();
}

hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  k_bf16_to_f32<<<(n + 255) / 256, 256, 0, s>>>(src, dst, n);
  return hipGetLastError();
}

hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  size_t g = (n + 255) / 256;
  if (g > 4096) g = 4096;
  k_zero_f32<<<(unsigned)g, 256, 0, s>>>(p, n);
  return hipGetLastError();
}

hipError_t launch_kv_import(void* kc, void* vc, int kv_f32, int hkv, int dh, int ctx_cap, int slot, int pos0,
                            int n, const void* k, const void* v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (kv_f32)
    k_kv_import_pair<<<dim3(n, hkv), dh, 0, s>>>(static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), hkv, dh,
                                                 ctx_cap, slot, pos0, static_cast<const float*>(k),
                                                 static_cast<const float*>(v));
  else
    k_kv_import<uint16_t><<<dim3(n, hkv), dh, 0, s>>>(static_cast<uint16_t*>(kc), static_cast<uint16_t*>(vc), hkv,
                                                      dh, ctx_cap, slot, pos0, static_cast<const uint16_t*>(k),
                                                      static_cast<const uint16_t*>(v));
  return hipGetLastError();
}

hipError_t launch_kv_export(const void* kc, const void* vc, int kv_f32, int hkv, int dh, int ctx_cap, int slot,
                            int pos0, int n, void* k, void* v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (kv_f32)
    k_kv_export_pair<<<dim3(n, hkv), dh, 0, s>>>(static_cast<const uint16_t*>(kc), static_cast<const uint16_t*>(vc),
                                                 hkv, dh, ctx_cap, slot, pos0, static_cast<float*>(k),
                                                 static_cast<float*>(v));
  else
    k_kv_export<uint16_t><<<dim3(n, hkv), dh, 0, s>>>(static_cast<const uint16_t*>(kc),
                                                      static_cast<const uint16_t*>(vc), hkv, dh, ctx_cap, slot, pos0,
                                                      static_cast<uint16_t*>(k), static_cast<uint16_t*>(v));
  return hipGetLastError();
}

hipError_t launch_argmax(const float* logits, int n, int V, int32_t* out, hipStream_t s) {
  k_argmax<<<n, 256, 0, s>>>(logits, V, out);
  return hipGetLastError();
}
