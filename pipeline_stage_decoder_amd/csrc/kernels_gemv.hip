// Decode GEMV for up to four rows: y[b, n] = sum_k x[b, k] W[n, k] with bf16 W streamed once.
//
// HBM-bound: every weight byte is read once per step.  A wave owns a pair of output rows
// (n, n + 16) -- a RoPE pair of the fused QKV layout or a gate/up pair of the interleaved MLP
// layout, so the epilogue finds both operands in the wave -- and streams the two rows along K with
// 16-byte loads (one 1 KiB contiguous segment per row per wave load), up to eight loads per row in
// flight.  f32 FMAs on bf16 operands, then a 64-lane butterfly reduces each sum.
// Fused prologue: the f32 input rows are RMS-normalised and scaled by the gain into LDS (f32) once
// per work-group, or an activation pair buffer is expanded to f32 (hi + lo); the grid is sized so
// each work-group covers many row pairs.
#include "kernels.h"
#include "norm.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGemvThreads = 256;
constexpr int kGemvUnrollDefault = 4;   // 16-byte loads per row per chunk (swept: 4 ~ 8 > 16)
constexpr int kGemvMaxGrid = 512;        // two work-groups per CU (swept: 512 beats 256 / 1024 / 2048)
constexpr int kGemvMaxLds = 64 * 1024;
constexpr int kGemv1Grid = 512;          // k_gemv1 work-groups at most (two per CU)

PSD_DEV void dot8(const uint4& w, const float4& x0, const float4& x1, float& acc) {
  acc = fmaf(bf_lo(w.x), x0.x, acc);
  acc = fmaf(bf_hi(w.x), x0.y, acc);
  acc = fmaf(bf_lo(w.y), x0.z, acc);
  acc = fmaf(bf_hi(w.y), x0.w, acc);
  acc = fmaf(bf_lo(w.z), x1.x, acc);
  acc = fmaf(bf_hi(w.z), x1.y, acc);
  acc = fmaf(bf_lo(w.w), x1.z, acc);
  acc = fmaf(bf_hi(w.w), x1.w, acc);
}

template <int NB, int EPI, int kGemvUnroll = kGemvUnrollDefault>
__global__ __launch_bounds__(kGemvThreads) void k_gemv(GemvArgs a) {
  extern __shared__ float4 lds_x[];                // NB rows of K f32 (operand values)
  __shared__ double red[4];
  const int K = a.K, K8 = K >> 3, B = a.B;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* xs = reinterpret_cast<float*>(lds_x);

  const int N = a.N;
  const int npairs = ((N + 31) >> 5) << 4;
  const int nwaves = gridDim.x * (kGemvThreads / 64);
  const int p_first = blockIdx.x * (kGemvThreads / 64) + wave;
  const int nchunks = (K8 + 64 * kGemvUnroll - 1) / (64 * kGemvUnroll);
  // weights of (pair pp, chunk cc), zero outside the matrix
  auto load_item = [&](int pp, int cc, uint4* d0, uint4* d1) {
    const int q0r = ((pp >> 4) << 5) + (pp & 15), q1r = q0r + 16;
    const bool ok0 = pp < npairs && q0r < N, ok1 = pp < npairs && q1r < N;
    const u32x4* w0 = reinterpret_cast<const u32x4*>(a.w + (size_t)(ok0 ? q0r : 0) * K);
    const u32x4* w1 = reinterpret_cast<const u32x4*>(a.w + (size_t)(ok1 ? q1r : 0) * K);
#pragma unroll
    for (int u = 0; u < kGemvUnroll; ++u) {
      const int idx = cc * 64 * kGemvUnroll + u * 64 + lane;
      const bool in = idx < K8;
      u32x4 t0 = {0, 0, 0, 0}, t1 = {0, 0, 0, 0};
      if (in && ok0) t0 = __builtin_nontemporal_load(w0 + idx);
      if (in && ok1) t1 = __builtin_nontemporal_load(w1 + idx);
      d0[u] = make_uint4(t0.x, t0.y, t0.z, t0.w);
      d1[u] = make_uint4(t1.x, t1.y, t1.z, t1.w);
    }
  };
  uint4 c0[kGemvUnroll], c1[kGemvUnroll];
  load_item(p_first, 0, c0, c1);

  // ---- prologue: input rows -> f32 operand values in LDS ---------------------------------------
  if (a.x) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < B) {
        const float* xr = a.x + (size_t)b * K;
        const double r = block_rms_scale(xr, K, a.eps, red);
        for (int i = threadIdx.x * 4; i < K; i += 1024) {
          const float4 v = *(const float4*)(xr + i);
          const float4 g = *(const float4*)(a.gain + i);
          *(float4*)(xs + (size_t)b * K + i) = make_float4(norm_mul(v.x, r, g.x), norm_mul(v.y, r, g.y),
                                                           norm_mul(v.z, r, g.z), norm_mul(v.w, r, g.w));
        }
      } else {
        for (int i = threadIdx.x * 4; i < K; i += 1024)
          *(float4*)(xs + (size_t)b * K + i) = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
  } else {
    for (int i = threadIdx.x * 4; i < NB * K; i += 1024) {
      float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i / K < B) {
        const uint2 h = *(const uint2*)(a.xb + i);
        const uint2 l = *(const uint2*)(a.xb + a.xb_ps + i);
        o = make_float4(bf_lo(h.x) + bf_lo(l.x), bf_hi(h.x) + bf_hi(l.x), bf_lo(h.y) + bf_lo(l.y),
                        bf_hi(h.y) + bf_hi(l.y));
      }
      *(float4*)(xs + i) = o;
    }
  }
  __syncthreads();

  // ---- row pairs -------------------------------------------------------------------------------
  // Work items are (pair, K chunk of 64 * kGemvUnroll 16-byte loads per row); the next item's
  // weights are loaded before the current one is consumed, and the first item's before the
  // prologue above, so the weight stream never waits on the norm or on a reduction.
  for (int p = p_first; p < npairs; p += nwaves) {
    float acc0[NB], acc1[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) acc0[b] = acc1[b] = 0.0f;
    const int r0 = ((p >> 4) << 5) + (p & 15), r1 = r0 + 16;
    const bool v0 = r0 < N, v1 = r1 < N;
    for (int c = 0; c < nchunks; ++c) {
      int pn = p, cn = c + 1;
      if (cn == nchunks) {
        pn = p + nwaves;
        cn = 0;
      }
      uint4 n0[kGemvUnroll], n1[kGemvUnroll];
      load_item(pn, cn, n0, n1);
      const int base = c * 64 * kGemvUnroll;
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u) {
        const int idx = base + u * 64 + lane;
        if (idx < K8) {
#pragma unroll
          for (int b = 0; b < NB; ++b) {
            const float4 xa = lds_x[(b * K8 + idx) * 2], xb = lds_x[(b * K8 + idx) * 2 + 1];
            dot8(c0[u], xa, xb, acc0[b]);
            dot8(c1[u], xa, xb, acc1[b]);
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kGemvUnroll; ++u) {
        c0[u] = n0[u];
        c1[u] = n1[u];
      }
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      acc0[b] = wave_sum(acc0[b]);
      acc1[b] = wave_sum(acc1[b]);
    }

    // ---- epilogue: lane b writes row b -------------------------------------------------------
    const EpiArgs& e = a.e;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if (b < B && lane == b) {
        const float x0 = acc0[b], x1 = acc1[b];
        switch (EPI) {
          case EPI_F32:
            if (v0) e.out[(size_t)b * e.ldo + r0] = x0;
            if (v1) e.out[(size_t)b * e.ldo + r1] = x1;
            break;
          case EPI_RESID:
            if (v0) e.out[(size_t)b * e.ldo + r0] = e.resid[(size_t)b * e.ldo + r0] + x0;
            if (v1) e.out[(size_t)b * e.ldo + r1] = e.resid[(size_t)b * e.ldo + r1] + x1;
            break;
          case EPI_SWIGLU:
            if (v1) store_pair(e.act, e.act_ps, (size_t)b * e.ldo + (p >> 4) * 16 + (p & 15), silu_mul(x0, x1));
            break;
          case EPI_QKV:
            if (v1) {
              int slot, pos;
              if (!row_slot_pos(e, b, slot, pos)) {
                if (r0 == 0) atomicAdd(e.err, 1u);
              } else {
                qkv_epilogue_pair(e, b, r0, x0, x1);
              }
            }
            break;
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------
// One row (B = 1), K a multiple of 2048: the work-group's 4 waves split K into quarters.  Each lane
// keeps its 8L input values (L = K / 2048) in registers -- no LDS copy of the input -- and every
// wave walks all of the work-group's P row pairs over its quarter, weights of the next D pairs in
// flight.  Per pair a wave reduces its lanes; the 4 quarter sums meet in LDS and are added in
// quarter order ((q0 + q1) + q2) + q3 before the epilogue.  The RMS scale comes from the same
// block_rms_scale as the row-norm kernel.
// ------------------------------------------------------------------------------------------------
template <int EPI, int L, int D>
__global__ __launch_bounds__(kGemvThreads) void k_gemv1(GemvArgs a, int P) {
  constexpr int kMaxP = 32;
  __shared__ float part[4][kMaxP][2];
  __shared__ double red[4];
  const int K = a.K, N = a.N;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int npairs = ((N + 31) >> 5) << 4;
  const int p0 = blockIdx.x * P;
  const int k0 = wave * (K >> 2);                 // this wave's quarter of K
  // weights of pair slot i (pair p0 + i): row r at k0 + (j * 64 + lane) * 8
  auto load_pair = [&](int i, u32x4 (&w0)[L], u32x4 (&w1)[L]) {
    const int pp = p0 + i;
    const int r0 = ((pp >> 4) << 5) + (pp & 15), r1 = r0 + 16;
    const bool ok0 = i < P && pp < npairs && r0 < N, ok1 = i < P && pp < npairs && r1 < N;
    const u32x4* q0 = reinterpret_cast<const u32x4*>(a.w + (size_t)(ok0 ? r0 : 0) * K + k0);
    const u32x4* q1 = reinterpret_cast<const u32x4*>(a.w + (size_t)(ok1 ? r1 : 0) * K + k0);
#pragma unroll
    for (int j = 0; j < L; ++j) {
      w0[j] = ok0 ? __builtin_nontemporal_load(q0 + j * 64 + lane) : u32x4{0, 0, 0, 0};
      w1[j] = ok1 ? __builtin_nontemporal_load(q1 + j * 64 + lane) : u32x4{0, 0, 0, 0};
    }
  };
  u32x4 wb0[D][L], wb1[D][L];
#pragma unroll
  for (int s = 0; s < D; ++s) load_pair(s, wb0[s], wb1[s]);

  // epilogue operands that do not depend on the sums (residual rows; the row's slot, position
  // and RoPE entry) load now, with the weights, rather than after the reduction: thread t < P
  // owns pair p0 + t
  const EpiArgs& e = a.e;
  const int t = threadIdx.x;
  const int p = p0 + t;
  const bool own = t < P && p < npairs;
  const int r0 = ((p >> 4) << 5) + (p & 15), r1 = r0 + 16;
  const bool v0 = own && r0 < N, v1 = own && r1 < N;
  float res0 = 0.0f, res1 = 0.0f;
  int slot = 0, pos = 0;
  bool row_ok = false;
  double2 cs = make_double2(1.0, 0.0);
  if (EPI == EPI_RESID) {
    if (v0) res0 = e.resid[r0];
    if (v1) res1 = e.resid[r1];
  }
  if (EPI == EPI_QKV && v1) {
    row_ok = row_slot_pos(e, 0, slot, pos);
    if (row_ok) cs = qkv_rope_cs(e, pos, r0);
  }

  // ---- input quarter -> registers (normalised f32, or the pair buffer expanded) -----------------
  float x[L][8];
  if (a.x) {
    const double r = block_rms_scale(a.x, K, a.eps, red);
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int k = k0 + (j * 64 + lane) * 8;
      const float4 v0 = *(const float4*)(a.x + k), v1 = *(const float4*)(a.x + k + 4);
      const float4 g0 = *(const float4*)(a.gain + k), g1 = *(const float4*)(a.gain + k + 4);
      x[j][0] = norm_mul(v0.x, r, g0.x); x[j][1] = norm_mul(v0.y, r, g0.y);
      x[j][2] = norm_mul(v0.z, r, g0.z); x[j][3] = norm_mul(v0.w, r, g0.w);
      x[j][4] = norm_mul(v1.x, r, g1.x); x[j][5] = norm_mul(v1.y, r, g1.y);
      x[j][6] = norm_mul(v1.z, r, g1.z); x[j][7] = norm_mul(v1.w, r, g1.w);
    }
  } else {
#pragma unroll
    for (int j = 0; j < L; ++j) {
      const int k = k0 + (j * 64 + lane) * 8;
      const uint4 h = *(const uint4*)(a.xb + k), l = *(const uint4*)(a.xb + a.xb_ps + k);
      const uint32_t hh[4] = {h.x, h.y, h.z, h.w}, ll[4] = {l.x, l.y, l.z, l.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[j][2 * e] = bf_lo(hh[e]) + bf_lo(ll[e]);
        x[j][2 * e + 1] = bf_hi(hh[e]) + bf_hi(ll[e]);
      }
    }
  }

  // ---- the work-group's pairs, D in flight --------------------------------------------------------
  for (int i0 = 0; i0 < P; i0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int i = i0 + s;
      if (i < P) {
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int j = 0; j < L; ++j) {
          const float4 xa = make_float4(x[j][0], x[j][1], x[j][2], x[j][3]);
          const float4 xc = make_float4(x[j][4], x[j][5], x[j][6], x[j][7]);
          const uint4 u0 = make_uint4(wb0[s][j].x, wb0[s][j].y, wb0[s][j].z, wb0[s][j].w);
          const uint4 u1 = make_uint4(wb1[s][j].x, wb1[s][j].y, wb1[s][j].z, wb1[s][j].w);
          dot8(u0, xa, xc, acc0);
          dot8(u1, xa, xc, acc1);
        }
        load_pair(i + D, wb0[s], wb1[s]);
        acc0 = wave_sum(acc0);
        acc1 = wave_sum(acc1);
        if (lane == 0) {
          part[wave][i][0] = acc0;
          part[wave][i][1] = acc1;
        }
      }
    }
  }
  __syncthreads();

  // ---- quarter sums in order, epilogue -------------------------------------------------------------
  if (!own) return;
  const float x0 = ((part[0][t][0] + part[1][t][0]) + part[2][t][0]) + part[3][t][0];
  const float x1 = ((part[0][t][1] + part[1][t][1]) + part[2][t][1]) + part[3][t][1];
  switch (EPI) {
    case EPI_F32:
      if (v0) e.out[r0] = x0;
      if (v1) e.out[r1] = x1;
      break;
    case EPI_RESID:
      if (v0) e.out[r0] = res0 + x0;
      if (v1) e.out[r1] = res1 + x1;
      break;
    case EPI_SWIGLU:
      if (v1) store_pair(e.act, e.act_ps, (size_t)(p >> 4) * 16 + (p & 15), silu_mul(x0, x1));
      break;
    case EPI_QKV:
      if (v1) {
        if (!row_ok) {
          if (r0 == 0) atomicAdd(e.err, 1u);
        } else {
          qkv_store_pair(e, 0, slot, pos, r0, x0, x1, cs);
        }
      }
      break;
  }
}

template <int EPI, int L, int D>
void launch_one(const GemvArgs& a, hipStream_t s) {
  const int npairs = ((a.N + 31) >> 5) << 4;
  const int P = (npairs + kGemv1Grid - 1) / kGemv1Grid;
  const int grid = (npairs + P - 1) / P;
  k_gemv1<EPI, L, D><<<grid, kGemvThreads, 0, s>>>(a, P);
}

template <int EPI>
void launch_one_l(const GemvArgs& a, hipStream_t s) {
  switch (a.K / 2048) {
    case 2: launch_one<EPI, 2, 2>(a, s); break;
    case 4: launch_one<EPI, 4, 2>(a, s); break;
    default: launch_one<EPI, 7, 2>(a, s); break;
  }
}

template <int EPI>
void launch_nb(const GemvArgs& a, int nb, int grid, size_t lds, hipStream_t s) {
  switch (nb) {
    case 1: k_gemv<1, EPI><<<grid, kGemvThreads, lds, s>>>(a); break;
    case 2: k_gemv<2, EPI><<<grid, kGemvThreads, lds, s>>>(a); break;
    default: k_gemv<4, EPI><<<grid, kGemvThreads, lds, s>>>(a); break;
  }
}

}  // namespace

bool gemv_fits(int B, int K) {
  const int nb = B <= 1 ? 1 : (B <= 2 ? 2 : 4);
  return B >= 1 && B <= 4 && (size_t)nb * K * 4 <= (size_t)kGemvMaxLds && K % 8 == 0;
}

// the K-split single-row kernel's shapes: K = 4096, 8192 or 14336, at most 32 row pairs per
// work-group at the maximum grid
bool gemv1_fits(int B, int K, int N) {
  const int L = K / 2048;
  const int npairs = ((N + 31) >> 5) << 4;
  return B == 1 && K % 2048 == 0 && (L == 2 || L == 4 || L == 7) && (npairs + kGemv1Grid - 1) / kGemv1Grid <= 32;
}

hipError_t launch_gemv(const GemvArgs& a, hipStream_t s) {
  if (a.e.kind == EPI_QKV && a.e.col_off != 0) return hipErrorInvalidValue;   // whole fused weight only
  if (gemv1_fits(a.B, a.K, a.N)) {
    switch (a.e.kind) {
      case EPI_F32: launch_one_l<EPI_F32>(a, s); break;
      case EPI_RESID: launch_one_l<EPI_RESID>(a, s); break;
      case EPI_SWIGLU: launch_one_l<EPI_SWIGLU>(a, s); break;
      default: launch_one_l<EPI_QKV>(a, s); break;
    }
    return hipGetLastError();
  }
  const int npairs = ((a.N + 31) >> 5) << 4;
  int grid = (npairs + 3) / 4;
  if (grid > kGemvMaxGrid) grid = kGemvMaxGrid;
  const int nb = a.B <= 1 ? 1 : (a.B <= 2 ? 2 : 4);
  const size_t lds = (size_t)nb * a.K * 4;
  switch (a.e.kind) {
    case EPI_F32: launch_nb<EPI_F32>(a, nb, grid, lds, s); break;
    case EPI_RESID: launch_nb<EPI_RESID>(a, nb, grid, lds, s); break;
    case EPI_SWIGLU: launch_nb<EPI_SWIGLU>(a, nb, grid, lds, s); break;
    default: launch_nb<EPI_QKV>(a, nb, grid, lds, s); break;
  }
  return hipGetLastError();
}
