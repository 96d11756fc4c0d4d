// Shared device helpers and launch-argument structs of the stage kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

#define PSD_DEV __device__ __forceinline__

// bf16 <-> f32 on raw bits.  f32 -> bf16 rounds to nearest, ties to even, on gfx950's packed
// conversion (v_cvt_pk_bf16_f32, two values per instruction): for every finite f32 it gives the
// bits (u + 0x7FFF + ((u >> 16) & 1)) >> 16 of the rounding written out on the integer bits
// (checked over all 2^32 patterns on MI355X).  Inputs are finite.
PSD_DEV float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }
PSD_DEV float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
PSD_DEV float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
PSD_DEV uint32_t pack_bf2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
PSD_DEV uint32_t f2bf(float f) { return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)f); }

PSD_DEV bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// IEEE binary16 on raw bits: f32 -> f16 rounds to nearest, ties to even (the hardware conversion
// in the default rounding mode); f16 -> f32 is exact.
PSD_DEV uint32_t pack_f16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
PSD_DEV float h_lo(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu)); }
PSD_DEV float h_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16)); }
PSD_DEV f16x8_t as_f16x8(uint4 v) { return __builtin_bit_cast(f16x8_t, v); }

PSD_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
PSD_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// 16x16x32 bf16 MFMA, f32 accumulate.  Lane l holds A[row l%16][k (l/16)*8 .. +8],
// B[k (l/16)*8 .. +8][col l%16]; C: lane l holds C[rows (l/16)*4 .. +4][col l%16].
PSD_DEV f32x4_t mfma16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// The same shape on binary16 operands (the F16 KV cache's attention products).
PSD_DEV f32x4_t mfma16(f16x8_t a, f16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Activations are carried as a pair of bf16 planes, hi = bf16(x) and lo = bf16(x - hi), so the
// effective operand hi + lo keeps ~16 significant bits and every MFMA product with a bf16 weight
// is taken twice (hi and lo).  A "pair buffer" is one pointer p with a plane stride ps: hi at
// p[i], lo at p[ps + i].
PSD_DEV void split2(float x, uint32_t& hi, uint32_t& lo) {
  hi = f2bf(x);
  lo = f2bf(x - bf2f(hi));
}
PSD_DEV float pair_value(uint32_t hi, uint32_t lo) { return bf2f(hi) + bf2f(lo); }
// Three planes (hi, mid, lo) carry ~24 significant bits: used for the operand of the projection
// whose outputs are rounded again (K and V go to the bf16 cache), so that rounding sees f32-grade
// values.  The first two planes equal the pair split.
PSD_DEV void split3(float x, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = f2bf(x);
  const float r = x - bf2f(hi);
  mid = f2bf(r);
  lo = f2bf(r - bf2f(mid));
}
// the same three planes of two values, packed as bf16 pairs
PSD_DEV void split3_pk(float x0, float x1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = pack_bf2(x0, x1);
  const float r0 = x0 - bf_lo(hi), r1 = x1 - bf_hi(hi);
  mid = pack_bf2(r0, r1);
  lo = pack_bf2(r0 - bf_lo(mid), r1 - bf_hi(mid));
}

// hi and lo planes of two values packed as bf16 pairs (the same split as split2, two at a time)
PSD_DEV void split2_pk(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf2(x0, x1);
  lo = pack_bf2(x0 - bf_lo(hi), x1 - bf_hi(hi));
}

// hi and lo binary16 planes of two values packed as f16 pairs: hi = f16(x), lo = f16(x - hi), so
// hi + lo keeps ~22 significant bits for values in binary16's normal range.
PSD_DEV void split2_pk_f16(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  hi = pack_f16x2(x0, x1);
  lo = pack_f16x2(x0 - h_lo(hi), x1 - h_hi(hi));
}

// Split an f32 x8 vector into binary16 hi + lo planes.
PSD_DEV void split_hi_lo_f16(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2_pk_f16(x[2 * i], x[2 * i + 1], h[i], l[i]);
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// Split an f32 x8 vector into bf16 hi + bf16 lo (x ~= hi + lo to ~2^-16 relative).
PSD_DEV void split_hi_lo(const float* x, uint4& hi, uint4& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2_pk(x[2 * i], x[2 * i + 1], h[i], l[i]);
  hi = make_uint4(h[0], h[1], h[2], h[3]);
  lo = make_uint4(l[0], l[1], l[2], l[3]);
}

// ------------------------------------------------------------------------------------------------
// Epilogue kinds shared by the decode GEMV and the MFMA GEMM.
// ------------------------------------------------------------------------------------------------
enum EpiKind {
  EPI_F32 = 0,      // out[m, n] = acc                          (readout logits, MLP partial)
  EPI_RESID = 1,    // out[m, n] = resid[m, n] + acc            (O-proj, down-proj)
  EPI_SWIGLU = 2,   // act[m, f] = bf16(silu(gate) * up)        (rows interleaved by 16)
  EPI_QKV = 3       // RoPE on q/k, q -> plane buffer, k/v -> KV cache
};

// KV cache element formats.  KV_BF16: one bf16 per value.  KV_F32: an F32-grade pair, each value
// kept as a bf16 hi plane and a bf16 lo plane (4 bytes).  KV_F16: one IEEE binary16 per value;
// its attention runs on f16 MFMAs, so q and the softmax probabilities are carried as binary16
// hi + lo planes there (the other formats carry them as bf16 planes).
enum KvFmt { KV_BF16 = 0, KV_F32 = 1, KV_F16 = 2 };

// Where each output row's token sits: slot and absolute position.
struct RowPos {
  const int32_t* slots;  // device [M] or null (then every row is `slot`)
  const int32_t* pos;    // device [M] or null (then row m is at pos0 + m)
  int slot, pos0;
};

struct EpiArgs {
  int kind;
  int ldo;                     // leading dim of out / resid / act (elements)
  float* out;                  // EPI_F32 / EPI_RESID
  const float* resid;          // EPI_RESID (may alias out)
  uint16_t* act;               // EPI_SWIGLU: pair buffer [M, F]
  size_t act_ps;
  // EPI_QKV
  uint16_t* q;                 // pair buffer [M, Hq*Dh], natural head-dim order
  size_t q_ps;
  void* kc;                    // K cache of this block: [slots][Hkv][ctx_cap][Dh]
  void* vc;                    // V cache of this block: [slots][Hkv][ctx_cap/8][Dh][8]
  int kv_fmt;                  // KvFmt.  KV_F32: each K row / V 8-key group holds a bf16 hi plane
                               // and then a lo plane (4 bytes per element); KV_F16 also stores
                               // q as binary16 planes
  const double2* rope;         // [ctx_cap][Dh/2] (cos, sin), f64
  int col_off;                 // fused-QKV stored row of output column 0: a GEMM over a row range of
                               // the fused weight (a multiple of 32; GEMM paths only, 0 for GEMVs)
  RowPos rp;
  int hq, hkv, dh, ctx_cap, max_slots;
  uint32_t* err;               // device error counter
};

// Fused-QKV row layout: within each q and k head, stored rows come in 32-row blocks whose first
// 16 rows are head dims [16b, 16b+16) and next 16 rows are dims [Dh/2 + 16b, Dh/2 + 16b + 16), so
// a stored row r with (r % 32) < 16 and row r + 16 are a RoPE pair (i, i + Dh/2).  V rows keep
// their natural order.  Gate/up are interleaved the same way: stored rows [32j, 32j+16) are gate
// rows [16j, 16j+16) and [32j+16, 32j+32) the matching up rows.
PSD_DEV int rope_pair_dim(int s /* stored row within head, s % 32 < 16 */) {
  return (s >> 5) * 16 + (s & 15);
}

// Resolve the slot and position of row m; false if out of range (then the row is skipped).
PSD_DEV bool row_slot_pos(const EpiArgs& e, int m, int& slot, int& pos) {
  slot = e.rp.slots ? e.rp.slots[m] : e.rp.slot;
  pos = e.rp.pos ? e.rp.pos[m] : e.rp.pos0 + m;
  return slot >= 0 && slot < e.max_slots && pos >= 0 && pos < e.ctx_cap;
}

// RoPE (cos, sin) of a stored QKV row pair at position pos: the table entry for q and k rows,
// unused (1, 0) for V rows.  col0 is the stored row index of the pair's first element.
PSD_DEV double2 qkv_rope_cs(const EpiArgs& e, int pos, int col0) {
  const int dh = e.dh, qk = (e.hq + e.hkv) * dh;
  if (col0 >= qk) return make_double2(1.0, 0.0);
  const int c = col0 < e.hq * dh ? col0 : col0 - e.hq * dh;
  const int s = c - (c / dh) * dh;
  return e.rope[(size_t)pos * (dh >> 1) + rope_pair_dim(s)];
}

// Store one RoPE pair / V pair of outputs of row m (slot and position valid): x0/x1 are the sums
// of stored rows col0 and col0 + 16 (col0 % 32 < 16), cs = qkv_rope_cs(e, pos, col0).
PSD_DEV void qkv_store_pair(const EpiArgs& e, int m, int slot, int pos, int col0, float x0, float x1,
                            double2 cs) {
  const int dh = e.dh, qw = e.hq * dh, kw = e.hkv * dh;
  if (col0 < qw + kw) {
    const bool is_q = col0 < qw;
    const int c = is_q ? col0 : col0 - qw;
    const int head = c / dh, s = c - head * dh;
    const int i = rope_pair_dim(s);
    // rotation in f64 from an f64 table, rounded once to f32 and then to the stored format
    const float y0 = (float)((double)x0 * cs.x - (double)x1 * cs.y);
    const float y1 = (float)((double)x1 * cs.x + (double)x0 * cs.y);
    if (is_q) {
      uint16_t* dst = e.q + (size_t)m * qw + head * dh;
      uint32_t h, l;
      if (e.kv_fmt == KV_F16) split2_pk_f16(y0, y1, h, l);
      else split2_pk(y0, y1, h, l);
      dst[i] = (uint16_t)h;
      dst[i + (dh >> 1)] = (uint16_t)(h >> 16);
      dst[e.q_ps + i] = (uint16_t)l;
      dst[e.q_ps + i + (dh >> 1)] = (uint16_t)(l >> 16);
    } else {
      const size_t o = (((size_t)slot * e.hkv + head) * e.ctx_cap + pos) * dh;
      if (e.kv_fmt == KV_F32) {
        // F32-grade cache: the key row holds the bf16 hi plane [Dh], then the lo plane [Dh]
        uint16_t* dst = static_cast<uint16_t*>(e.kc) + 2 * o;
        uint32_t h, l;
        split2_pk(y0, y1, h, l);
        dst[i] = (uint16_t)h;
        dst[i + (dh >> 1)] = (uint16_t)(h >> 16);
        dst[dh + i] = (uint16_t)l;
        dst[dh + i + (dh >> 1)] = (uint16_t)(l >> 16);
      } else {
        uint16_t* dst = static_cast<uint16_t*>(e.kc) + o;
        const uint32_t h = e.kv_fmt == KV_F16 ? pack_f16x2(y0, y1) : pack_bf2(y0, y1);
        dst[i] = (uint16_t)h;
        dst[i + (dh >> 1)] = (uint16_t)(h >> 16);
      }
    }
  } else {
    const int c = col0 - qw - kw;
    const int head = c / dh, d0 = c - head * dh;
    const size_t o = (((size_t)slot * e.hkv + head) * (e.ctx_cap >> 3) + (pos >> 3)) * dh * 8;
    const size_t i0 = (size_t)d0 * 8 + (pos & 7), i1 = (size_t)(d0 + 16) * 8 + (pos & 7);
    if (e.kv_fmt == KV_F32) {
      // F32-grade cache: the 8-key group holds the hi plane [Dh][8], then the lo plane [Dh][8]
      uint16_t* base = static_cast<uint16_t*>(e.vc) + 2 * o;
      uint32_t h, l;
      split2_pk(x0, x1, h, l);
      base[i0] = (uint16_t)h;
      base[i1] = (uint16_t)(h >> 16);
      base[(size_t)dh * 8 + i0] = (uint16_t)l;
      base[(size_t)dh * 8 + i1] = (uint16_t)(l >> 16);
    } else {
      uint16_t* base = static_cast<uint16_t*>(e.vc) + o;
      const uint32_t h = e.kv_fmt == KV_F16 ? pack_f16x2(x0, x1) : pack_bf2(x0, x1);
      base[i0] = (uint16_t)h;
      base[i1] = (uint16_t)(h >> 16);
    }
  }
}

// Apply the QKV epilogue to one RoPE pair / V pair of outputs of row m (nothing for a row whose
// slot or position is out of range).
PSD_DEV void qkv_epilogue_pair(const EpiArgs& e, int m, int col0, float x0, float x1) {
  int slot, pos;
  if (!row_slot_pos(e, m, slot, pos)) return;
  col0 += e.col_off;
  qkv_store_pair(e, m, slot, pos, col0, x0, x1, qkv_rope_cs(e, pos, col0));
}

PSD_DEV float silu_mul(float g, float u) { return g / (1.0f + __expf(-g)) * u; }

PSD_DEV void store_pair(uint16_t* p, size_t ps, size_t i, float x) {
  uint32_t h, l;
  split2(x, h, l);
  p[i] = (uint16_t)h;
  p[ps + i] = (uint16_t)l;
}
