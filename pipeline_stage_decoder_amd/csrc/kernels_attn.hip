// Causal grouped-query attention over a slot's KV cache (bf16 or F32 elements), on MFMA.
//
// Definition ("41. Many GPUs", Ring attention: attention_partial / merge_partials): scores
// q.k * Dh^-1/2, keys after the query's position masked, softmax, weighted sum of V; partial
// results over key ranges merge by their log-sum-exp.  GQA: query head h reads KV head
// h / (Hq / Hkv) ("41. Many GPUs", Tensor parallelism).
//
// Both kernels work on 16 "columns" per wave -- (query, head) pairs that share one KV head -- and
// 32 keys per step:
//   S^T[key, col] = K[key, :] . q[col, :]    16x16x32 MFMAs per 32-dim slice of the head, once for
//       the bf16 hi plane of q and once for its lo plane (q keeps ~16 significant bits); the
//       A rows are permuted so lane l ends up with the 8 consecutive keys 8*(l/16) .. +8 of its
//       column l%16 -- exactly the B operand layout of the next product.
//   O^T[d, col] += V^T[d, key] P^T[key, col]   A = V^T read as 8 consecutive elements from the
//       packed V cache [pos/8][Dh][8]; B = P^T straight from registers, split into bf16 hi + lo
//       (two MFMAs) so the probabilities keep ~16 bits.
//   An F32-grade cache holds each value as bf16 hi + lo planes and adds the K_lo.q_hi and V_lo.P_hi
//   MFMAs.  An F16 cache holds binary16 values, multiplied on f16 MFMAs with q and P split into
//   binary16 hi + lo planes instead (~22 significant bits each); otherwise identical to bf16.
// The softmax is online per column (max and rescale), in base 2 with the scale folded in.  O^T
// puts a column's values in the same lane as its softmax state, so rescaling needs no shuffles.
//
// Decode: work-group = (split of about `chunk` keys, KV head, batch row); its 4 waves take every fourth
// 32-key step of the chunk and merge through LDS into one partial per split; a second kernel merges the
// splits of each (row, query head) in split order.
// Prefill: work-group = 64 columns (consecutive queries x the group's heads) of one KV head; the
// 4 waves share 32-key K/V tiles staged in LDS (double-buffered), each wave skipping tiles past its
// last query.
#include "kernels.h"

#include <type_traits>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr float kNegInf = -__builtin_huge_valf();

// 2^x by the hardware instruction alone: exp2f adds a range fix so that results below 2^-126 come
// out denormal, which a softmax weight never needs (the instruction flushes them to zero).  It
// gives exactly 1 for x = 0 and 0 for x = -inf, as the online softmax relies on.
PSD_DEV float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Lazy softmax base: a column's running base moves only when a score exceeds it by more than this
// (log2 units), so its weights stay at most 2^8 = 256 -- the output and the sum carry the same
// factor, and the output rescale runs only when some column of the wave moved.
constexpr float kLazyBase = 8.0f;

// Keys of the two S^T MFMAs that A row `rho` (0..15) of chunk c feeds: (rho/4)*8 + c*4 + rho%4.
PSD_DEV int key_of_row(int rho, int c) { return ((rho >> 2) << 3) + (c << 2) + (rho & 3); }

// Cache format traits: the MFMA operand type (binary16 for the F16 cache, bf16 otherwise), whether
// each value is a hi + lo pair of planes (F32-grade cache), and bytes per value.
template <int FMT>
struct Kv {
  static constexpr bool pair = FMT == KV_F32;
  static constexpr bool f16 = FMT == KV_F16;
  static constexpr int bytes = pair ? 4 : 2;
  typedef typename std::conditional<f16, f16x8_t, bf16x8_t>::type op;
  static PSD_DEV op as_op(uint4 v) { return __builtin_bit_cast(op, v); }
  // hi + lo planes of 8 probabilities in the operand format
  static PSD_DEV void split(const float* x, uint4& hi, uint4& lo) {
    if (f16) split_hi_lo_f16(x, hi, lo);
    else split_hi_lo(x, hi, lo);
  }
};

// 8 consecutive cache elements: a bf16 / binary16 cache's bits at element offset `off` (lo = 0), or
// an F32-grade cache's hi plane there and its lo plane `lo_off` elements further (both bf16, split
// when written).  (Written as a branch: as a select between the load and zero, the compiler split
// each 16-byte load into four 4-byte loads behind branches.)
// NT: non-temporal loads (the batched decode's K/V streams: a plain 4 GiB read measured 6.2 TB/s
// with ordinary 16-byte loads and 6.8 TB/s with non-temporal ones; at B = 1 they were slower).
template <bool KF32, bool NT = false>
PSD_DEV void load8(const uint16_t* base, size_t off, size_t lo_off, bool ok, uint4& hi, uint4& lo) {
  hi = make_uint4(0, 0, 0, 0);
  lo = make_uint4(0, 0, 0, 0);
  if (ok) {
    if constexpr (NT) {
      const u32x4 h = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off));
      hi = make_uint4(h.x, h.y, h.z, h.w);
      if (KF32) {
        const u32x4 l = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + off + lo_off));
        lo = make_uint4(l.x, l.y, l.z, l.w);
      }
    } else {
      hi = *reinterpret_cast<const uint4*>(base + off);
      if (KF32) lo = *reinterpret_cast<const uint4*>(base + off + lo_off);
    }
  }
}

PSD_DEV uint4 mask_tail(uint4 v, int nvalid) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    if (e >= nvalid) w[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
  return make_uint4(w[0], w[1], w[2], w[3]);
}

template <int DH, int FMT>
struct Col16 {
  typename Kv<FMT>::op qh[DH / 32];    // B operand of S^T: q[col][ks*32 + grp*8 .. +8], hi plane
  typename Kv<FMT>::op ql[DH / 32];    // lo plane
  f32x4_t o[DH / 16];      // O^T[dt*16 + grp*4 + j][col]
  float m, l;              // running max (base-2 scaled) and this lane's share of the sum
};

// o *= alpha for the wave's columns.  A column whose running max did not move has alpha exactly 1,
// and one that has seen no visible key still has o exactly 0; the product changes no bit in either
// case, so the wave skips the multiplies when one of the two holds for every lane.
template <int DH, int FMT>
PSD_DEV void rescale_o(Col16<DH, FMT>& st, float m_old, float m_new, float alpha) {
  if (__any(m_old != m_new && m_old != kNegInf)) {
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt) st.o[dt] *= alpha;
  }
}

// One 32-key step for a wave's 16 columns.  kb: first key (multiple of 8); the keys below kend count
// for every column, keys >= kend are never read.
template <int DH, int FMT, bool NT>
PSD_DEV void attn_step(Col16<DH, FMT>& st, const uint16_t* __restrict__ kbase, const uint16_t* __restrict__ vbase,
                       int kb, int kend, float scale_log2) {
  typedef Kv<FMT> F;
  constexpr bool KF32 = F::pair;
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  // issue every K and V load of the step first: one memory round trip per step
  uint4 kh[2][DH / 32], kl[2][DH / 32];
  // K row `key` starts at element key * DH (bf16) or key * 2 DH (hi plane, then lo plane); V group
  // g at g * DH * 8 or g * 2 DH * 8 (likewise)
  constexpr int NPL = KF32 ? 2 : 1;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int key = kb + key_of_row(col, c);
    const bool ok = key < kend;
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks)
      load8<KF32, NT>(kbase, (size_t)key * NPL * DH + ks * 32 + grp * 8, DH, ok, kh[c][ks], kl[c][ks]);
  }
  const int kg = kb + grp * 8;              // this lane's 8 keys in the PV product
  const int nvalid = kend - kg;             // keys of the group below kend
  uint4 vh[DH / 16], vl[DH / 16];
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt)
    load8<KF32, NT>(vbase, (size_t)(kg >> 3) * NPL * DH * 8 + (dt * 16 + col) * 8, DH * 8, nvalid > 0, vh[dt],
                    vl[dt]);
  f32x4_t sc[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    sc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < DH / 32; ++ks) {
      sc[c] = mfma16(F::as_op(kh[c][ks]), st.qh[ks], sc[c]);
      sc[c] = mfma16(F::as_op(kh[c][ks]), st.ql[ks], sc[c]);
      if (KF32) sc[c] = mfma16(F::as_op(kl[c][ks]), st.qh[ks], sc[c]);
    }
  }
  float s[8];
  float mx = kNegInf;
  auto scores = [&](auto masked_c) {
    constexpr bool masked = decltype(masked_c)::value;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kb + grp * 8 + c * 4 + j;
        const float v = (!masked || key < kend) ? sc[c][j] * scale_log2 : kNegInf;
        s[c * 4 + j] = v;
        mx = fmaxf(mx, v);
      }
  };
  // a whole step below kend: the same values without the per-key test
  if (kb + 32 <= kend) scores(std::false_type{});
  else scores(std::true_type{});
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  const float m_old = st.m, m_new = mx > st.m + kLazyBase ? mx : st.m;
  // m_new is -inf only if this column has seen no visible key yet; keep everything at zero then.
  const float base = (m_new == kNegInf) ? 0.0f : m_new;
  const float alpha = exp2_hw(m_old - base);
  float p[8], ps = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p[e] = exp2_hw(s[e] - base);
    ps += p[e];
  }
  st.l = st.l * alpha + ps;
  st.m = m_new;
  rescale_o(st, m_old, m_new, alpha);
  uint4 phi, plo;
  F::split(p, phi, plo);
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) {
    uint4 a = vh[dt], b = vl[dt];
    if (nvalid < 8) {
      a = mask_tail(a, nvalid);
      b = mask_tail(b, nvalid);
    }
    st.o[dt] = mfma16(F::as_op(a), F::as_op(phi), st.o[dt]);
    st.o[dt] = mfma16(F::as_op(a), F::as_op(plo), st.o[dt]);
    if (KF32) st.o[dt] = mfma16(F::as_op(b), F::as_op(phi), st.o[dt]);
  }
}

template <int DH, int FMT>
PSD_DEV void load_q(Col16<DH, FMT>& st, const uint16_t* __restrict__ qrow /* null = padded column */, size_t q_ps) {
  const int grp = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int ks = 0; ks < DH / 32; ++ks) {
    uint4 h = make_uint4(0, 0, 0, 0), l = make_uint4(0, 0, 0, 0);
    if (qrow) {
      h = *reinterpret_cast<const uint4*>(qrow + ks * 32 + grp * 8);
      l = *reinterpret_cast<const uint4*>(qrow + q_ps + ks * 32 + grp * 8);
    }
    st.qh[ks] = Kv<FMT>::as_op(h);
    st.ql[ks] = Kv<FMT>::as_op(l);
  }
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) st.o[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = kNegInf;
  st.l = 0.0f;
}

// ------------------------------------------------------------------------------------------------
// decode: partial attention per (split, KV head, row)
// ------------------------------------------------------------------------------------------------
template <int DH, int FMT, bool NT>
__global__ __launch_bounds__(256) void k_attn_decode(AttnDecodeArgs a) {
  __shared__ float sm[4][16], sl[4][16];
  __shared__ float so[4][DH][17];
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int slot = a.slots[b], pos = a.pos[b];
  const int G = a.hq / a.hkv;
  if (slot < 0 || slot >= a.max_slots || pos < 0 || pos >= a.ctx_cap) return;
  const int ctx = pos + 1;
  const int ns = attn_decode_splits(ctx, a.chunk);
  if (split >= ns) return;
  const int k0 = split * a.chunk;
  const int k1 = split == ns - 1 ? ctx : k0 + a.chunk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;

  Col16<DH, FMT> st;
  load_q(st, col < G ? a.q + ((size_t)b * a.hq + kvh * G + col) * DH : nullptr, a.q_ps);
  const size_t eb = Kv<FMT>::bytes;
  const uint16_t* kbase = reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.kc) +
                                                            ((size_t)slot * a.hkv + kvh) * a.ctx_cap * DH * eb);
  const uint16_t* vbase = reinterpret_cast<const uint16_t*>(static_cast<const char*>(a.vc) +
                                                            ((size_t)slot * a.hkv + kvh) * (size_t)a.ctx_cap * DH * eb);
  // the 4 waves take interleaved 32-key steps, so that the work-group reads one contiguous 128-key
  // stretch of K and of V at a time (4% faster than a quarter of the chunk per wave at B = 128)
  for (int kb = k0 + wave * 32; kb < k1; kb += 128)
    attn_step<DH, FMT, NT>(st, kbase, vbase, kb, k1, a.scale_log2);

  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (grp == 0) {
    sm[wave][col] = st.m;
    sl[wave][col] = l;
  }
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) so[wave][dt * 16 + grp * 4 + j][col] = st.o[dt][j];
  __syncthreads();

  // merge the four waves (fixed order) and write this split's normalised partial
  for (int idx = threadIdx.x; idx < G * DH; idx += 256) {
    const int h = idx / DH, d = idx - h * DH;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < 4; ++w) mm = fmaxf(mm, sm[w][h]);
    float L = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = (sm[w][h] == kNegInf) ? 0.0f : exp2f(sm[w][h] - mm);
      L += f * sl[w][h];
      acc += f * so[w][d][h];
    }
    const size_t row = ((size_t)b * a.hq + kvh * G + h) * a.nsplit + split;
    a.part_o[row * DH + d] = acc / L;
    if (d == 0) a.part_lse[row] = mm + log2f(L);
  }

}

// Merge the splits of one (row, query head) in split order -> attention output pair buffer.  A
// thread owns one output dim: it loads the head's split log-sum-exps and its dim of every split's
// partial together (up to 16 splits per round trip), takes the maximum, then sums the weighted
// partials in split order.
// A separate launch rather than a last-arriving work-group inside the partial kernel: making the
// partials visible across work-groups inside one kernel takes a device-scope release/acquire,
// which on gfx950 writes back and invalidates the L2 of each work-group's XCD.  Measured on the
// 8B-shaped block at B = 1, ctx 1536: 8.4 + 4.7 us as two kernels; 19.0 us fused with
// __threadfence, 15.8 us with agent-scope release / acquire fences.
template <int DH>
__global__ __launch_bounds__(DH) void k_attn_merge(AttnDecodeArgs a) {
  constexpr int R = 16;                       // splits per round of loads
  const int head = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int slot = a.slots[b], pos = a.pos[b];
  const size_t o = ((size_t)b * a.hq + head) * DH + d;
  if (slot < 0 || slot >= a.max_slots || pos < 0 || pos >= a.ctx_cap) {
    a.out[o] = 0;
    a.out[a.out_ps + o] = 0;
    return;
  }
  const int ns = attn_decode_splits(pos + 1, a.chunk);
  const size_t row0 = ((size_t)b * a.hq + head) * a.nsplit;
  const float* lse = a.part_lse + row0;
  const float* po = a.part_o + row0 * DH + d;
  float L = 0.0f, acc = 0.0f;
  if (ns <= R) {
    float l[R], v[R];
    float mm = kNegInf;
#pragma unroll
    for (int j = 0; j < R; ++j) {
      l[j] = j < ns ? lse[j] : kNegInf;
      v[j] = j < ns ? po[(size_t)j * DH] : 0.0f;
    }
#pragma unroll
    for (int j = 0; j < R; ++j) mm = fmaxf(mm, l[j]);
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const float f = exp2f(l[j] - mm);        // 0 for the padding
      L += f;
      acc += f * v[j];
    }
  } else {
    float mm = kNegInf;
    for (int s0 = 0; s0 < ns; s0 += R) {
      float l[R];
#pragma unroll
      for (int j = 0; j < R; ++j) l[j] = s0 + j < ns ? lse[s0 + j] : kNegInf;
#pragma unroll
      for (int j = 0; j < R; ++j) mm = fmaxf(mm, l[j]);
    }
    for (int s0 = 0; s0 < ns; s0 += R) {
      float l[R], v[R];
#pragma unroll
      for (int j = 0; j < R; ++j) {
        l[j] = s0 + j < ns ? lse[s0 + j] : kNegInf;
        v[j] = s0 + j < ns ? po[(size_t)(s0 + j) * DH] : 0.0f;
      }
#pragma unroll
      for (int j = 0; j < R; ++j) {
        const float f = exp2f(l[j] - mm);
        L += f;
        acc += f * v[j];
      }
    }
  }
  store_pair(a.out, a.out_ps, o, acc / L);
}

// ------------------------------------------------------------------------------------------------
// prefill: 64 columns (queries x heads of one KV head) per work-group; the 4 waves share 64-key K/V
// tiles staged in LDS (consumed as two 32-key steps), the next tile's global loads in flight while
// the current one is consumed
// ------------------------------------------------------------------------------------------------
constexpr int kKeyTile = 64;   // keys per LDS tile; MFMA steps take 32

// XOR applied to the 16-byte chunk index within K tile row `key` (0..31), RC chunks per row.  The
// 16 keys one A-operand read touches (key_of_row(col, c), col 0..15) have distinct
// (key & 3) | (key >> 3) << 2 = col; scaled to the row width, the same chunk of those 16 rows lands
// in 16 distinct 16-byte bank groups (a 128-byte row shares a 256-byte bank line with its neighbour
// of opposite parity, so there the value is halved).
template <int RC>
PSD_DEV int k_swz(int key) {
  static_assert(RC == 8 || RC == 16 || RC == 32, "row chunks");
  const int c = (key & 3) | ((key >> 3) << 2);
  return RC >= 16 ? c * (RC / 16) : c >> 1;
}

// NBUF LDS tile buffers: 2 (one tile's global loads in flight while the current one is consumed),
// or 3 for a 2-byte cache on a grid of at most one work-group per CU, where no second work-group
// hides the load latency: the loads of tile t + 2 are issued while tile t is consumed, into the
// register set that tile t + 1 does not occupy.
template <int DH, int FMT, int NBUF>
__global__ __launch_bounds__(256) void k_attn_prefill(AttnPrefillArgs a) {
  typedef Kv<FMT> F;
  constexpr bool KF32 = F::pair;
  constexpr int EB = F::bytes;
  constexpr int TILE_CHUNKS = kKeyTile * DH * EB / 16;     // 16-byte global chunks per K (and V) tile
  constexpr int PER_THREAD = TILE_CHUNKS / 256;
  static_assert(TILE_CHUNKS % 256 == 0, "tile chunks per thread");
  // LDS holds bf16 planes: the cache's bf16 values, or an F32-grade cache's hi and lo planes (split
  // when the cache was written), so every wave reads ready MFMA operands in the bf16 layout
  constexpr int NPL = KF32 ? 2 : 1;
  constexpr int RC = DH / 8;                               // 16-byte chunks per bf16 K row
  constexpr int PLANE = kKeyTile * RC;                     // uint4 per plane tile
  static_assert(NBUF == 2 || (NBUF == 3 && !KF32), "three buffers: 2-byte caches only");
  __shared__ uint4 kt[NBUF][NPL][PLANE];
  __shared__ uint4 vt[NBUF][NPL][PLANE];

  const int G = a.hq / a.hkv;
  // Work-groups go to the 8 XCDs round-robin in linear block order, so block b takes KV head
  // b % Hkv: with 8 KV heads each XCD's L2 holds one head's K/V, which all of that head's column
  // blocks re-read.  Heavier (later) column blocks first.
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  const int kvh = b % a.hkv;
  const int ncols = a.T * G;
  const int cblk = gridDim.x - 1 - b / a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 15, grp = lane >> 4;
  const int c0 = cblk * 64 + wave * 16;
  const int c = c0 + col;
  const bool cvalid = c < ncols;
  const int t = cvalid ? c / G : 0, h = cvalid ? c - (c / G) * G : 0;
  const int head = kvh * G + h;
  const int my_pos = a.pos0 + t;
  const bool wave_live = c0 < ncols;
  const int wlast = wave_live ? min(c0 + 15, ncols - 1) : 0;
  const int wave_kend = a.pos0 + wlast / G + 1;            // keys [0, wave_kend) matter to this wave
  const int blast = min(cblk * 64 + 63, ncols - 1);
  const int kend = min(a.pos0 + blast / G + 1, a.k_hi);   // keys the work-group walks: [k_lo, kend)
  const int tile0 = a.k_lo / kKeyTile;
  const int ntiles = kend > a.k_lo ? (kend + kKeyTile - 1) / kKeyTile : tile0;

  Col16<DH, FMT> st;
  load_q(st, cvalid ? a.q + ((size_t)t * a.hq + head) * DH : nullptr, a.q_ps);
  const u32x4* kg = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.kc) +
                                                  ((size_t)a.slot * a.hkv + kvh) * a.ctx_cap * DH * EB);
  const u32x4* vg = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.vc) +
                                                  ((size_t)a.slot * a.hkv + kvh) * (size_t)a.ctx_cap * DH * EB);
  // a tile is one contiguous byte range of K (kKeyTile rows) and of V (kKeyTile / 8 packed groups)
  u32x4 kr[PER_THREAD], vr[PER_THREAD], kr2[PER_THREAD], vr2[PER_THREAD];
  auto gload_into = [&](int tile, u32x4 (&gk)[PER_THREAD], u32x4 (&gv)[PER_THREAD]) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = threadIdx.x + i * 256;
      gk[i] = kg[(size_t)tile * TILE_CHUNKS + q];
      gv[i] = vg[(size_t)tile * TILE_CHUNKS + q];
    }
  };
  auto gload = [&](int tile) { gload_into(tile, kr, vr); };
  auto sstore_from = [&](int buf, const u32x4 (&kr)[PER_THREAD], const u32x4 (&vr)[PER_THREAD]) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = threadIdx.x + i * 256;
      if (KF32) {
        // K: a row is RC hi-plane chunks, then RC lo-plane chunks (planes PLANE chunks apart in LDS)
        const int row = q / (2 * RC), cc = q - row * (2 * RC);
        const int pl = cc / RC, ch = cc % RC;
        reinterpret_cast<u32x4*>(&kt[buf][0][0])[pl * PLANE + row * RC + (ch ^ k_swz<RC>(row & 31))] = kr[i];
        // V: an 8-key group is DH hi-plane chunks (one per dim), then DH lo-plane chunks
        const int g = q / (2 * DH), cv = q - g * (2 * DH);
        reinterpret_cast<u32x4*>(&vt[buf][0][0])[(cv / DH) * PLANE + g * DH + cv % DH] = vr[i];
      } else {
        const int row = q / RC, ch = q - row * RC;
        reinterpret_cast<u32x4*>(kt[buf][0])[row * RC + (ch ^ k_swz<RC>(row & 31))] = kr[i];
        reinterpret_cast<u32x4*>(vt[buf][0])[q] = vr[i];
      }
    }
  };
  auto sstore = [&](int buf) { sstore_from(buf, kr, vr); };

  // every wave's steps of tile `tile` from LDS buffer `cur`
  auto consume = [&](int tile, int cur) {
#pragma unroll
    for (int sub = 0; sub < kKeyTile / 32; ++sub) {
    const int kb = tile * kKeyTile + sub * 32;
    if (wave_live && kb < wave_kend && kb < kend) {
      // K fragments: A row rho of chunk c is key key_of_row(rho, c); 8 elements at dim ks*32 + grp*8
      uint4 kh[2][DH / 32], kl[2][DH / 32];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        const int key = key_of_row(col, cc);
        const int sw = k_swz<RC>(key);
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) {
          const int at = (sub * 32 + key) * RC + ((ks * 4 + grp) ^ sw);
          kh[cc][ks] = kt[cur][0][at];
          kl[cc][ks] = KF32 ? kt[cur][NPL - 1][at] : make_uint4(0, 0, 0, 0);
        }
      }
      f32x4_t sc[2];
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) {
        sc[cc] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < DH / 32; ++ks) {
          sc[cc] = mfma16(F::as_op(kh[cc][ks]), st.qh[ks], sc[cc]);
          sc[cc] = mfma16(F::as_op(kh[cc][ks]), st.ql[ks], sc[cc]);
          if (KF32) sc[cc] = mfma16(F::as_op(kl[cc][ks]), st.qh[ks], sc[cc]);
        }
      }
      float sv[8];
      float mx = kNegInf;
      auto scores = [&](auto masked_c) {
        constexpr bool masked = decltype(masked_c)::value;
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int key = kb + grp * 8 + cc * 4 + j;
            const bool vis = !masked || (key >= a.k_lo && key < kend && key <= my_pos);
            const float v = vis ? sc[cc][j] * a.scale_log2 : kNegInf;
            sv[cc * 4 + j] = v;
            mx = fmaxf(mx, v);
          }
      };
      // every key of the step visible to every live column of the wave (inside [k_lo, kend) and at
      // or before the wave's first query): the same values without the per-key mask
      if (kb >= a.k_lo && kb + 32 <= kend && kb + 31 <= a.pos0 + c0 / G) scores(std::false_type{});
      else scores(std::true_type{});
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float m_old = st.m, m_new = mx > st.m + kLazyBase ? mx : st.m;
      const float base = (m_new == kNegInf) ? 0.0f : m_new;
      const float alpha = exp2_hw(m_old - base);
      float p[8], ps = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = exp2_hw(sv[e] - base);
        ps += p[e];
      }
      st.l = st.l * alpha + ps;
      st.m = m_new;
      rescale_o(st, m_old, m_new, alpha);
      uint4 phi, plo;
      F::split(p, phi, plo);
      // V fragments: 8 keys of group grp at dim dt*16 + col; keys at or past kend (p = 0) are
      // zeroed so that whatever the cache holds there cannot reach the sum
      const int nvalid = kend - (kb + grp * 8);
#pragma unroll
      for (int dt = 0; dt < DH / 16; ++dt) {
        const int q = (sub * 4 + grp) * DH + dt * 16 + col;
        uint4 vh = vt[cur][0][q];
        uint4 vl = KF32 ? vt[cur][NPL - 1][q] : make_uint4(0, 0, 0, 0);
        if (nvalid < 8) {
          vh = mask_tail(vh, nvalid);
          vl = mask_tail(vl, nvalid);
        }
        st.o[dt] = mfma16(F::as_op(vh), F::as_op(phi), st.o[dt]);
        st.o[dt] = mfma16(F::as_op(vh), F::as_op(plo), st.o[dt]);
        if (KF32) st.o[dt] = mfma16(F::as_op(vl), F::as_op(phi), st.o[dt]);
      }
    }
    }
  };

  if constexpr (NBUF == 2) {
    if (tile0 < ntiles) {
      gload(tile0);
      sstore(tile0 & 1);
    }
    __syncthreads();
    for (int tile = tile0; tile < ntiles; ++tile) {
      const int cur = tile & 1;
      if (tile + 1 < ntiles) gload(tile + 1);
      consume(tile, cur);
      if (tile + 1 < ntiles) sstore(cur ^ 1);
      __syncthreads();
    }
  } else {
    // Set 1 holds tile t + 1 while set 2 receives tile t + 2 (the roles swap every tile, so the
    // loop is unrolled by two).  The loads are unconditional -- past the last tile they re-read
    // it -- so that at each store the only loads still in flight are the other set's.
    const int last = ntiles - 1;
    auto step = [&](int tile, u32x4 (&ldk)[PER_THREAD], u32x4 (&ldv)[PER_THREAD],
                    const u32x4 (&stk)[PER_THREAD], const u32x4 (&stv)[PER_THREAD]) {
      gload_into(min(tile + 2, last), ldk, ldv);
      consume(tile, tile % 3);
      if (tile + 1 < ntiles) sstore_from((tile + 1) % 3, stk, stv);
      __syncthreads();
    };
    if (tile0 < ntiles) {
      gload_into(tile0, kr, vr);
      sstore_from(tile0 % 3, kr, vr);
      gload_into(min(tile0 + 1, last), kr, vr);
    }
    __syncthreads();
    for (int tile = tile0; tile < ntiles; tile += 2) {
      step(tile, kr2, vr2, kr, vr);
      if (tile + 1 < ntiles) step(tile + 1, kr, vr, kr2, vr2);
    }
  }

  float l = st.l;
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
  if (!cvalid) return;
  if (a.part_o) {
    // partial of the key range: normalised output and base-2 log-sum-exp (no key: 0 and -inf)
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* po = a.part_o + ((size_t)t * a.hq + head) * DH;
#pragma unroll
    for (int dt = 0; dt < DH / 16; ++dt)
      *reinterpret_cast<float4*>(po + dt * 16 + grp * 4) =
          make_float4(st.o[dt][0] * inv, st.o[dt][1] * inv, st.o[dt][2] * inv, st.o[dt][3] * inv);
    if (grp == 0) a.part_lse[(size_t)t * a.hq + head] = l > 0.0f ? st.m + log2f(l) : kNegInf;
    return;
  }
  const float inv = 1.0f / l;
  uint16_t* out = a.out + (size_t)t * a.hq * DH + (size_t)head * DH;
#pragma unroll
  for (int dt = 0; dt < DH / 16; ++dt) {
    const int d = dt * 16 + grp * 4;
    uint32_t hh[4], ll[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) split2(st.o[dt][j] * inv, hh[j], ll[j]);
    *reinterpret_cast<uint2*>(out + d) = make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
    *reinterpret_cast<uint2*>(out + a.out_ps + d) = make_uint2(ll[0] | (ll[1] << 16), ll[2] | (ll[3] << 16));
  }
}

// ------------------------------------------------------------------------------------------------
// prefill over a 2-byte cache: 32 columns per wave on 32 x 32 x 16 MFMAs
// ------------------------------------------------------------------------------------------------
// The same online-softmax attention as k_attn_prefill, with each wave owning 32 (query, head)
// columns instead of 16: every K and V fragment read from LDS then feeds twice the columns, so a
// work-group of 4 waves (128 columns) reads each 32-key step of K and V once per 32 columns.
//   S^T[key][col] = K[key] . q[col]: A = 32 keys x 16 dims of K, B = 16 dims x 32 columns of q
//   (hi and lo planes, two products); O^T[dim][col] += V^T[dim][key] P^T[key][col]: A = 32 dims x
//   16 keys of V (one 16-byte cache chunk: 8 keys of one dim), B = P^T in hi + lo planes.
// Lane l holds column l % 32 of both products (C layout: row (j / 4) * 8 + (l / 32) * 4 + j % 4 in
// slot j), so a column's softmax state, its scores and its output live in the same two lanes.  The
// A rows of S^T are permuted (key_of_row32) so that the 16 score slots of lane half h are keys
// h * 8 + 0..7 and 16 + h * 8 + 0..7: exactly the B operand of the two 16-key PV products.

typedef float f32x16_t __attribute__((ext_vector_type(16)));
PSD_DEV f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
PSD_DEV f32x16_t mfma32(f16x8_t a, f16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}


// key (within a 32-key step) of S^T row rho = 8a + 4h + r: (a / 2) * 16 + h * 8 + (a % 2) * 4 + r
PSD_DEV int key_of_row32(int rho) {
  const int a = rho >> 3, h = (rho >> 2) & 1, r = rho & 3;
  return ((a >> 1) << 4) + (h << 3) + ((a & 1) << 2) + r;
}

// XOR applied to the 16-byte chunk index of K tile row `key`, RC chunks per row: the 8 rows one
// phase of an A-operand read touches (keys {0..3, 8..11} + 4k + 16m of a step) land in distinct
// bank groups (RC = 16: a row is a whole 256-byte bank line; RC = 8: two rows share one).
template <int RC>
PSD_DEV int k_swz32(int key) {
  static_assert(RC == 8 || RC == 16, "row chunks");
  return RC == 16 ? (key & 15) : (((key >> 1) & 1) | (((key >> 3) & 1) << 1));
}

template <int DH, int FMT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void k_attn_prefill32(AttnPrefillArgs a) {
  typedef Kv<FMT> F;
  static_assert(!F::pair, "2-byte caches only");
  constexpr int RC = DH / 8;                               // 16-byte chunks per K row
  constexpr int TILE_CHUNKS = kKeyTile * RC;               // per K (and V) tile
  constexpr int PER_THREAD = TILE_CHUNKS / 256;
  static_assert(TILE_CHUNKS % 256 == 0, "tile chunks per thread");
  constexpr int KS = DH / 16;                              // 16-dim steps of S^T
  constexpr int DB = DH / 32;                              // 32-dim blocks of O^T
  __shared__ uint4 kt[2][TILE_CHUNKS];
  __shared__ uint4 vt[2][TILE_CHUNKS];

  const int G = a.hq / a.hkv;
  // block b takes KV head b % Hkv (one head per XCD with 8 heads), heavier column blocks first
  const int b = blockIdx.y * gridDim.x + blockIdx.x;
  const int kvh = b % a.hkv;
  const int ncols = a.T * G;
  const int cblk = gridDim.x - 1 - b / a.hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, col = lane & 31, half = lane >> 5;
  const int c0 = cblk * 128 + wave * 32;
  const int c = c0 + col;
  const bool cvalid = c < ncols;
  const int t = cvalid ? c / G : 0, h = cvalid ? c - (c / G) * G : 0;
  const int head = kvh * G + h;
  const int my_pos = a.pos0 + t;
  const bool wave_live = c0 < ncols;
  const int wlast = wave_live ? min(c0 + 31, ncols - 1) : 0;
  const int wave_kend = a.pos0 + wlast / G + 1;            // keys [0, wave_kend) matter to this wave
  const int blast = min(cblk * 128 + 127, ncols - 1);
  const int kend = min(a.pos0 + blast / G + 1, a.k_hi);   // keys the work-group walks: [k_lo, kend)
  const int tile0 = a.k_lo / kKeyTile;
  const int ntiles = kend > a.k_lo ? (kend + kKeyTile - 1) / kKeyTile : tile0;

  // q^T fragments (B operand): dims ks * 16 + half * 8 + 0..7 of this column, hi and lo planes
  typename F::op qh[KS], ql[KS];
  {
    const uint16_t* qrow = a.q + ((size_t)t * a.hq + head) * DH;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 hv = make_uint4(0, 0, 0, 0), lv = make_uint4(0, 0, 0, 0);
      if (cvalid) {
        hv = *reinterpret_cast<const uint4*>(qrow + ks * 16 + half * 8);
        lv = *reinterpret_cast<const uint4*>(qrow + a.q_ps + ks * 16 + half * 8);
      }
      qh[ks] = F::as_op(hv);
      ql[ks] = F::as_op(lv);
    }
  }
  f32x16_t o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[db][j] = 0.0f;
  float m = kNegInf, l = 0.0f;                             // l: this lane's 16 keys per step

  // staged through vector-typed registers (as HIP's uint4 struct the copy goes through private memory)
  const u32x4* kg = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.kc) +
                                                   ((size_t)a.slot * a.hkv + kvh) * a.ctx_cap * DH * 2);
  const u32x4* vg = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.vc) +
                                                   ((size_t)a.slot * a.hkv + kvh) * (size_t)a.ctx_cap * DH * 2);
  u32x4 kr[PER_THREAD], vr[PER_THREAD];
  auto gload = [&](int tile) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = threadIdx.x + i * 256;
      kr[i] = kg[(size_t)tile * TILE_CHUNKS + q];
      vr[i] = vg[(size_t)tile * TILE_CHUNKS + q];
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_THREAD; ++i) {
      const int q = threadIdx.x + i * 256;
      const int row = q / RC, ch = q - row * RC;
      reinterpret_cast<u32x4*>(kt[buf])[row * RC + (ch ^ k_swz32<RC>(row))] = kr[i];
      reinterpret_cast<u32x4*>(vt[buf])[q] = vr[i];
    }
  };

  const int arow = key_of_row32(col);                      // this lane's A row of S^T: its key
  if (tile0 < ntiles) {
    gload(tile0);
    sstore(tile0 & 1);
  }
  __syncthreads();
  for (int tile = tile0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    if (tile + 1 < ntiles) gload(tile + 1);
#pragma unroll
    for (int sub = 0; sub < kKeyTile / 32; ++sub) {
      const int kb = tile * kKeyTile + sub * 32;
      if (wave_live && kb < wave_kend && kb < kend) {
        f32x16_t sc;
#pragma unroll
        for (int j = 0; j < 16; ++j) sc[j] = 0.0f;
        const int krow = sub * 32 + arow;
        const int ksw = k_swz32<RC>(krow);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const typename F::op kf = F::as_op(kt[cur][krow * RC + ((ks * 2 + half) ^ ksw)]);
          sc = mfma32(kf, qh[ks], sc);
          sc = mfma32(kf, ql[ks], sc);
        }
        // slot j: key kb + (j / 8) * 16 + half * 8 + j % 8
        // every key of the step visible to every live column of the wave (a wave-uniform test):
        // the scores without the per-key mask
        float sv[16];
        float mx = kNegInf;
        if (kb >= a.k_lo && kb + 32 <= kend && kb + 31 <= a.pos0 + c0 / G) {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            sv[j] = sc[j] * a.scale_log2;
            mx = fmaxf(mx, sv[j]);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kb + ((j >> 3) << 4) + (half << 3) + (j & 7);
            const bool vis = key >= a.k_lo && key < kend && key <= my_pos;
            sv[j] = vis ? sc[j] * a.scale_log2 : kNegInf;
            mx = fmaxf(mx, sv[j]);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        // the column's base moves only when a score exceeds it by more than kLazyBase (2^8): the
        // weights below are then at most 256, the output and the sum carry the same factor, and
        // the 64-value rescale runs only when some column of the wave moved
        const bool move = mx > m + kLazyBase;
        const float m_new = move ? mx : m;
        const float base = (m_new == kNegInf) ? 0.0f : m_new;
        const float alpha = exp2_hw(m - base);
        float p0[8], p1[8], ps = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p0[j] = exp2_hw(sv[j] - base);
          p1[j] = exp2_hw(sv[8 + j] - base);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) ps += p0[j];
#pragma unroll
        for (int j = 0; j < 8; ++j) ps += p1[j];
        l = l * alpha + ps;
        // alpha is exactly 1 (base unmoved) or o is still 0 (no key seen) for every lane: skip
        if (__any(move && m != kNegInf)) {
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db] *= alpha;
        }
        m = m_new;
        uint4 phi[2], plo[2];
        F::split(p0, phi[0], plo[0]);
        F::split(p1, phi[1], plo[1]);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          // keys kb + s * 16 + half * 8 + 0..7: V group (kb + s * 16 + half * 8) / 8 of the tile
          const int g = sub * 4 + s * 2 + half;
          const int nvalid = kend - (kb + s * 16 + half * 8);
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            uint4 vv = vt[cur][g * DH + db * 32 + col];
            if (nvalid < 8) vv = mask_tail(vv, nvalid);
            o[db] = mfma32(F::as_op(vv), F::as_op(phi[s]), o[db]);
            o[db] = mfma32(F::as_op(vv), F::as_op(plo[s]), o[db]);
          }
        }
      }
    }
    if (tile + 1 < ntiles) sstore(cur ^ 1);
    __syncthreads();
  }

  l += __shfl_xor(l, 32, 64);
  if (!cvalid) return;
  // slot j of block db: dim db * 32 + (j / 4) * 8 + half * 4 + j % 4
  if (a.part_o) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    float* po = a.part_o + ((size_t)t * a.hq + head) * DH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *reinterpret_cast<float4*>(po + db * 32 + q4 * 8 + half * 4) =
            make_float4(o[db][q4 * 4] * inv, o[db][q4 * 4 + 1] * inv, o[db][q4 * 4 + 2] * inv,
                        o[db][q4 * 4 + 3] * inv);
    if (half == 0) a.part_lse[(size_t)t * a.hq + head] = l > 0.0f ? m + log2f(l) : kNegInf;
    return;
  }
  const float inv = 1.0f / l;
  uint16_t* out = a.out + (size_t)t * a.hq * DH + (size_t)head * DH;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = db * 32 + q4 * 8 + half * 4;
      uint32_t hh[4], ll[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) split2(o[db][q4 * 4 + j] * inv, hh[j], ll[j]);
      *reinterpret_cast<uint2*>(out + d) = make_uint2(hh[0] | (hh[1] << 16), hh[2] | (hh[3] << 16));
      *reinterpret_cast<uint2*>(out + a.out_ps + d) = make_uint2(ll[0] | (ll[1] << 16), ll[2] | (ll[3] << 16));
    }
}

// ------------------------------------------------------------------------------------------------
// ring attention: merge a key range's partial into running accumulators, in hop order
// ------------------------------------------------------------------------------------------------
// One work-group per (row, head), one thread per dim.  All threads read the old log-sum-exp before
// thread 0 replaces it.
template <int DH>
__global__ __launch_bounds__(DH) void k_ring_merge(float* __restrict__ acc_o, float* __restrict__ acc_lse,
                                                   const float* __restrict__ part_o,
                                                   const float* __restrict__ part_lse, int first) {
  const size_t rh = blockIdx.x;
  const int d = threadIdx.x;
  const float pl = part_lse[rh], po = part_o[rh * DH + d];
  if (first) {
    acc_o[rh * DH + d] = po;
    if (d == 0) acc_lse[rh] = pl;
    return;
  }
  const float al = acc_lse[rh];
  float top = fmaxf(al, pl);
  if (top == kNegInf) top = 0.0f;
  const float wa = exp2f(al - top), wb = exp2f(pl - top), tot = wa + wb;
  acc_o[rh * DH + d] = tot > 0.0f ? (acc_o[rh * DH + d] * wa + po * wb) / tot : 0.0f;
  __syncthreads();
  if (d == 0) acc_lse[rh] = tot > 0.0f ? top + log2f(tot) : kNegInf;
}

template <int DH>
__global__ __launch_bounds__(DH) void k_ring_store(const float* __restrict__ acc_o, uint16_t* __restrict__ out,
                                                   size_t out_ps) {
  const size_t i = (size_t)blockIdx.x * DH + threadIdx.x;
  store_pair(out, out_ps, i, acc_o[i]);
}

}  // namespace

// keys per decode work-group: more splits when few rows must fill the chip
int attn_decode_chunk(int B) {
  if (B <= 1) return 128;
  if (B <= 4) return 256;
  return 512;
}

// 70B-shaped B = 128 at ctx 8192: 1024-key splits (8192 work-groups) against 512 (16384): 14.7 ->
// 14.4 ms of attention per decode step.  At B = 64, ctx 4096 the doubled chunk would leave 2048
// work-groups and was ~1% slower, so the rule keeps 512 there.
int attn_decode_chunk_for(int B, int hkv, int ctx_cap) {
  const int c = attn_decode_chunk(B);
  return (c >= 512 && (long)attn_decode_splits(ctx_cap, 2 * c) * B * hkv >= 4096) ? 2 * c : c;
}

template <int DH, bool NT>
void attn_decode_fmt(const AttnDecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (a.kv_fmt) {
    case KV_F32: k_attn_decode<DH, KV_F32, NT><<<grid, 256, 0, s>>>(a); break;
    case KV_F16: k_attn_decode<DH, KV_F16, NT><<<grid, 256, 0, s>>>(a); break;
    default: k_attn_decode<DH, KV_BF16, NT><<<grid, 256, 0, s>>>(a); break;
  }
  k_attn_merge<DH><<<dim3(a.hq, a.B), DH, 0, s>>>(a);
}

template <int DH>
void attn_prefill_fmt(const AttnPrefillArgs& a, dim3 grid, hipStream_t s) {
  // at most one work-group per CU: three LDS tile buffers for a 2-byte cache
  const bool deep = (long)grid.x * grid.y <= 256;
  switch (a.kv_fmt) {
    case KV_F32: k_attn_prefill<DH, KV_F32, 2><<<grid, 256, 0, s>>>(a); break;
    case KV_F16:
      if (deep) k_attn_prefill<DH, KV_F16, 3><<<grid, 256, 0, s>>>(a);
      else k_attn_prefill<DH, KV_F16, 2><<<grid, 256, 0, s>>>(a);
      break;
    default:
      if (deep) k_attn_prefill<DH, KV_BF16, 3><<<grid, 256, 0, s>>>(a);
      else k_attn_prefill<DH, KV_BF16, 2><<<grid, 256, 0, s>>>(a);
      break;
  }
}

hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s) {
  // splits of a full-length row (every row holds at most ctx_cap keys); never more than allocated
  const int ns = attn_decode_splits(a.ctx_cap, a.chunk);
  if (ns > a.nsplit) return hipErrorInvalidValue;
  dim3 grid(ns, a.hkv, a.B);
  // non-temporal K/V loads for batched decode: 70B-shaped B = 128 at ctx 8192 14.5 -> 14.1 ms per
  // step, 8B-shaped B = 64 at ctx 4096 3.16 -> 3.09 ms; at B = 1 (8B, ctx 512..2048) 11.3 -> 12.2 us
  const bool nt = a.B > 4;
  if (a.dh == 128) {
    if (nt) attn_decode_fmt<128, true>(a, grid, s);
    else attn_decode_fmt<128, false>(a, grid, s);
  } else {
    if (nt) attn_decode_fmt<64, true>(a, grid, s);
    else attn_decode_fmt<64, false>(a, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  // 2-byte caches with at least two work-groups per CU at 128 columns each: 32 columns per wave
  // (70B-shaped 4096-token chunk: 18.0 -> 15.3 ms over 20 blocks; 8B-shaped block at T = 4096:
  // 1.25 -> 1.20 ms).  Smaller grids keep 64 columns per work-group, whose twice as many
  // work-groups fill the chip (at T = 512 of the 8B shape the wide kernel had 128: 2% slower,
  // ring-attention chunks 24% slower).
  if (a.kv_fmt != KV_F32 && (long)((a.T * G + 127) / 128) * a.hkv >= 512) {
    dim3 grid((a.T * G + 127) / 128, a.hkv);
    if (a.dh == 128) {
      if (a.kv_fmt == KV_F16) k_attn_prefill32<128, KV_F16><<<grid, 256, 0, s>>>(a);
      else k_attn_prefill32<128, KV_BF16><<<grid, 256, 0, s>>>(a);
    } else {
      if (a.kv_fmt == KV_F16) k_attn_prefill32<64, KV_F16><<<grid, 256, 0, s>>>(a);
      else k_attn_prefill32<64, KV_BF16><<<grid, 256, 0, s>>>(a);
    }
    return hipGetLastError();
  }
  dim3 grid((a.T * G + 63) / 64, a.hkv);
  if (a.dh == 128) attn_prefill_fmt<128>(a, grid, s);
  else attn_prefill_fmt<64>(a, grid, s);
  return hipGetLastError();
}

hipError_t launch_ring_merge(float* acc_o, float* acc_lse, const float* part_o, const float* part_lse, int rows,
                             int hq, int dh, int first, hipStream_t s) {
  const unsigned n = (unsigned)rows * hq;
  if (n == 0) return hipSuccess;
  if (dh == 128) k_ring_merge<128><<<n, 128, 0, s>>>(acc_o, acc_lse, part_o, part_lse, first);
  else k_ring_merge<64><<<n, 64, 0, s>>>(acc_o, acc_lse, part_o, part_lse, first);
  return hipGetLastError();
}

hipError_t launch_ring_store(const float* acc_o, int rows, int hq, int dh, uint16_t* out, size_t out_ps,
                             hipStream_t s) {
  const unsigned n = (unsigned)rows * hq;
  if (n == 0) return hipSuccess;
  if (dh == 128) k_ring_store<128><<<n, 128, 0, s>>>(acc_o, out, out_ps);
  else k_ring_store<64><<<n, 64, 0, s>>>(acc_o, out, out_ps);
  return hipGetLastError();
}
