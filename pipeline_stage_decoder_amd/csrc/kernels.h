// Launch interfaces of the stage kernels (host side).  Every launcher enqueues on `s` and returns
// the hipError_t of the launch.
#pragma once
#include "common.h"

struct NormArgs {
  const float* x;     // [M][K] f32 rows
  const float* gain;  // [K] f32
  float eps;
  int M, K;
  float* out_f32;     // [M][K] normalised rows x*r*g (nullable)
  uint16_t* out_pair; // three bf16 planes [3][M][K] of x*r*g (hi, mid, lo; nullable)
  size_t pair_ps;     // plane stride
};

struct GemvArgs {
  const float* x;      // [B][K] f32 rows (normalised inside: x*r*g)  -- or null
  const float* gain;   // [K]
  float eps;
  const uint16_t* xb;  // pair buffer [B][K] used as is when x is null
  size_t xb_ps;
  const uint16_t* w;   // [N][K] bf16
  int N, K, B;
  EpiArgs e;
};

struct GemmArgs {
  const uint16_t* a;   // activation planes [planes][M][K] (hi, lo or hi, mid, lo), stride a_ps
  size_t a_ps;
  int planes;          // 2 or 3
  const uint16_t* w;   // [N][K] bf16
  int M, N, K;
  int splitk;          // K splits; each split's K range is a multiple of 64
  float* part;         // [splitk][M][N] f32 partials when splitk > 1
  EpiArgs e;
  int w_stream;        // set by launch_gemm: one row of M-tiles, each weight byte read once
};

struct GemmPlan {
  int cfg;      // tile configuration index
  int bm, bn;
  int splitk;
  int tiles_m, tiles_n;
};

struct AttnDecodeArgs {
  const uint16_t* q;        // pair buffer [B][Hq][Dh] (binary16 planes with KV_F16, else bf16)
  size_t q_ps;
  const void* kc;           // K cache of the block
  const void* vc;           // V cache of the block
  int kv_fmt;               // KvFmt: KV_BF16, KV_F32 (bf16 hi + lo planes per K row / V group) or KV_F16
  const int32_t* slots;     // [B]
  const int32_t* pos;       // [B]; keys [0, pos] are attended
  int B, hq, hkv, dh, ctx_cap, max_slots;
  int chunk;                // keys per split (a row's last split takes the remainder)
  int nsplit;               // splits allocated per row (>= attn_decode_splits of every row)
  float scale_log2;         // Dh^-1/2 * log2(e)
  float* part_o;            // [B][Hq][nsplit][Dh]
  float* part_lse;          // [B][Hq][nsplit]  (base-2 log-sum-exp)
  uint16_t* out;            // merged output, pair buffer [B][Hq*Dh]
  size_t out_ps;
  uint32_t* err;
};

struct AttnPrefillArgs {
  const uint16_t* q;        // pair buffer [T][Hq][Dh]
  size_t q_ps;
  const void* kc;
  const void* vc;
  int kv_fmt;               // KvFmt
  int slot, pos0, T, hq, hkv, dh, ctx_cap;
  float scale_log2;
  uint16_t* out;            // pair buffer [T][Hq*Dh]
  size_t out_ps;
  // keys attended: positions [k_lo, k_hi) that are also <= the query's position (0, INT_MAX: all)
  int k_lo, k_hi;
  // partial mode (non-null): per (row, head) the normalised partial output [T][Hq][Dh] F32 and its
  // base-2 log-sum-exp [T][Hq] (-inf for a row that sees no key) instead of the pair buffer
  float* part_o;
  float* part_lse;
};

// Ring merge of one partial into running (out, lse) F32 accumulators [rows][Hq](*Dh): first != 0
// copies, otherwise the log-sum-exp merge; store_pairs writes the accumulated output as pairs.
hipError_t launch_ring_merge(float* acc_o, float* acc_lse, const float* part_o, const float* part_lse, int rows,
                             int hq, int dh, int first, hipStream_t s);
hipError_t launch_ring_store(const float* acc_o, int rows, int hq, int dh, uint16_t* out, size_t out_ps,
                             hipStream_t s);

// norm / misc
hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t s);
hipError_t launch_embed(const uint16_t* table, int V, int d, const int32_t* tokens, int n, float* out,
                        uint32_t* err, hipStream_t s);
hipError_t launch_embed_range(const uint16_t* table, int V, int d, int lo, const int32_t* tokens, int n, float* out,
                              int accumulate, uint32_t* err, hipStream_t s);
hipError_t launch_bf16_to_f32(const uint16_t* src, float* dst, int n, hipStream_t s);
// k, v: [n][Hkv][Dh] in the cache's element type (bf16 or binary16 bits, copied as they are; or F32,
// split into the F32-grade cache's hi + lo pair when kv_f32 is set)
hipError_t launch_kv_import(void* kc, void* vc, int kv_f32, int hkv, int dh, int ctx_cap, int slot, int pos0,
                            int n, const void* k, const void* v, hipStream_t s);
hipError_t launch_kv_export(const void* kc, const void* vc, int kv_f32, int hkv, int dh, int ctx_cap, int slot,
                            int pos0, int n, void* k, void* v, hipStream_t s);
hipError_t launch_zero_f32(float* p, size_t n, hipStream_t s);
hipError_t launch_argmax(const float* logits, int n, int V, int32_t* out, hipStream_t s);

// decode GEMV (B <= 4)
bool gemv_fits(int B, int K);
hipError_t launch_gemv(const GemvArgs& a, hipStream_t s);

// MFMA GEMM
// planes: bf16 planes of the activation operand (2 or 3); qkv: the QKV epilogue (RoPE + cache stores)
GemmPlan gemm_plan(int M, int N, int K, int planes, bool qkv);
// then_norm (nullable): when the plan splits K, the epilogue is EPI_RESID and M >= 256, the split-K
// sum also writes the RMSNorm of the result rows (then_norm->x is ignored: the rows are e.out) into
// then_norm->out_pair, and *normed (nullable) is set; otherwise *normed is false.
hipError_t launch_gemm(const GemmArgs& a, const GemmPlan& p, hipStream_t s, const NormArgs* then_norm = nullptr,
                       bool* normed = nullptr);

// attention
int attn_decode_chunk(int B);
// Splits of a row that attends n keys in chunks of `chunk`: n / chunk rounded to nearest, at least
// one; split s covers keys [s * chunk, (s + 1) * chunk) except the last, which runs to n.  Every
// split of a multi-split row holds between chunk / 2 and 1.5 chunk keys, so a row of 8193 keys is
// 16 splits of 512 (the last with 513), not 17 with one key in the last.
__host__ __device__ inline int attn_decode_splits(int n, int chunk) {
  const int s = (n + chunk / 2) / chunk;
  return s > 0 ? s : 1;
}
// Keys per split for a decode launch of B rows over Hkv heads in a cache of ctx_cap positions:
// attn_decode_chunk(B), doubled (from 512 up) when the longer splits of a full-length row still
// give at least 4096 work-groups (eight per CU), so that each streams a longer stretch of K and V.
int attn_decode_chunk_for(int B, int hkv, int ctx_cap);
hipError_t launch_attn_decode(const AttnDecodeArgs& a, hipStream_t s);
hipError_t launch_attn_prefill(const AttnPrefillArgs& a, hipStream_t s);
