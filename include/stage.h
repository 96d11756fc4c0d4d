/*
 * stage.h -- C ABI of one pipeline stage of a decoder-only transformer on an MI355X (gfx950).
 *
 * A stage owns a contiguous, half-open range of GLOBAL block ids [block_begin, block_end) with its
 * own weights and per-slot KV cache, takes F32 hidden rows in and gives F32 hidden rows out.  The
 * first stage also embeds tokens; the last stage also applies the final RMSNorm and the readout.
 *
 * Sources (page title, section):
 *  - "RFC: pipeline placement across multiple GPUs for models larger than one device",
 *    What I found / Proposed architecture: each stage owns its resident weights, KV state, heap and
 *    workspace; only the hidden activation crosses the boundary; a step is accepted only after all
 *    stages succeed; a placement is a global block range with weight roles, a state plan and a
 *    resource plan; a model that does not fit returns a typed DoesNotFit.
 *  - "41. Many GPUs: tensor, pipeline, expert and data parallelism", Pipeline parallelism
 *    (PipelineStage.forward): embed on the first stage, per block add_norm -> attention ->
 *    add_norm -> MLP, the residual x + delta is what crosses, final norm at the end; Tensor
 *    parallelism: [out, in] weights, GQA head map h // (Hq / Hkv), MLP down(silu(gate) * up);
 *    Ring attention: causal attention with keys k_pos > q_pos masked, split-KV merge by LSE.
 *  - "Multi-node layer splitting and tensor parallelism" (TensorSharp), Supported stage executors:
 *    the dense pipeline hands F32 hidden activations; each stage loads only its layer weights and
 *    KV state; the first embeds, the last computes logits; unsupported families are refused before
 *    any GPU allocation.
 *
 * Conventions for every entry point:
 *  - Return an int status (STAGE_OK or a STAGE_E_* code); nothing throws across the ABI.
 *  - Pointers are DEVICE pointers unless marked "host".  Buffers are caller-owned, contiguous and
 *    row-major; the stage keeps no pointer to them after the call returns.
 *  - All device work is enqueued asynchronously on the given hipStream_t (0 = default stream);
 *    a call returns once the work is enqueued.  Arguments are validated on the host before any
 *    work is enqueued; a call that fails validation enqueues nothing.
 *  - Positions and sequence lengths belong to the caller and are passed with every call.  A call
 *    writes KV only at the positions it is given, so a failed step is retried at the same
 *    positions, and "reset"/"truncate" are rewinds of the caller's positions.
 *  - One host thread per handle; calls that overlap on one handle are not supported.
 *  - Values that only the device sees (token ids, decode slots and positions) are checked on the
 *    device and nothing is ever written out of bounds.  An out-of-range token id gives a zero
 *    embedding row and counts one device error (stage_device_errors).  A decode row whose slot or
 *    position is out of range writes no K/V and attends to no key: its attention output is zero,
 *    so each block passes it on as x + MLP(x); it counts one device error per block.  Its output
 *    is therefore defined but meaningless, and the other rows of the call are unaffected.
 *  - Activations enter the matrix products as a bf16 "hi" plane and a bf16 "lo" plane
 *    (hi = bf16(v), lo = bf16(v - hi): about 16 significant bits), weights as their bf16 values,
 *    with F32 accumulation; norms and RoPE are evaluated in float64.  Over a 2-byte KV cache the
 *    products whose outputs are rounded into the cache (the K and V rows of the QKV projection)
 *    take a third plane (bf16(v - hi - lo), about 24 bits).  The decode projections for up to 4
 *    rows take the F32 activation directly.  No activation is rounded to bf16 alone.
 */
#ifndef PIPELINE_STAGE_DECODER_STAGE_H
#define PIPELINE_STAGE_DECODER_STAGE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------------- */
enum {
  STAGE_OK = 0,
  STAGE_E_INVALID = 1,      /* null pointer, non-positive size, T or B above max_tokens */
  STAGE_E_UNSUPPORTED = 2,  /* configuration refused before any allocation */
  STAGE_E_DOES_NOT_FIT = 3, /* arena_bytes below the plan's total_bytes */
  STAGE_E_ROLE = 4,         /* embed off the first stage, readout off the last, role/block outside range */
  STAGE_E_RANGE = 5,        /* slot >= max_slots, pos0 + T > max_ctx, n_elems wrong for the role */
  STAGE_E_HIP = 6           /* a HIP call or kernel launch failed; stage_last_error() has the text */
};

/* ---- configuration -------------------------------------------------------------------------- */
/* Decoder dimensions (identical on every stage of one model). */
typedef struct {
  int32_t d_model;        /* hidden width d; multiple of 64 */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 and Hq / Hkv <= 16 */
  int32_t head_dim;       /* Dh in {64, 128} */
  int32_t d_ffn;          /* SwiGLU width F; multiple of 16 */
  int32_t vocab;          /* V */
  int32_t n_blocks_total; /* blocks of the whole model */
  float rms_eps;          /* RMSNorm epsilon (inside the square root) */
  float rope_theta;       /* RoPE base; angle(pos, i) = pos * theta^(-2i/Dh) */
} stage_model_cfg;

#define STAGE_FIRST 1u  /* owns the token embedding */
#define STAGE_LAST 2u   /* owns the final RMSNorm and the readout */
#define STAGE_KV_F32 4u /* F32-grade KV cache instead of bf16 (twice the bytes): each K/V value
                           is kept as a bf16 hi + lo pair (~16 significant bits), the two planes
                           attention multiplies, split once when the value is written.  With bf16,
                           a K/V value that a float64 reference and the GPU's f32 sums put on
                           different sides of a bf16 rounding boundary perturbs attention, which
                           flips more roundings in later blocks; the pair keeps a deep stage
                           within 1e-3 of a float64 reference. */
#define STAGE_KV_F16 8u /* IEEE binary16 KV cache (2 bytes per value, the cache precision of the
                           TensorSharp runs, "Measured on two SSH-connected nodes": F16 KV).
                           Eleven significant bits instead of bf16's eight make the rounding
                           flips above eight times rarer and smaller: a 16- or 20-block stage stays
                           within 1e-3 of a float64 reference at bf16's byte cost.  Attention
                           multiplies it on binary16 MFMAs with q and the probabilities carried as
                           binary16 hi + lo planes.  Values must lie in binary16's range (|v| <=
                           65504).  Exclusive with STAGE_KV_F32. */

typedef struct {
  int32_t block_begin; /* first GLOBAL block id (inclusive) */
  int32_t block_end;   /* one past the last GLOBAL block id; block_begin <= block_end */
  uint32_t flags;      /* STAGE_FIRST | STAGE_LAST | at most one of STAGE_KV_F32, STAGE_KV_F16 */
  int32_t max_slots;   /* KV slots (sequences) */
  int32_t max_ctx;     /* positions per slot: every position used is < max_ctx */
  int32_t max_tokens;  /* rows per call: prefill T and decode B are <= max_tokens */
} stage_stage_cfg;

typedef struct {
  uint64_t weight_bytes;    /* bf16 matrices, F32 norm gains */
  uint64_t kv_bytes;        /* K and V (2 bytes per value; 4 with STAGE_KV_F32) for every owned block and slot */
  uint64_t table_bytes;     /* RoPE cos/sin table (float64) */
  uint64_t workspace_bytes; /* per-call activations, split-K and split-KV partials, error counter */
  uint64_t total_bytes;     /* arena size stage_create needs (sum of the above with alignment) */
} stage_plan_t;

typedef struct stage stage_t;

/* ---- weight roles ----------------------------------------------------------------------------- */
/* Every matrix is bf16 [out, in] row-major (the nn.Linear layout); gains are bf16 [d]. */
enum {
  STAGE_ROLE_EMBED = 0,      /* [V, d], first stage, global_block = -1 */
  STAGE_ROLE_ATTN_NORM = 1,  /* [d] */
  STAGE_ROLE_WQ = 2,         /* [Hq*Dh, d] */
  STAGE_ROLE_WK = 3,         /* [Hkv*Dh, d] */
  STAGE_ROLE_WV = 4,         /* [Hkv*Dh, d] */
  STAGE_ROLE_WO = 5,         /* [d, Hq*Dh] */
  STAGE_ROLE_MLP_NORM = 6,   /* [d] */
  STAGE_ROLE_WGATE = 7,      /* [F, d] */
  STAGE_ROLE_WUP = 8,        /* [F, d] */
  STAGE_ROLE_WDOWN = 9,      /* [d, F] */
  STAGE_ROLE_FINAL_NORM = 10,/* [d], last stage, global_block = -1 */
  STAGE_ROLE_READOUT = 11    /* [V, d], last stage, global_block = -1 (untied from the embedding) */
};

/* ---- entry points ------------------------------------------------------------------------------ */

/* Byte plan of a stage (host only, no GPU call): its resource plan -- weights, KV state, tables
 * and workspace -- as one allocation domain ("RFC: pipeline placement ...", What I found: a fit is
 * assessed against one allocation domain including state and workspace; Proposed architecture:
 * a stage placement carries a state plan and a resource plan).  The arena of stage_create must
 * hold out->total_bytes.  STAGE_E_UNSUPPORTED for a configuration the kernels do not cover
 * (checked before anything is allocated), STAGE_E_INVALID for a malformed one. */
int stage_plan(const stage_model_cfg* model, const stage_stage_cfg* stage, stage_plan_t* out /*host*/);

/* Create a stage inside a caller-allocated device arena (e.g. a torch uint8 tensor) on device
 * `device` ("RFC: pipeline placement ...", What I found: each stage owns its resident weights, KV
 * state, heap and workspace, with no allocator shared between stages; TensorSharp, Supported
 * stage executors: an unsupported configuration is refused before any GPU allocation).  The stage sub-allocates weights, KV cache, tables and workspace inside the arena and
 * never allocates device memory itself.  The arena must stay allocated until stage_destroy.
 * Zero-fills the KV cache and uploads the RoPE table synchronously.  *out receives a host handle.
 * STAGE_E_DOES_NOT_FIT if arena_bytes < plan.total_bytes. */
int stage_create(const stage_model_cfg* model, const stage_stage_cfg* stage, void* arena,
                 uint64_t arena_bytes, int device, stage_t** out);

/* Copy one weight tensor into the stage (TensorSharp, Supported stage executors: each stage loads
 * only its own layers' weights; "RFC: pipeline placement ...", Proposed architecture: weight roles
 * over a global block range).  src: bf16 bits in the role's [out, in] layout, host or
 * device memory; n_elems must equal the role's element count.  global_block is the GLOBAL block
 * id for per-block roles (inside [block_begin, block_end)) and -1 for EMBED/FINAL_NORM/READOUT.
 * The stage stores its own layout (fused QKV, interleaved gate/up, F32 gains).  Host sources are
 * copied synchronously; device sources are copied on `stream`. */
int stage_load_weight(stage_t* st, int role, int global_block, const uint16_t* src, uint64_t n_elems,
                      hipStream_t stream);

/* First stage: hidden_out[i, :] = f32(E[tokens[i], :]) for i < n (exact bf16 -> f32)
 * ("41. Many GPUs", Pipeline parallelism: the first stage embeds the tokens; TensorSharp,
 * Supported stage executors: the first stage embeds).  STAGE_E_ROLE off the first stage. */
int stage_embed(stage_t* st, int n, const int32_t* tokens, float* hidden_out, hipStream_t stream);

/* Prefill (or a prefill chunk) of T rows of one slot at positions pos0 .. pos0+T-1: runs every
 * owned block over hidden_in [T, d] (F32), writes K/V at those positions, attends causally over
 * positions [0, pos0 + t] for row t, and writes the stage output residual to hidden_out [T, d]
 * ("41. Many GPUs", Pipeline parallelism: each block adds attention and then the MLP to the
 * residual stream, which alone crosses to the next stage; Ring attention for very long contexts:
 * a key is visible to a query unless its position is later; TensorSharp, Supported stage
 * executors: F32 hidden activations at the boundary; Reproducible validation: full and chunked
 * prefill).  hidden_out may equal hidden_in.  Positions below pos0 must hold KV written earlier.
 * STAGE_E_RANGE if slot >= max_slots or pos0 + T > max_ctx; STAGE_E_INVALID if T > max_tokens. */
int stage_prefill(stage_t* st, int slot, int pos0, int T, const float* hidden_in, float* hidden_out,
                  hipStream_t stream);

/* One decode step for B rows: row b is slot slots[b] at position positions[b] (device int32
 * arrays; slots distinct), attending over positions [0, positions[b]].  hidden_in/out [B, d] F32;
 * hidden_out may equal hidden_in ("41. Many GPUs", Pipeline parallelism: one token per sequence
 * through the blocks; "RFC: pipeline placement ...", What I found: a decode step is accepted only
 * after every stage has completed it, so the caller owns positions and retries a failed step at
 * the same ones).  The kernel schedule depends only on B, the shapes and max_ctx, so the call can
 * be captured in a HIP graph and replayed with new slots/positions.  Out-of-range slots or
 * positions are handled per row on the device (see the conventions above). */
int stage_decode(stage_t* st, int B, const int32_t* slots, const int32_t* positions,
                 const float* hidden_in, float* hidden_out, hipStream_t stream);

/* Last stage: h = RMSNorm(hidden_in) * g_final, written to normed_out as the F32 "final hidden"
 * (nullable), and logits_out [n, V] (F32) = h W_readout^T, h entering the product as its bf16 hi
 * and lo planes ("41. Many GPUs", Pipeline parallelism: the final norm follows the last block;
 * TensorSharp, Supported stage executors: the last stage computes logits; "RFC: pipeline
 * placement ...", Numerical correctness proof: full logits and final features are the outputs
 * compared).  STAGE_E_ROLE off the last stage. */
int stage_readout(stage_t* st, int n, const float* hidden_in, float* logits_out, float* normed_out,
                  hipStream_t stream);

/* SwiGLU MLP of one owned block without its residual: out [n, d] (F32) = W_down a with
 * a = silu(W_gate h) * (W_up h) and h = RMSNorm(hidden_in) * g_mlp, each entering its product as
 * bf16 hi and lo planes.  With accumulate != 0
 * the result is added to out (out = out + W_down a, one F32 add per element), so calling it over
 * column/row slices of one MLP in slice order sums the partials as ((p0 + p1) + p2) + ...
 * ("41. Many GPUs", Tensor parallelism: take_rows / take_cols and the one all-reduce per MLP;
 * TensorSharp, Transport and tuning: node-order summation). */
int stage_mlp(stage_t* st, int global_block, int n, const float* hidden_in, float* out, int accumulate,
              hipStream_t stream);

/* Attention sublayer of one owned block without its residual, for T rows of one slot at positions
 * pos0 .. pos0+T-1 (as in stage_prefill: K/V written there, row t attends positions
 * [0, pos0 + t]): out [T, d] (F32) = W_o attention(q, K, V) with q, k, v from
 * h = RMSNorm(hidden_in) g_attn.  With accumulate != 0 the result is added to out (one F32 add
 * per element), so stages holding head slices of one attention block -- their query heads' rows
 * of W_q, their KV heads' rows of W_k / W_v, the matching columns of W_o -- called in slice order
 * sum the partials as ((p0 + p1) + p2) + ... ("41. Many GPUs", Tensor parallelism: Q, K, V
 * column-parallel by heads, W_o row-parallel, one all-reduce per attention). */
int stage_attn(stage_t* st, int global_block, int slot, int pos0, int T, const float* hidden_in, float* out,
               int accumulate, hipStream_t stream);

/* Context-parallel (ring) form of stage_attn for a whole sequence of T rows at positions 0..T-1 of
 * one slot ("41. Many GPUs", Ring attention for very long contexts): the sequence is cut into
 * n_ranks chunks (zigzag != 0: 2 n_ranks chunks, rank r holding chunks r and 2 n_ranks - 1 - r);
 * each rank attends its queries to the K/V chunks it holds at each hop h (those of rank
 * (r - h) mod n_ranks), and the partial results merge in hop order by their log-sum-exp -- the
 * split-KV merge.  On one device the ranks run one after another over the slot's cache; the result
 * equals stage_attn's up to F32 rounding of the merges.  T must be a multiple of the chunk count.
 * workspace: device memory of stage_attn_ring_workspace() bytes, 256-byte aligned. */
int stage_attn_ring_workspace(const stage_t* st, int T, uint64_t* bytes /*host*/);
int stage_attn_ring(stage_t* st, int global_block, int slot, int T, int n_ranks, int zigzag, const float* hidden_in,
                    float* out, int accumulate, void* workspace, uint64_t workspace_bytes, hipStream_t stream);

/* stage_attn_ring without the workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation): the hops'
 * partials and their running merge live in a device array inside the library, 32 MiB per GPU, held
 * from the first stage_create on that GPU until the process ends.  It allocates nothing and is
 * otherwise stage_attn_ring (the same kernels, bit-identical results).  Calls whose workspace
 * (stage_attn_ring_workspace) would exceed 32 MiB -- 8 (Dh + 1) bytes per (row, query head), so
 * about 1000 rows for 32 query heads of dim 128 -- are refused with STAGE_E_DOES_NOT_FIT before
 * anything is enqueued.  Every call on one GPU shares that array: calls that overlap on one GPU
 * (other streams, other handles, other threads) race and must be serialised by the caller.
 * Nothing in the array needs to start at zero, and each call overwrites what it uses. */
int stage_attn_ring_noalloc(stage_t* st, int global_block, int slot, int T, int n_ranks, int zigzag,
                            const float* hidden_in, float* out, int accumulate, hipStream_t stream);

/* Embedding of a vocabulary slice on a first stage: the stage's table holds ids
 * [vocab_lo, vocab_lo + V) of a larger vocabulary.  hidden_out[i, :] = (accumulate ? hidden_out[i, :]
 * : 0) + (tokens[i] inside ? E[tokens[i] - vocab_lo, :] : 0), so slices called in order assemble
 * every token's row ("41. Many GPUs", Tensor parallelism: a vocabulary-parallel embedding looks up
 * zeros outside its slice and the all-reduce sums the slices).  Negative ids count as device
 * errors. */
int stage_embed_range(stage_t* st, int n, const int32_t* tokens, int vocab_lo, float* hidden_out, int accumulate,
                      hipStream_t stream);

/* Copy KV positions [0, n_pos) of every owned block from src_slot to dst_slot, e.g. to give many
 * sequences one shared context ("RFC: pipeline placement ...", What I found: the KV state is the
 * stage's own and never crosses the boundary).  STAGE_E_RANGE for a slot or n_pos out of range. */
int stage_kv_copy(stage_t* st, int src_slot, int dst_slot, int n_pos, hipStream_t stream);

/* Write / read KV of one owned block and slot at positions [pos0, pos0+n): k, v are device
 * [n, Hkv, Dh] arrays -- bf16 bits, or F32 with STAGE_KV_F32 (imported values are split into the
 * cache's hi + lo pair; exported values are hi + lo) -- with K after RoPE, as attention reads it. */
int stage_kv_import(stage_t* st, int global_block, int slot, int pos0, int n, const void* k, const void* v,
                    hipStream_t stream);
int stage_kv_export(stage_t* st, int global_block, int slot, int pos0, int n, void* k, void* v,
                    hipStream_t stream);

/* Greedy sampling: tokens_out[i] = argmax_j logits[i, j] over j < V for i < n, the lowest index
 * on ties ("41. Many GPUs", Measured: the greedy driver's argmax of the last row's logits).  NaN
 * never wins (a row of NaN and -inf gives 0).  Needs no stage handle. */
int stage_greedy(int n, int V, const float* logits, int32_t* tokens_out, hipStream_t stream);

/* The configuration a handle was created with (host copies) and its device. */
int stage_describe(const stage_t* st, stage_model_cfg* model /*host*/, stage_stage_cfg* stage /*host*/,
                   int* device /*host*/);

/* Device-side error counter (rows skipped for out-of-range tokens, slots or positions); reading it
 * synchronises `stream`.  reset != 0 clears it afterwards. */
int stage_device_errors(stage_t* st, int reset, uint32_t* count /*host*/, hipStream_t stream);

/* ---- kernel timing for benchmarks ------------------------------------------------------------
 * When enabled for a set of kernel kinds, the stage records a HIP event pair on the call's stream
 * around every launch of those kinds and keeps the pairs until they are read.  Off by default;
 * the events add a few microseconds per timed launch.  Not for use while a stream is being
 * captured into a graph. */
enum {
  STAGE_KT_EMBED = 0,   /* token embedding */
  STAGE_KT_NORM = 1,    /* RMSNorm row pass (MFMA path and readout) */
  STAGE_KT_QKV = 2,     /* QKV projection + RoPE + KV write */
  STAGE_KT_ATTN = 3,    /* attention (decode: partials + merge) */
  STAGE_KT_O = 4,       /* output projection + residual */
  STAGE_KT_GATEUP = 5,  /* gate/up projection + SwiGLU */
  STAGE_KT_DOWN = 6,    /* down projection + residual */
  STAGE_KT_READOUT = 7, /* readout projection */
  STAGE_KT_COUNT = 8
};
/* Enable timing for the kinds whose bit (1u << kind) is set in kind_mask; 0 disables.  Discards
 * any recorded pairs. */
int stage_timing(stage_t* st, uint32_t kind_mask);
/* Launch count and summed duration (ms) of one kind since timing was enabled or last read;
 * waits for the recorded events, then forgets them. */
int stage_timing_read(stage_t* st, int kind, uint64_t* launches /*host*/, double* total_ms /*host*/);

/* Release the handle; the arena, which holds the stage's weights and KV state, stays the
 * caller's ("RFC: pipeline placement ...", What I found: each stage owns its heap and memory
 * accounting, with no allocator shared between stages). */
int stage_destroy(stage_t* st);

const char* stage_status_str(int status);
/* Text of the last STAGE_E_HIP / validation failure on this handle ("" if none). */
const char* stage_last_error(const stage_t* st);

#ifdef __cplusplus
}
#endif
#endif
