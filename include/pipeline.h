/*
 * pipeline.h -- greedy generation through an ordered chain of pipeline stages on one device, with
 * several micro-batches in flight.
 *
 * Source (page title, section): "41. Many GPUs: tensor, pipeline, expert and data parallelism",
 * Pipeline parallelism.  With one batch in flight, each of p stages works while the others wait
 * (busy 1/p of the time).  The remedy keeps p batches in flight, each a step behind the one ahead,
 * and no two of them share a request.  Only the residual stream crosses a stage boundary, and the
 * last stage can keep the head and hand back sampled tokens instead of hidden rows.
 *
 * Here every stage gets its own HIP stream.  Micro-batch m's work on stage k waits (HIP event)
 * for m's work on stage k - 1; stage 0's next decode step for m waits for m's sampled tokens from
 * the last stage.  Different micro-batches therefore overlap across stages, while one stage's
 * calls stay in order on its stream (a stage handle is never used by two streams at once).  The
 * F32 hidden rows stay in device buffers of the workspace: a stage reads its predecessor's output
 * in place.
 *
 * Conventions: as in stage.h (int status, device pointers unless marked host, nothing allocated
 * on the device by the library).
 */
#ifndef PIPELINE_STAGE_DECODER_PIPELINE_H
#define PIPELINE_STAGE_DECODER_PIPELINE_H

#include "stage.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t n_micro;    /* micro-batches in flight (>= 1) */
  int32_t rows;       /* sequences per micro-batch (>= 1); the decode rows of one stage call */
  int32_t prompt_len; /* prompt tokens of every sequence (>= 1) */
  int32_t n_new;      /* tokens generated per sequence (>= 1); the first comes from the prompt's last row */
} stage_gen_cfg;

/* Workspace bytes stage_pipeline_generate needs for this chain and configuration (host only).
 * Validates the chain and configuration exactly as stage_pipeline_generate does. */
int stage_pipeline_workspace(stage_t* const* stages /*host array*/, int n_stages, const stage_gen_cfg* cfg,
                             uint64_t* bytes /*host*/);

/* Greedy generation.  stages[0 .. n_stages) must be one model's stages in order: stages[0] has
 * STAGE_FIRST, stages[n_stages - 1] has STAGE_LAST, each stage's block_end is the next one's
 * block_begin, all on one device, each with max_slots >= n_micro * rows, max_ctx >= prompt_len +
 * n_new - 1 and max_tokens >= max(prompt_len, rows).
 *   prompts:    int32 [n_micro][rows][prompt_len]
 *   tokens_out: int32 [n_micro][n_new][rows]; tokens_out[m][s][r] is sequence (m, r)'s token s,
 *               the argmax of its logits (lowest index on ties; NaN logits never win)
 * Sequence (m, r) uses KV slot m * rows + r on every stage (its previous contents are overwritten
 * at positions 0 .. prompt_len + n_new - 2).  streams: n_stages streams (host array), or NULL to
 * run everything on the default stream (one batch in flight in effect).  Work is enqueued on the
 * streams; the call returns after all of it has completed.  workspace: device memory of at least
 * stage_pipeline_workspace() bytes, 256-byte aligned.  Invalid token ids are caught on the device
 * (stage_device_errors of the first stage). */
int stage_pipeline_generate(stage_t* const* stages /*host array*/, int n_stages, const stage_gen_cfg* cfg,
                            const int32_t* prompts, int32_t* tokens_out, void* workspace,
                            uint64_t workspace_bytes, const hipStream_t* streams /*host array or NULL*/);

#ifdef __cplusplus
}
#endif
#endif
