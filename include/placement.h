/*
 * placement.h -- where a model's blocks go: one contiguous stage per device (host only).
 *
 * Sources (page title, section):
 *  - "RFC: pipeline placement across multiple GPUs for models larger than one device",
 *    Heterogeneous GPUs: a placement is valid only if every stage's requirement fits its own
 *    device's usable budget, device by device (never the sum of the budgets against the sum of the
 *    model); an asymmetric split is chosen when budgets differ; a model that fits nowhere gets
 *    the typed DoesNotFit result (Larger-than-single-card proof).
 *  - "Multi-node layer splitting and tensor parallelism" (TensorSharp), Supported stage
 *    executors: placement balances estimated resident bytes, keeps each node's layers contiguous,
 *    gives every selected GPU at least one layer, and counts the embedding/output endpoints.
 *
 * Reading adopted: the requirement of a stage is stage_plan()'s total_bytes for that block range
 * (weights with the embedding on the first stage and final norm + readout on the last, KV for
 * every slot and position, tables, workspace).  Among valid placements the one whose most-filled
 * device has the lowest requirement / budget ratio is chosen -- byte balance when budgets are
 * equal, proportional when they differ.  Among placements with the same ratio, each device's
 * first block is the smallest that still reaches the optimum, fixed from the last device
 * backwards.  Ratios are compared exactly (integer cross products).
 */
#ifndef PIPELINE_STAGE_DECODER_PLACEMENT_H
#define PIPELINE_STAGE_DECODER_PLACEMENT_H

#include "stage.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Split blocks [0, model->n_blocks_total) over n_devices devices in pipeline order.
 *   shape:    max_slots, max_ctx, max_tokens and the STAGE_KV_F32 flag every stage will be
 *             created with (its block range and FIRST / LAST flags are ignored)
 *   budgets:  host [n_devices], usable bytes of each device
 *   cuts:     host [n_devices + 1]; device i gets blocks [cuts[i], cuts[i + 1]), cuts[0] = 0,
 *             cuts[n_devices] = n_blocks_total, every range non-empty; device 0 embeds, the last
 *             device holds the final norm and readout
 *   required: host [n_devices] (nullable), stage_plan total_bytes of each chosen stage
 * STAGE_E_DOES_NOT_FIT when no contiguous placement fits every budget; STAGE_E_INVALID for bad
 * arguments or more devices than blocks; STAGE_E_UNSUPPORTED when stage_plan refuses the model. */
int stage_place(const stage_model_cfg* model, const stage_stage_cfg* shape, int n_devices,
                const uint64_t* budgets /*host*/, int32_t* cuts /*host*/, uint64_t* required /*host*/);

#ifdef __cplusplus
}
#endif
#endif
