// Greedy generation through a chain of stages with micro-batches in flight ("41. Many GPUs",
// Pipeline parallelism: p batches of disjoint requests in flight, each a step behind the one
// ahead; the last stage keeps the head and hands back sampled tokens).
//
// Host-side scheduler over the stage C ABI: one HIP stream per stage, one event per (stage,
// micro-batch).  Enqueue order is step-major, then micro-batch, then stage, so when micro-batch m's
// work is enqueued on stage k, the latest record of event (k - 1, m) is m's work on stage k - 1 of
// the same step, and the latest record of event (last, m) is m's previous step.  Waits:
//   * stage k > 0 waits for (k - 1, m): its input rows;
//   * stage 0 waits for (last, m): the tokens it embeds next;
// and a stage's own stream orders its calls.  Every other hazard follows: micro-batch m's buffers
// are written again only after m's previous step has left the last stage, which is after every
// stage read them.
#include <string>
#include <vector>

#include "pipeline.h"

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Chain {
  std::vector<stage_model_cfg> m;
  std::vector<stage_stage_cfg> s;
  int device = -1;
};

struct PipeLayout {
  uint64_t act = 0;       // [n_micro][n_stages + 1][rows * prompt_len * d] F32: stage k reads buffer k, writes k + 1
  uint64_t act_elems = 0; // floats per buffer
  uint64_t last_rows = 0; // [n_micro][rows * d] F32: the prompts' last rows for the first readout
  uint64_t logits = 0;    // [n_micro][rows * V] F32
  uint64_t slots = 0;     // [n_micro * rows] int32
  uint64_t pos = 0;       // [n_new][rows] int32: decode step s at position prompt_len + s - 1
  uint64_t total = 0;
};

int check_chain(stage_t* const* stages, int n, const stage_gen_cfg* cfg, Chain& c) {
  if (!stages || n <= 0 || !cfg) return STAGE_E_INVALID;
  if (cfg->n_micro <= 0 || cfg->rows <= 0 || cfg->prompt_len <= 0 || cfg->n_new <= 0) return STAGE_E_INVALID;
  c.m.resize(n);
  c.s.resize(n);
  for (int k = 0; k < n; ++k) {
    int dev = -1;
    if (!stages[k] || stage_describe(stages[k], &c.m[k], &c.s[k], &dev) != STAGE_OK) return STAGE_E_INVALID;
    if (k == 0) c.device = dev;
    if (dev != c.device) return STAGE_E_UNSUPPORTED;
  }
  if (!(c.s[0].flags & STAGE_FIRST) || !(c.s[n - 1].flags & STAGE_LAST)) return STAGE_E_ROLE;
  const int64_t seqs = (int64_t)cfg->n_micro * cfg->rows;
  const int64_t last_pos = (int64_t)cfg->prompt_len + cfg->n_new - 1;   // positions used: [0, last_pos)
  for (int k = 0; k < n; ++k) {
    const stage_model_cfg& a = c.m[k];
    const stage_model_cfg& b = c.m[0];
    if (a.d_model != b.d_model || a.vocab != b.vocab || a.n_q_heads != b.n_q_heads ||
        a.n_kv_heads != b.n_kv_heads || a.head_dim != b.head_dim || a.d_ffn != b.d_ffn ||
        a.n_blocks_total != b.n_blocks_total)
      return STAGE_E_INVALID;
    if (k + 1 < n && c.s[k].block_end != c.s[k + 1].block_begin) return STAGE_E_INVALID;
    if (k > 0 && (c.s[k].flags & STAGE_FIRST)) return STAGE_E_ROLE;
    if (k + 1 < n && (c.s[k].flags & STAGE_LAST)) return STAGE_E_ROLE;
    if (c.s[k].max_slots < seqs || c.s[k].max_ctx < last_pos) return STAGE_E_RANGE;
    if (c.s[k].max_tokens < cfg->prompt_len || c.s[k].max_tokens < cfg->rows) return STAGE_E_INVALID;
  }
  return STAGE_OK;
}

PipeLayout layout(const Chain& c, int n, const stage_gen_cfg* cfg) {
  PipeLayout L;
  const uint64_t d = (uint64_t)c.m[0].d_model, V = (uint64_t)c.m[0].vocab;
  const uint64_t nm = (uint64_t)cfg->n_micro, rows = (uint64_t)cfg->rows;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t at = off;
    off = align_up(off + bytes);
    return at;
  };
  L.act_elems = align_up(rows * (uint64_t)cfg->prompt_len * d * 4) / 4;
  L.act = take(nm * (uint64_t)(n + 1) * L.act_elems * 4);
  L.last_rows = take(nm * rows * d * 4);
  L.logits = take(nm * rows * V * 4);
  L.slots = take(nm * rows * 4);
  L.pos = take((uint64_t)cfg->n_new * rows * 4);
  L.total = off;
  return L;
}

}  // namespace

extern "C" int stage_pipeline_workspace(stage_t* const* stages, int n_stages, const stage_gen_cfg* cfg,
                                        uint64_t* bytes) {
  Chain c;
  const int rc = check_chain(stages, n_stages, cfg, c);
  if (rc != STAGE_OK) return rc;
  if (!bytes) return STAGE_E_INVALID;
  *bytes = layout(c, n_stages, cfg).total;
  return STAGE_OK;
}

extern "C" int stage_pipeline_generate(stage_t* const* stages, int n_stages, const stage_gen_cfg* cfg,
                                       const int32_t* prompts, int32_t* tokens_out, void* workspace,
                                       uint64_t workspace_bytes, const hipStream_t* streams) {
  Chain c;
  int rc = check_chain(stages, n_stages, cfg, c);
  if (rc != STAGE_OK) return rc;
  if (!prompts || !tokens_out || !workspace) return STAGE_E_INVALID;
  const PipeLayout L = layout(c, n_stages, cfg);
  if (workspace_bytes < L.total || reinterpret_cast<uintptr_t>(workspace) % kAlign != 0) return STAGE_E_DOES_NOT_FIT;
  if (hipSetDevice(c.device) != hipSuccess) return STAGE_E_HIP;

  const int n = n_stages, nm = cfg->n_micro, rows = cfg->rows, T = cfg->prompt_len, n_new = cfg->n_new;
  const int d = c.m[0].d_model, V = c.m[0].vocab;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  auto act = [&](int m, int k) { return reinterpret_cast<float*>(ws + L.act) + ((size_t)m * (n + 1) + k) * L.act_elems; };
  float* last_rows = reinterpret_cast<float*>(ws + L.last_rows);
  float* logits = reinterpret_cast<float*>(ws + L.logits);
  int32_t* slots = reinterpret_cast<int32_t*>(ws + L.slots);
  int32_t* pos = reinterpret_cast<int32_t*>(ws + L.pos);
  auto S = [&](int k) { return streams ? streams[k] : (hipStream_t)0; };

  // slot and position tables (synchronous host -> device copies before any stream work)
  {
    std::vector<int32_t> hs((size_t)nm * rows), hp((size_t)n_new * rows);
    for (size_t i = 0; i < hs.size(); ++i) hs[i] = (int32_t)i;
    for (int s = 0; s < n_new; ++s)
      for (int r = 0; r < rows; ++r) hp[(size_t)s * rows + r] = T + s - 1;
    if (hipMemcpy(slots, hs.data(), hs.size() * 4, hipMemcpyHostToDevice) != hipSuccess ||
        hipMemcpy(pos, hp.data(), hp.size() * 4, hipMemcpyHostToDevice) != hipSuccess)
      return STAGE_E_HIP;
  }

  std::vector<hipEvent_t> done((size_t)n * nm, nullptr);
  for (auto& e : done)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
      rc = STAGE_E_HIP;
      break;
    }
  auto ev = [&](int k, int m) { return done[(size_t)k * nm + m]; };

#define PIPE_TRY(expr)                  \
  do {                                  \
    if (rc == STAGE_OK) {               \
      const int _r = (expr);            \
      if (_r != STAGE_OK) rc = _r;      \
    }                                   \
  } while (0)
#define PIPE_HIP(expr)                                                  \
  do {                                                                  \
    if (rc == STAGE_OK && (expr) != hipSuccess) rc = STAGE_E_HIP;       \
  } while (0)

  // step 0: every sequence's prompt through the chain; the last stage samples token 0
  for (int m = 0; m < nm && rc == STAGE_OK; ++m) {
    for (int k = 0; k < n; ++k) {
      const hipStream_t st = S(k);
      if (k > 0) PIPE_HIP(hipStreamWaitEvent(st, ev(k - 1, m), 0));
      for (int r = 0; r < rows; ++r) {
        const size_t ro = (size_t)r * T * d;
        if (k == 0) PIPE_TRY(stage_embed(stages[0], T, prompts + ((size_t)m * rows + r) * T, act(m, 0) + ro, st));
        PIPE_TRY(stage_prefill(stages[k], m * rows + r, 0, T, act(m, k) + ro, act(m, k + 1) + ro, st));
      }
      if (k == n - 1) {
        float* lr = last_rows + (size_t)m * rows * d;
        PIPE_HIP(hipMemcpy2DAsync(lr, (size_t)d * 4, act(m, n) + (size_t)(T - 1) * d, (size_t)T * d * 4,
                                  (size_t)d * 4, rows, hipMemcpyDeviceToDevice, st));
        float* lg = logits + (size_t)m * rows * V;
        PIPE_TRY(stage_readout(stages[k], rows, lr, lg, nullptr, st));
        PIPE_TRY(stage_greedy(rows, V, lg, tokens_out + (size_t)m * n_new * rows, st));
      }
      PIPE_HIP(hipEventRecord(ev(k, m), st));
    }
  }
  // steps 1 .. n_new - 1: one decode row per sequence
  for (int s = 1; s < n_new && rc == STAGE_OK; ++s) {
    for (int m = 0; m < nm; ++m) {
      for (int k = 0; k < n; ++k) {
        const hipStream_t st = S(k);
        PIPE_HIP(hipStreamWaitEvent(st, k == 0 ? ev(n - 1, m) : ev(k - 1, m), 0));
        if (k == 0)
          PIPE_TRY(stage_embed(stages[0], rows, tokens_out + ((size_t)m * n_new + s - 1) * rows, act(m, 0), st));
        PIPE_TRY(stage_decode(stages[k], rows, slots + (size_t)m * rows, pos + (size_t)s * rows, act(m, k),
                              act(m, k + 1), st));
        if (k == n - 1) {
          float* lg = logits + (size_t)m * rows * V;
          PIPE_TRY(stage_readout(stages[k], rows, act(m, n), lg, nullptr, st));
          PIPE_TRY(stage_greedy(rows, V, lg, tokens_out + ((size_t)m * n_new + s) * rows, st));
        }
        PIPE_HIP(hipEventRecord(ev(k, m), st));
      }
    }
  }
#undef PIPE_TRY
#undef PIPE_HIP

  // wait for everything enqueued so far (also after a failure part-way), then release the events
  for (int k = 0; k < n; ++k)
    if (hipStreamSynchronize(S(k)) != hipSuccess && rc == STAGE_OK) rc = STAGE_E_HIP;
  for (auto e : done)
    if (e) (void)hipEventDestroy(e);
  return rc;
}
