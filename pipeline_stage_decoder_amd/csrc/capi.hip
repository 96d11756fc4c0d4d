// Host runtime of one pipeline stage: byte plan, arena layout, weight layouts, launch sequence.
//
// One stage = one arena ("RFC: pipeline placement ...", What I found: each stage owns its weights,
// KV state, heap and workspace; there is no unified allocator).  The arena is carved as
//   [weights | KV cache | RoPE table | workspace]
// and every call enqueues kernels on the caller's stream.  The per-block sequence follows
// PipelineStage.forward of "41. Many GPUs" (Pipeline parallelism):
//   norm -> QKV (+RoPE, KV write) -> attention -> O-proj (+residual) -> norm -> gate/up (+SwiGLU)
//   -> down (+residual)
// with rows <= 4 on the GEMV kernels (norm fused in their prologue) and larger row counts on the
// MFMA GEMM (norm as a row pass that writes the bf16 operand).  The kernel schedule depends only
// on the row count and the shapes, never on the block range, so a model split into stages runs
// exactly the kernels of the unsplit model on every block.
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "stage.h"

// Device scratch of the no-allocation ring entry point (stage_attn_ring_noalloc): the partial
// outputs and log-sum-exps of its hops and their running merge.  Each GPU that loads the library
// holds one copy at its own address until the process ends.  In host code `scratch` only names the
// symbol: its device address is looked up once per device (scratch_ptr) and only that is used.
constexpr uint64_t kScratchBytes = 32ull << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr uint64_t kAlign = 256;

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The calling thread's current device must be `device`.  Looks the scratch array's address on that
// device up on first use and keeps it; nullptr if the lookup fails or the device id is out of range.
void* scratch_ptr(int device) {
  if (device < 0 || device >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[device]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_ptr[device] = p;
  }
  return g_scratch_ptr[device];
}

uint64_t align_up(uint64_t v) { return (v + kAlign - 1) & ~(kAlign - 1); }

struct BlockW {
  float* attn_norm;
  float* mlp_norm;
  uint16_t* wqkv;   // [(Hq + 2 Hkv) Dh, d], RoPE-pair row order within q and k heads
  uint16_t* wo;     // [d, Hq Dh]
  uint16_t* wgu;    // [2F, d], gate/up interleaved by 16 rows
  uint16_t* wd;     // [d, F]
};

// Byte layout of the arena, computed identically by stage_plan and stage_create.
struct Layout {
  // offsets (bytes from the arena base)
  std::vector<uint64_t> attn_norm, mlp_norm, wqkv, wo, wgu, wd;
  uint64_t embed = 0, readout = 0, final_norm = 0;
  uint64_t kcache = 0, vcache = 0, kv_block_elems = 0;
  uint64_t rope = 0;
  uint64_t xn = 0, q = 0, attn = 0, act = 0, part_o = 0, part_lse = 0, gemm_part = 0,
           err = 0, staging = 0;
  int ctx_cap = 0, qkv_n = 0, nsplit_max_rows = 0;
  stage_plan_t plan{};
};

int validate(const stage_model_cfg* m, const stage_stage_cfg* s) {
  if (!m || !s) return STAGE_E_INVALID;
  if (m->d_model <= 0 || m->n_q_heads <= 0 || m->n_kv_heads <= 0 || m->head_dim <= 0 || m->d_ffn <= 0 ||
      m->n_blocks_total < 0 || !(m->rms_eps > 0.0f) || !(m->rope_theta > 0.0f))
    return STAGE_E_INVALID;
  if (s->block_begin < 0 || s->block_end < s->block_begin || s->block_end > m->n_blocks_total)
    return STAGE_E_INVALID;
  if (s->max_slots <= 0 || s->max_ctx <= 0 || s->max_tokens <= 0) return STAGE_E_INVALID;
  if ((s->flags & ~(STAGE_FIRST | STAGE_LAST | STAGE_KV_F32 | STAGE_KV_F16)) != 0) return STAGE_E_INVALID;
  if ((s->flags & STAGE_KV_F32) && (s->flags & STAGE_KV_F16)) return STAGE_E_INVALID;
  if ((s->flags & (STAGE_FIRST | STAGE_LAST)) && m->vocab <= 0) return STAGE_E_INVALID;
  // what the kernels cover (refused before anything is allocated)
  if (m->head_dim != 64 && m->head_dim != 128) return STAGE_E_UNSUPPORTED;
  if (m->n_q_heads % m->n_kv_heads != 0 || m->n_q_heads / m->n_kv_heads > 16) return STAGE_E_UNSUPPORTED;
  if (m->d_model % 64 != 0 || m->d_ffn % 16 != 0) return STAGE_E_UNSUPPORTED;
  if (s->max_ctx > (1 << 24) || s->max_tokens > (1 << 20) || s->max_slots > (1 << 20)) return STAGE_E_UNSUPPORTED;
  return STAGE_OK;
}

int nsplit_for(int B, int ctx_cap) {
  return attn_decode_splits(ctx_cap, attn_decode_chunk(B));
}

Layout make_layout(const stage_model_cfg& m, const stage_stage_cfg& s) {
  Layout L;
  const uint64_t d = m.d_model, dh = m.head_dim, hq = m.n_q_heads, hkv = m.n_kv_heads, F = m.d_ffn,
                 V = m.vocab > 0 ? m.vocab : 0;
  const int nb = s.block_end - s.block_begin;
  L.qkv_n = (int)((hq + 2 * hkv) * dh);
  L.ctx_cap = (int)((s.max_ctx + 63) / 64 * 64);
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) {
    const uint64_t o = off;
    off = align_up(off + bytes);
    return o;
  };
  // weights
  if (s.flags & STAGE_FIRST) L.embed = take(V * d * 2);
  for (int b = 0; b < nb; ++b) {
    L.attn_norm.push_back(take(d * 4));
    L.mlp_norm.push_back(take(d * 4));
    L.wqkv.push_back(take((uint64_t)L.qkv_n * d * 2));
    L.wo.push_back(take(d * hq * dh * 2));
    L.wgu.push_back(take(2 * F * d * 2));
    L.wd.push_back(take(d * F * 2));
  }
  if (s.flags & STAGE_LAST) {
    L.final_norm = take(d * 4);
    L.readout = take(V * d * 2);
  }
  L.plan.weight_bytes = off;
  // KV cache
  const uint64_t kv_start = off;
  const uint64_t kvb = (s.flags & STAGE_KV_F32) ? 4 : 2;
  L.kv_block_elems = (uint64_t)s.max_slots * hkv * L.ctx_cap * dh;
  L.kcache = take(L.kv_block_elems * nb * kvb);
  L.vcache = take(L.kv_block_elems * nb * kvb);
  L.plan.kv_bytes = off - kv_start;
  // tables
  const uint64_t tab_start = off;
  L.rope = take((uint64_t)L.ctx_cap * (dh / 2) * 16);
  L.plan.table_bytes = off - tab_start;
  // workspace
  const uint64_t ws_start = off;
  const uint64_t M = s.max_tokens;
  // activation pair buffers (bf16 hi plane, then lo plane)
  L.xn = take(3 * M * d * 2);
  L.q = take(2 * M * hq * dh * 2);
  L.attn = take(2 * M * hq * dh * 2);
  L.act = take(2 * M * F * 2);
  uint64_t part_rows = 0;
  for (int B = 1; B <= s.max_tokens; ++B) {
    const uint64_t r = (uint64_t)B * nsplit_for(B, L.ctx_cap);
    if (r > part_rows) part_rows = r;
  }
  L.part_o = take(part_rows * hq * dh * 4);
  L.part_lse = take(part_rows * hq * 4);
  uint64_t gpart = 0;
  // the projections, the fused QKV also in its q and K/V row ranges (rows 0, 5, 6: QKV epilogue)
  const int shapes[7][2] = {{L.qkv_n, (int)d}, {(int)d, (int)(hq * dh)}, {(int)(2 * F), (int)d},
                            {(int)d, (int)F}, {(int)V, (int)d}, {(int)(hq * dh), (int)d},
                            {(int)(2 * hkv * dh), (int)d}};
  for (int Mr = 1; Mr <= s.max_tokens; ++Mr)
    for (int k = 0; k < 7; ++k)
      for (int planes = 2; planes <= 3; ++planes) {
        if (shapes[k][0] <= 0) continue;
        const GemmPlan p = gemm_plan(Mr, shapes[k][0], shapes[k][1], planes, k == 0 || k >= 5);
        if (p.splitk > 1) {
          const uint64_t need = (uint64_t)p.splitk * Mr * shapes[k][0] * 4;
          if (need > gpart) gpart = need;
        }
      }
  L.gemm_part = take(gpart);
  L.err = take(4);
  L.staging = take(d * 2);
  L.plan.workspace_bytes = off - ws_start;
  L.plan.total_bytes = off;
  return L;
}

}  // namespace

struct stage {
  stage_model_cfg m;
  stage_stage_cfg s;
  int device;
  uint8_t* arena;
  uint64_t arena_bytes;
  Layout L;
  int nb;
  std::vector<BlockW> blocks;
  uint16_t* embed;
  uint16_t* readout;
  float* final_norm;
  uint8_t *kcache, *vcache;
  int kv_fmt;  // KvFmt of the cache
  size_t kvb;  // bytes per KV element
  double2* rope;
  uint16_t *xn, *q, *attn, *act;
  float *part_o, *part_lse, *gemm_part;
  uint32_t* err;
  uint16_t* staging;
  std::string last_error;
  // kernel timing (benchmarks)
  uint32_t tmask = 0;
  std::vector<hipEvent_t> ev_pool;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> recs[STAGE_KT_COUNT];
};

namespace {

template <typename T>
T* at(stage* st, uint64_t off) {
  return reinterpret_cast<T*>(st->arena + off);
}

int hip_fail(stage* st, hipError_t e, const char* what) {
  char buf[256];
  snprintf(buf, sizeof buf, "%s: %s", what, hipGetErrorString(e));
  if (st) st->last_error = buf;
  return STAGE_E_HIP;
}

int fail(stage* st, int code, const char* what) {
  if (st) st->last_error = what;
  return code;
}

#define HIP_TRY(st, expr)                                   \
  do {                                                      \
    hipError_t _e = (expr);                                 \
    if (_e != hipSuccess) return hip_fail((st), _e, #expr); \
  } while (0)

hipEvent_t take_event(stage* st) {
  if (st->ev_pool.empty()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  hipEvent_t e = st->ev_pool.back();
  st->ev_pool.pop_back();
  return e;
}

// Event pair around the launches of one kernel kind while timing is enabled for it.
struct Timed {
  stage* st;
  int kind;
  hipStream_t s;
  hipEvent_t a = nullptr, b = nullptr;
  Timed(stage* st_, int kind_, hipStream_t s_) : st(st_), kind(kind_), s(s_) {
    if (st->tmask & (1u << kind)) {
      a = take_event(st);
      b = take_event(st);
      if (a) (void)hipEventRecord(a, s);
    }
  }
  ~Timed() {
    if (a && b) {
      (void)hipEventRecord(b, s);
      st->recs[kind].push_back({a, b});
    } else {   // an event could not be created: hand back the one that was
      if (a) st->ev_pool.push_back(a);
      if (b) st->ev_pool.push_back(b);
    }
  }
};

EpiArgs epi_base(stage* st, int kind) {
  EpiArgs e{};
  e.kind = kind;
  e.hq = st->m.n_q_heads;
  e.hkv = st->m.n_kv_heads;
  e.dh = st->m.head_dim;
  e.ctx_cap = st->L.ctx_cap;
  e.max_slots = st->s.max_slots;
  e.rope = st->rope;
  e.err = st->err;
  return e;
}

// plane strides of the workspace pair buffers
size_t ps_xn(const stage* st) { return (size_t)st->s.max_tokens * st->m.d_model; }
size_t ps_q(const stage* st) { return (size_t)st->s.max_tokens * st->m.n_q_heads * st->m.head_dim; }
size_t ps_act(const stage* st) { return (size_t)st->s.max_tokens * st->m.d_ffn; }

// Planes of the QKV operand: three (~24 bits) when K/V are rounded into a bf16 or binary16 cache,
// so that the rounding sees f32-grade values; two with the F32-grade cache, which keeps each value
// as a bf16 hi + lo pair (~16 bits) anyway.
int qkv_planes(const stage* st) { return st->kv_fmt == KV_F32 ? 2 : 3; }

// The RMSNorm a projection's output feeds next: `gain` (null: none requested).  `done` is set when
// the projection's split-K sum wrote the normalised rows into the norm workspace (st->xn), so the
// next projection can skip its own norm pass.
struct NextNorm {
  const float* gain = nullptr;
  bool done = false;
};

// One projection y = x W^T with its epilogue.  x_f32 + gain: the input is RMS-normalised first
// (fused in the GEMV prologue, or a row pass into the bf16 workspace before the GEMM; x_normed: the
// workspace already holds it).  planes: bf16 planes of the GEMM operand (2, or 3 for the QKV
// projection whose K/V outputs are rounded to the bf16 cache).  next: see NextNorm.
hipError_t project(stage* st, int kind, int rows, const float* x_f32, const float* gain, const uint16_t* x_pair,
                   size_t x_ps, const uint16_t* w, int N, int K, const EpiArgs& e, hipStream_t s,
                   int planes = 2, NextNorm* next = nullptr, bool x_normed = false) {
  if (next) next->done = false;
  if (gemv_fits(rows, K)) {
    Timed t(st, kind, s);
    GemvArgs a{};
    a.x = x_f32 ? x_f32 : nullptr;
    a.gain = gain;
    a.eps = st->m.rms_eps;
    a.xb = x_pair;
    a.xb_ps = x_ps;
    a.w = w;
    a.N = N;
    a.K = K;
    a.B = rows;
    a.e = e;
    return launch_gemv(a, s);
  }
  const uint16_t* A = x_pair;
  size_t a_ps = x_ps;
  if (x_f32) {
    if (!x_normed) {
      NormArgs n{x_f32, gain, st->m.rms_eps, rows, K, nullptr, st->xn, ps_xn(st)};
      hipError_t err;
      {
        Timed t(st, STAGE_KT_NORM, s);
        err = launch_rmsnorm(n, s);
      }
      if (err != hipSuccess) return err;
    }
    A = st->xn;
    a_ps = ps_xn(st);
  }
  GemmArgs g{};
  g.a = A;
  g.a_ps = a_ps;
  g.planes = x_f32 ? planes : 2;
  g.w = w;
  g.M = rows;
  g.N = N;
  g.K = K;
  const GemmPlan p = gemm_plan(rows, N, K, g.planes, e.kind == EPI_QKV);
  g.splitk = p.splitk;
  g.part = st->gemm_part;
  g.e = e;
  NormArgs then{nullptr, next ? next->gain : nullptr, st->m.rms_eps, rows, N, nullptr, st->xn, ps_xn(st)};
  Timed t(st, kind, s);
  return launch_gemm(g, p, s, next && next->gain ? &then : nullptr, next ? &next->done : nullptr);
}

// The QKV projection of norm(x_in) (x_normed: the norm workspace already holds it), its epilogue
// applying RoPE and writing q and the K/V cache.  Over a 2-byte cache the K/V outputs need the
// three-plane operand; q goes to attention as a pair and gains nothing from a third plane, so when
// the q rows alone fill a round of 256 tiles the fused weight is taken in two row ranges: the q
// rows over two planes, the K/V rows over three (the norm workspace holds all three; the first two
// are the pair split).  The q rows' sums are those of the two-plane product, the K/V rows' those
// of the fused one.  Smaller launches (batched decode, head slices) stay fused: there the two
// launches, each with its own K split and sum, are slower than one.
hipError_t project_qkv(stage* st, int rows, const float* x_in, const float* gain, const uint16_t* w,
                       const EpiArgs& e, hipStream_t s, bool x_normed) {
  const int d = st->m.d_model, qw = st->m.n_q_heads * st->m.head_dim;
  const long q_tiles = (long)((rows + 127) / 128) * ((qw + 255) / 256);   // 128 x 256 tiles of the q rows
  if (qkv_planes(st) == 2 || gemv_fits(rows, d) || rows < 256 || q_tiles < 256)
    return project(st, STAGE_KT_QKV, rows, x_in, gain, nullptr, 0, w, st->L.qkv_n, d, e, s, qkv_planes(st),
                   nullptr, x_normed);
  hipError_t err = project(st, STAGE_KT_QKV, rows, x_in, gain, nullptr, 0, w, qw, d, e, s, 2, nullptr, x_normed);
  if (err != hipSuccess) return err;
  EpiArgs ekv = e;
  ekv.col_off = qw;
  return project(st, STAGE_KT_QKV, rows, x_in, gain, nullptr, 0, w + (size_t)qw * d, st->L.qkv_n - qw, d, ekv,
                 s, 3, nullptr, true);
}

// The MLP half of a block: out = resid + W_down(silu(W_gate h) * W_up h), h = norm(x).
// x_normed: the norm workspace already holds norm(x); next: see NextNorm (after the down projection).
hipError_t mlp_half(stage* st, int lb, int rows, const float* x, const float* resid, float* out,
                    hipStream_t s, bool x_normed = false, NextNorm* next = nullptr) {
  const BlockW& bw = st->blocks[lb];
  const int d = st->m.d_model, F = st->m.d_ffn;
  EpiArgs e1 = epi_base(st, EPI_SWIGLU);
  e1.act = st->act;
  e1.act_ps = ps_act(st);
  e1.ldo = F;
  hipError_t err = project(st, STAGE_KT_GATEUP, rows, x, bw.mlp_norm, nullptr, 0, bw.wgu, 2 * F, d, e1, s, 2,
                           nullptr, x_normed);
  if (err != hipSuccess) return err;
  EpiArgs e2 = epi_base(st, resid ? EPI_RESID : EPI_F32);
  e2.out = out;
  e2.resid = resid;
  e2.ldo = d;
  return project(st, STAGE_KT_DOWN, rows, nullptr, nullptr, st->act, ps_act(st), bw.wd, d, F, e2, s, 2, next);
}

// One block over `rows` rows.  Prefill: rp = (slot, pos0), attention over keys [0, pos];
// decode: rp = per-row slots/positions, split-KV attention.
// The attention sublayer of owned block lb: x_out = (resid ? resid : 0) + W_o attention(QKV(norm(x_in))),
// with K/V written at the rows' positions.
hipError_t attn_half(stage* st, int lb, int rows, const float* x_in, const float* resid, float* x_out,
                     const RowPos& rp, bool decode, hipStream_t s, bool x_normed = false,
                     NextNorm* next = nullptr) {
  const BlockW& bw = st->blocks[lb];
  const int d = st->m.d_model, hq = st->m.n_q_heads, hkv = st->m.n_kv_heads, dh = st->m.head_dim;
  uint8_t* kc = st->kcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb;
  uint8_t* vc = st->vcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb;
  EpiArgs e = epi_base(st, EPI_QKV);
  e.kv_fmt = st->kv_fmt;
  e.q = st->q;
  e.q_ps = ps_q(st);
  e.kc = kc;
  e.vc = vc;
  e.rp = rp;
  hipError_t err = project_qkv(st, rows, x_in, bw.attn_norm, bw.wqkv, e, s, x_normed);
  if (err != hipSuccess) return err;
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
  if (decode) {
    AttnDecodeArgs a{};
    a.q = st->q;
    a.q_ps = ps_q(st);
    a.out_ps = ps_q(st);
    a.kc = kc;
    a.vc = vc;
    a.kv_fmt = st->kv_fmt;
    a.slots = rp.slots;
    a.pos = rp.pos;
    a.B = rows;
    a.hq = hq;
    a.hkv = hkv;
    a.dh = dh;
    a.ctx_cap = st->L.ctx_cap;
    a.max_slots = st->s.max_slots;
    a.chunk = attn_decode_chunk_for(rows, hkv, st->L.ctx_cap);
    a.nsplit = nsplit_for(rows, st->L.ctx_cap);
    a.scale_log2 = scale_log2;
    a.part_o = st->part_o;
    a.part_lse = st->part_lse;
    a.out = st->attn;
    a.err = st->err;
    Timed t(st, STAGE_KT_ATTN, s);
    err = launch_attn_decode(a, s);
  } else {
    AttnPrefillArgs a{};
    a.q = st->q;
    a.q_ps = ps_q(st);
    a.out_ps = ps_q(st);
    a.kc = kc;
    a.vc = vc;
    a.kv_fmt = st->kv_fmt;
    a.slot = rp.slot;
    a.pos0 = rp.pos0;
    a.T = rows;
    a.hq = hq;
    a.hkv = hkv;
    a.dh = dh;
    a.ctx_cap = st->L.ctx_cap;
    a.scale_log2 = scale_log2;
    a.out = st->attn;
    a.k_lo = 0;
    a.k_hi = INT32_MAX;
    Timed t(st, STAGE_KT_ATTN, s);
    err = launch_attn_prefill(a, s);
  }
  if (err != hipSuccess) return err;
  EpiArgs eo = epi_base(st, resid ? EPI_RESID : EPI_F32);
  eo.out = x_out;
  eo.resid = resid;
  eo.ldo = d;
  return project(st, STAGE_KT_O, rows, nullptr, nullptr, st->attn, ps_q(st), bw.wo, d, hq * dh, eo, s, 2, next);
}

// One block.  *normed: on entry, whether the norm workspace already holds norm(x_in) for this
// block's QKV projection; on exit, whether it holds the next block's (the down projection's split-K
// sum normalises with the next block's attention-norm gain when there is one).
int run_block(stage* st, int lb, int rows, const float* x_in, float* x_out, const RowPos& rp, bool decode,
              hipStream_t s, bool* normed) {
  NextNorm n1;
  n1.gain = st->blocks[lb].mlp_norm;
  HIP_TRY(st, attn_half(st, lb, rows, x_in, x_in, x_out, rp, decode, s, *normed, &n1));
  NextNorm n2;
  n2.gain = lb + 1 < st->nb ? st->blocks[lb + 1].attn_norm : nullptr;
  HIP_TRY(st, mlp_half(st, lb, rows, x_out, x_out, x_out, s, n1.done, &n2));
  *normed = n2.done;
  return STAGE_OK;
}

int run_blocks(stage* st, int rows, const float* hin, float* hout, const RowPos& rp, bool decode,
               hipStream_t s) {
  if (st->nb == 0) {
    if (hin != hout) HIP_TRY(st, hipMemcpyAsync(hout, hin, (size_t)rows * st->m.d_model * 4,
                                                 hipMemcpyDeviceToDevice, s));
    return STAGE_OK;
  }
  bool normed = false;
  for (int lb = 0; lb < st->nb; ++lb) {
    const int rc = run_block(st, lb, rows, lb == 0 ? hin : hout, hout, rp, decode, s, &normed);
    if (rc != STAGE_OK) return rc;
  }
  return STAGE_OK;
}

bool is_device_ptr(const void* p) {
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return attr.type == hipMemoryTypeDevice;
}

uint64_t role_elems(const stage* st, int role) {
  const uint64_t d = st->m.d_model, dh = st->m.head_dim, hq = st->m.n_q_heads, hkv = st->m.n_kv_heads,
                 F = st->m.d_ffn, V = st->m.vocab;
  switch (role) {
    case STAGE_ROLE_EMBED: case STAGE_ROLE_READOUT: return V * d;
    case STAGE_ROLE_ATTN_NORM: case STAGE_ROLE_MLP_NORM: case STAGE_ROLE_FINAL_NORM: return d;
    case STAGE_ROLE_WQ: return hq * dh * d;
    case STAGE_ROLE_WK: case STAGE_ROLE_WV: return hkv * dh * d;
    case STAGE_ROLE_WO: return d * hq * dh;
    case STAGE_ROLE_WGATE: case STAGE_ROLE_WUP: case STAGE_ROLE_WDOWN: return F * d;
    default: return 0;
  }
}

// Copy `rows` rows of q or k weights of one head group into the RoPE-pair row order.
hipError_t copy_rope_rows(uint16_t* dst_rows, const uint16_t* src_rows, int heads, int dh, int d,
                          hipStream_t s) {
  const size_t row_b = (size_t)d * 2;
  for (int h = 0; h < heads; ++h) {
    const uint16_t* src = src_rows + (size_t)h * dh * d;
    uint16_t* dst = dst_rows + (size_t)h * dh * d;
    for (int half = 0; half < 2; ++half) {
      // source rows half*Dh/2 + [16b, 16b+16) -> stored rows 32b + 16*half + [0, 16)
      hipError_t e = hipMemcpy2DAsync(dst + (size_t)16 * half * d, 32 * row_b,
                                      src + (size_t)half * (dh / 2) * d, 16 * row_b, 16 * row_b, dh / 32,
                                      hipMemcpyDefault, s);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace

namespace {

// Ring workspace: per (row, head) partial output and log-sum-exp, and their running accumulators.
uint64_t ring_ws_bytes(const stage* st, int T) {
  const uint64_t rh = (uint64_t)T * st->m.n_q_heads;
  return 2 * ((rh * st->m.head_dim * 4 + 255) / 256 * 256 + (rh * 4 + 255) / 256 * 256);
}

// Position ranges each of n ranks holds of a T-token sequence: one chunk each, or with zigzag the
// 2n chunks r and 2n - 1 - r ("41. Many GPUs", Ring attention for very long contexts).
std::vector<std::vector<std::pair<int, int>>> ring_chunks(int T, int n, bool zigzag) {
  std::vector<std::vector<std::pair<int, int>>> c(n);
  if (zigzag) {
    const int w = T / (2 * n);
    for (int r = 0; r < n; ++r) c[r] = {{r * w, (r + 1) * w}, {(2 * n - 1 - r) * w, (2 * n - r) * w}};
  } else {
    const int w = T / n;
    for (int r = 0; r < n; ++r) c[r] = {{r * w, (r + 1) * w}};
  }
  return c;
}

}  // namespace

extern "C" {

int stage_attn(stage_t* st, int global_block, int slot, int pos0, int T, const float* hin, float* out,
               int accumulate, hipStream_t s) {
  if (!st || !hin || !out || T <= 0) return fail(st, STAGE_E_INVALID, "bad attn arguments");
  if (global_block < st->s.block_begin || global_block >= st->s.block_end)
    return fail(st, STAGE_E_ROLE, "block outside the stage's range");
  if (T > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "T > max_tokens");
  if (slot < 0 || slot >= st->s.max_slots || pos0 < 0 || (int64_t)pos0 + T > st->s.max_ctx)
    return fail(st, STAGE_E_RANGE, "slot or positions out of range");
  HIP_TRY(st, hipSetDevice(st->device));
  RowPos rp{nullptr, nullptr, slot, pos0};
  HIP_TRY(st, attn_half(st, global_block - st->s.block_begin, T, hin, accumulate ? out : nullptr, out, rp, false, s));
  return STAGE_OK;
}

int stage_embed_range(stage_t* st, int n, const int32_t* tokens, int vocab_lo, float* hidden_out, int accumulate,
                      hipStream_t s) {
  if (!st || !tokens || !hidden_out || n <= 0 || vocab_lo < 0) return fail(st, STAGE_E_INVALID, "bad embed arguments");
  if (!(st->s.flags & STAGE_FIRST)) return fail(st, STAGE_E_ROLE, "embed on a non-first stage");
  if (n > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "n > max_tokens");
  HIP_TRY(st, hipSetDevice(st->device));
  Timed t(st, STAGE_KT_EMBED, s);
  HIP_TRY(st, launch_embed_range(st->embed, st->m.vocab, st->m.d_model, vocab_lo, tokens, n, hidden_out, accumulate,
                                 st->err, s));
  return STAGE_OK;
}

int stage_attn_ring_workspace(const stage_t* st, int T, uint64_t* bytes) {
  if (!st || T <= 0 || !bytes) return STAGE_E_INVALID;
  *bytes = ring_ws_bytes(st, T);
  return STAGE_OK;
}

namespace {

// Arguments of a ring call, checked on the host before anything is enqueued.
int ring_check(stage_t* st, int global_block, int slot, int T, int n_ranks, int zigzag, const float* hin, float* out) {
  if (!st || !hin || !out || T <= 0 || n_ranks <= 0) return fail(st, STAGE_E_INVALID, "bad ring arguments");
  if (global_block < st->s.block_begin || global_block >= st->s.block_end)
    return fail(st, STAGE_E_ROLE, "block outside the stage's range");
  if (T > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "T > max_tokens");
  if (T % (n_ranks * (zigzag ? 2 : 1)) != 0) return fail(st, STAGE_E_INVALID, "T is not a multiple of the chunk count");
  if (slot < 0 || slot >= st->s.max_slots || T > st->s.max_ctx) return fail(st, STAGE_E_RANGE, "slot or positions out of range");
  return STAGE_OK;
}

// The ring sublayer over a checked call, its partials and accumulators in `workspace` (256-byte
// aligned, ring_ws_bytes(st, T) bytes; nothing in it needs to start at zero).
int ring_run(stage_t* st, int global_block, int slot, int T, int n_ranks, int zigzag, const float* hin, float* out,
             int accumulate, void* workspace, hipStream_t s) {
  const int lb = global_block - st->s.block_begin;
  const BlockW& bw = st->blocks[lb];
  const int d = st->m.d_model, hq = st->m.n_q_heads, hkv = st->m.n_kv_heads, dh = st->m.head_dim;
  uint8_t* kc = st->kcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb;
  uint8_t* vc = st->vcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb;
  const uint64_t rh = (uint64_t)T * hq;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* part_o = reinterpret_cast<float*>(ws);
  ws += (rh * dh * 4 + 255) / 256 * 256;
  float* part_lse = reinterpret_cast<float*>(ws);
  ws += (rh * 4 + 255) / 256 * 256;
  float* acc_o = reinterpret_cast<float*>(ws);
  ws += (rh * dh * 4 + 255) / 256 * 256;
  float* acc_lse = reinterpret_cast<float*>(ws);

  // q, K and V of the whole sequence (K/V into the slot's cache at positions 0 .. T-1)
  EpiArgs e = epi_base(st, EPI_QKV);
  e.kv_fmt = st->kv_fmt;
  e.q = st->q;
  e.q_ps = ps_q(st);
  e.kc = kc;
  e.vc = vc;
  e.rp = RowPos{nullptr, nullptr, slot, 0};
  HIP_TRY(st, project_qkv(st, T, hin, bw.attn_norm, bw.wqkv, e, s, false));

  // every rank attends its query chunks to the KV chunks it holds at each hop, merging in hop order
  const auto chunks = ring_chunks(T, n_ranks, zigzag != 0);
  AttnPrefillArgs a{};
  a.q_ps = ps_q(st);
  a.kc = kc;
  a.vc = vc;
  a.kv_fmt = st->kv_fmt;
  a.slot = slot;
  a.hq = hq;
  a.hkv = hkv;
  a.dh = dh;
  a.ctx_cap = st->L.ctx_cap;
  a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)dh));
  for (int r = 0; r < n_ranks; ++r)
    for (const auto& qc : chunks[r]) {
      const int qa = qc.first, qn = qc.second - qc.first;
      bool first = true;
      for (int hop = 0; hop < n_ranks; ++hop) {
        const int owner = ((r - hop) % n_ranks + n_ranks) % n_ranks;
        for (const auto& kc2 : chunks[owner]) {
          if (kc2.first >= qc.second) continue;   // keys after every query: an empty partial
          a.q = st->q + (size_t)qa * hq * dh;
          a.pos0 = qa;
          a.T = qn;
          a.k_lo = kc2.first;
          a.k_hi = kc2.second;
          a.part_o = part_o + (size_t)qa * hq * dh;
          a.part_lse = part_lse + (size_t)qa * hq;
          HIP_TRY(st, launch_attn_prefill(a, s));
          HIP_TRY(st, launch_ring_merge(acc_o + (size_t)qa * hq * dh, acc_lse + (size_t)qa * hq, a.part_o,
                                        a.part_lse, qn, hq, dh, first ? 1 : 0, s));
          first = false;
        }
      }
    }
  HIP_TRY(st, launch_ring_store(acc_o, T, hq, dh, st->attn, ps_q(st), s));
  EpiArgs eo = epi_base(st, accumulate ? EPI_RESID : EPI_F32);
  eo.out = out;
  eo.resid = accumulate ? out : nullptr;
  eo.ldo = d;
  HIP_TRY(st, project(st, STAGE_KT_O, T, nullptr, nullptr, st->attn, ps_q(st), bw.wo, d, hq * dh, eo, s));
  return STAGE_OK;
}

}  // namespace

int stage_attn_ring(stage_t* st, int global_block, int slot, int T, int n_ranks, int zigzag, const float* hin,
                    float* out, int accumulate, void* workspace, uint64_t workspace_bytes, hipStream_t s) {
  const int rc = ring_check(st, global_block, slot, T, n_ranks, zigzag, hin, out);
  if (rc != STAGE_OK) return rc;
  if (!workspace) return fail(st, STAGE_E_INVALID, "bad ring arguments");
  if (workspace_bytes < ring_ws_bytes(st, T) || reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(st, STAGE_E_DOES_NOT_FIT, "ring workspace too small or misaligned");
  HIP_TRY(st, hipSetDevice(st->device));
  return ring_run(st, global_block, slot, T, n_ranks, zigzag, hin, out, accumulate, workspace, s);
}

int stage_attn_ring_noalloc(stage_t* st, int global_block, int slot, int T, int n_ranks, int zigzag,
                            const float* hin, float* out, int accumulate, hipStream_t s) {
  const int rc = ring_check(st, global_block, slot, T, n_ranks, zigzag, hin, out);
  if (rc != STAGE_OK) return rc;
  if (ring_ws_bytes(st, T) > kScratchBytes)
    return fail(st, STAGE_E_DOES_NOT_FIT, "ring scratch needs more than the library's 32 MiB for this T; use stage_attn_ring");
  HIP_TRY(st, hipSetDevice(st->device));
  void* ws = scratch_ptr(st->device);
  if (!ws) return fail(st, STAGE_E_HIP, "hipGetSymbolAddress of the ring scratch failed");
  return ring_run(st, global_block, slot, T, n_ranks, zigzag, hin, out, accumulate, ws, s);
}

int stage_greedy(int n, int V, const float* logits, int32_t* tokens_out, hipStream_t s) {
  if (n < 0 || V <= 0 || (n > 0 && (!logits || !tokens_out))) return STAGE_E_INVALID;
  if (n == 0) return STAGE_OK;
  return launch_argmax(logits, n, V, tokens_out, s) == hipSuccess ? STAGE_OK : STAGE_E_HIP;
}

int stage_describe(const stage_t* st, stage_model_cfg* model, stage_stage_cfg* stage, int* device) {
  if (!st) return STAGE_E_INVALID;
  if (model) *model = st->m;
  if (stage) *stage = st->s;
  if (device) *device = st->device;
  return STAGE_OK;
}

const char* stage_status_str(int status) {
  switch (status) {
    case STAGE_OK: return "ok";
    case STAGE_E_INVALID: return "invalid argument";
    case STAGE_E_UNSUPPORTED: return "unsupported configuration";
    case STAGE_E_DOES_NOT_FIT: return "does not fit in the arena";
    case STAGE_E_ROLE: return "role not owned by this stage";
    case STAGE_E_RANGE: return "slot, position or size out of range";
    case STAGE_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* stage_last_error(const stage_t* st) { return st ? st->last_error.c_str() : ""; }

int stage_plan(const stage_model_cfg* model, const stage_stage_cfg* stg, stage_plan_t* out) {
  const int rc = validate(model, stg);
  if (rc != STAGE_OK) return rc;
  if (!out) return STAGE_E_INVALID;
  *out = make_layout(*model, *stg).plan;
  return STAGE_OK;
}

int stage_create(const stage_model_cfg* model, const stage_stage_cfg* stg, void* arena, uint64_t arena_bytes,
                 int device, stage_t** out) {
  int rc = validate(model, stg);
  if (rc != STAGE_OK) return rc;
  if (!arena || !out) return STAGE_E_INVALID;
  Layout L = make_layout(*model, *stg);
  if (arena_bytes < L.plan.total_bytes) return STAGE_E_DOES_NOT_FIT;
  if (reinterpret_cast<uintptr_t>(arena) % kAlign != 0) return STAGE_E_INVALID;
  stage* st = new (std::nothrow) stage();
  if (!st) return STAGE_E_INVALID;
  st->m = *model;
  st->s = *stg;
  st->device = device;
  st->arena = static_cast<uint8_t*>(arena);
  st->arena_bytes = arena_bytes;
  st->L = L;
  st->nb = stg->block_end - stg->block_begin;
  for (int b = 0; b < st->nb; ++b)
    st->blocks.push_back(BlockW{at<float>(st, L.attn_norm[b]), at<float>(st, L.mlp_norm[b]),
                                at<uint16_t>(st, L.wqkv[b]), at<uint16_t>(st, L.wo[b]),
                                at<uint16_t>(st, L.wgu[b]), at<uint16_t>(st, L.wd[b])});
  st->embed = (stg->flags & STAGE_FIRST) ? at<uint16_t>(st, L.embed) : nullptr;
  st->readout = (stg->flags & STAGE_LAST) ? at<uint16_t>(st, L.readout) : nullptr;
  st->final_norm = (stg->flags & STAGE_LAST) ? at<float>(st, L.final_norm) : nullptr;
  st->kcache = at<uint8_t>(st, L.kcache);
  st->vcache = at<uint8_t>(st, L.vcache);
  st->kv_fmt = (stg->flags & STAGE_KV_F32) ? KV_F32 : (stg->flags & STAGE_KV_F16) ? KV_F16 : KV_BF16;
  st->kvb = st->kv_fmt == KV_F32 ? 4 : 2;
  st->rope = at<double2>(st, L.rope);
  st->xn = at<uint16_t>(st, L.xn);
  st->q = at<uint16_t>(st, L.q);
  st->attn = at<uint16_t>(st, L.attn);
  st->act = at<uint16_t>(st, L.act);
  st->part_o = at<float>(st, L.part_o);
  st->part_lse = at<float>(st, L.part_lse);
  st->gemm_part = at<float>(st, L.gemm_part);
  st->err = at<uint32_t>(st, L.err);
  st->staging = at<uint16_t>(st, L.staging);

  hipError_t e = hipSetDevice(device);
  if (e == hipSuccess) e = hipMemset(st->arena + L.kcache, 0, L.plan.kv_bytes);
  if (e == hipSuccess) e = hipMemset(st->err, 0, 4);
  if (e == hipSuccess) {
    // RoPE table in f64: angle(pos, i) = pos * theta^(-2i/Dh)
    const int half = model->head_dim / 2;
    std::vector<double2> tab((size_t)L.ctx_cap * half);
    for (int p = 0; p < L.ctx_cap; ++p)
      for (int i = 0; i < half; ++i) {
        const double inv = std::pow((double)model->rope_theta, -2.0 * i / model->head_dim);
        const double a = (double)p * inv;
        tab[(size_t)p * half + i] = make_double2(std::cos(a), std::sin(a));
      }
    e = hipMemcpy(st->rope, tab.data(), tab.size() * sizeof(double2), hipMemcpyHostToDevice);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    delete st;
    return STAGE_E_HIP;
  }
  (void)scratch_ptr(device);   // the device's scratch address, looked up once with the device current
  *out = st;
  return STAGE_OK;
}

int stage_destroy(stage_t* st) {
  if (!st) return STAGE_OK;
  for (auto& v : st->recs)
    for (auto& pr : v) {
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  for (auto e : st->ev_pool) (void)hipEventDestroy(e);
  delete st;
  return STAGE_OK;
}

int stage_timing(stage_t* st, uint32_t kind_mask) {
  if (!st) return STAGE_E_INVALID;
  if (kind_mask >> STAGE_KT_COUNT) return fail(st, STAGE_E_INVALID, "unknown kernel kind in mask");
  for (auto& v : st->recs) {
    for (auto& pr : v) {
      st->ev_pool.push_back(pr.first);
      st->ev_pool.push_back(pr.second);
    }
    v.clear();
  }
  st->tmask = kind_mask;
  return STAGE_OK;
}

int stage_timing_read(stage_t* st, int kind, uint64_t* launches, double* total_ms) {
  if (!st || !launches || !total_ms || kind < 0 || kind >= STAGE_KT_COUNT)
    return fail(st, STAGE_E_INVALID, "bad timing arguments");
  double tot = 0.0;
  auto& v = st->recs[kind];
  for (auto& pr : v) {
    HIP_TRY(st, hipEventSynchronize(pr.second));
    float ms = 0.0f;
    HIP_TRY(st, hipEventElapsedTime(&ms, pr.first, pr.second));
    tot += ms;
    st->ev_pool.push_back(pr.first);
    st->ev_pool.push_back(pr.second);
  }
  *launches = v.size();
  *total_ms = tot;
  v.clear();
  return STAGE_OK;
}

int stage_load_weight(stage_t* st, int role, int global_block, const uint16_t* src, uint64_t n_elems,
                      hipStream_t s) {
  if (!st || !src) return fail(st, STAGE_E_INVALID, "null handle or source");
  const bool per_block = !(role == STAGE_ROLE_EMBED || role == STAGE_ROLE_FINAL_NORM || role == STAGE_ROLE_READOUT);
  if (role < 0 || role > STAGE_ROLE_READOUT) return fail(st, STAGE_E_ROLE, "unknown role");
  if (per_block && (global_block < st->s.block_begin || global_block >= st->s.block_end))
    return fail(st, STAGE_E_ROLE, "block outside the stage's range");
  if (!per_block && global_block != -1) return fail(st, STAGE_E_ROLE, "end tensors take global_block = -1");
  if (role == STAGE_ROLE_EMBED && !(st->s.flags & STAGE_FIRST)) return fail(st, STAGE_E_ROLE, "embed on a non-first stage");
  if ((role == STAGE_ROLE_READOUT || role == STAGE_ROLE_FINAL_NORM) && !(st->s.flags & STAGE_LAST))
    return fail(st, STAGE_E_ROLE, "readout on a non-last stage");
  if (n_elems != role_elems(st, role)) return fail(st, STAGE_E_RANGE, "n_elems does not match the role");
  HIP_TRY(st, hipSetDevice(st->device));
  const int d = st->m.d_model, dh = st->m.head_dim, hq = st->m.n_q_heads, hkv = st->m.n_kv_heads, F = st->m.d_ffn;
  const BlockW* bw = per_block ? &st->blocks[global_block - st->s.block_begin] : nullptr;
  const size_t row_b = (size_t)d * 2;
  switch (role) {
    case STAGE_ROLE_EMBED:
      HIP_TRY(st, hipMemcpyAsync(st->embed, src, n_elems * 2, hipMemcpyDefault, s));
      break;
    case STAGE_ROLE_READOUT:
      HIP_TRY(st, hipMemcpyAsync(st->readout, src, n_elems * 2, hipMemcpyDefault, s));
      break;
    case STAGE_ROLE_ATTN_NORM: case STAGE_ROLE_MLP_NORM: case STAGE_ROLE_FINAL_NORM: {
      float* dst = role == STAGE_ROLE_ATTN_NORM ? bw->attn_norm
                   : role == STAGE_ROLE_MLP_NORM ? bw->mlp_norm : st->final_norm;
      HIP_TRY(st, hipMemcpyAsync(st->staging, src, n_elems * 2, hipMemcpyDefault, s));
      HIP_TRY(st, launch_bf16_to_f32(st->staging, dst, d, s));
      break;
    }
    case STAGE_ROLE_WQ:
      HIP_TRY(st, copy_rope_rows(bw->wqkv, src, hq, dh, d, s));
      break;
    case STAGE_ROLE_WK:
      HIP_TRY(st, copy_rope_rows(bw->wqkv + (size_t)hq * dh * d, src, hkv, dh, d, s));
      break;
    case STAGE_ROLE_WV:
      HIP_TRY(st, hipMemcpyAsync(bw->wqkv + (size_t)(hq + hkv) * dh * d, src, n_elems * 2, hipMemcpyDefault, s));
      break;
    case STAGE_ROLE_WO:
      HIP_TRY(st, hipMemcpyAsync(bw->wo, src, n_elems * 2, hipMemcpyDefault, s));
      break;
    case STAGE_ROLE_WGATE: case STAGE_ROLE_WUP:
      // source row f -> stored row 32*(f/16) + f%16 (+16 for up)
      HIP_TRY(st, hipMemcpy2DAsync(bw->wgu + (role == STAGE_ROLE_WUP ? (size_t)16 * d : 0), 32 * row_b, src,
                                   16 * row_b, 16 * row_b, F / 16, hipMemcpyDefault, s));
      break;
    case STAGE_ROLE_WDOWN:
      HIP_TRY(st, hipMemcpyAsync(bw->wd, src, n_elems * 2, hipMemcpyDefault, s));
      break;
  }
  if (!is_device_ptr(src)) HIP_TRY(st, hipStreamSynchronize(s));
  return STAGE_OK;
}

int stage_embed(stage_t* st, int n, const int32_t* tokens, float* hidden_out, hipStream_t s) {
  if (!st || !tokens || !hidden_out || n <= 0) return fail(st, STAGE_E_INVALID, "bad embed arguments");
  if (!(st->s.flags & STAGE_FIRST)) return fail(st, STAGE_E_ROLE, "embed on a non-first stage");
  if (n > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "n > max_tokens");
  HIP_TRY(st, hipSetDevice(st->device));
  Timed t(st, STAGE_KT_EMBED, s);
  HIP_TRY(st, launch_embed(st->embed, st->m.vocab, st->m.d_model, tokens, n, hidden_out, st->err, s));
  return STAGE_OK;
}

int stage_prefill(stage_t* st, int slot, int pos0, int T, const float* hin, float* hout, hipStream_t s) {
  if (!st || !hin || !hout || T <= 0) return fail(st, STAGE_E_INVALID, "bad prefill arguments");
  if (T > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "T > max_tokens");
  if (slot < 0 || slot >= st->s.max_slots || pos0 < 0 || (int64_t)pos0 + T > st->s.max_ctx)
    return fail(st, STAGE_E_RANGE, "slot or positions out of range");
  HIP_TRY(st, hipSetDevice(st->device));
  RowPos rp{nullptr, nullptr, slot, pos0};
  return run_blocks(st, T, hin, hout, rp, false, s);
}

int stage_decode(stage_t* st, int B, const int32_t* slots, const int32_t* positions, const float* hin,
                 float* hout, hipStream_t s) {
  if (!st || !slots || !positions || !hin || !hout || B <= 0) return fail(st, STAGE_E_INVALID, "bad decode arguments");
  if (B > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "B > max_tokens");
  HIP_TRY(st, hipSetDevice(st->device));
  RowPos rp{slots, positions, 0, 0};
  return run_blocks(st, B, hin, hout, rp, true, s);
}

int stage_readout(stage_t* st, int n, const float* hin, float* logits, float* normed, hipStream_t s) {
  if (!st || !hin || !logits || n <= 0) return fail(st, STAGE_E_INVALID, "bad readout arguments");
  if (!(st->s.flags & STAGE_LAST)) return fail(st, STAGE_E_ROLE, "readout on a non-last stage");
  if (n > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "n > max_tokens");
  HIP_TRY(st, hipSetDevice(st->device));
  const int d = st->m.d_model;
  NormArgs na{hin, st->final_norm, st->m.rms_eps, n, d, normed, st->xn, ps_xn(st)};
  {
    Timed t(st, STAGE_KT_NORM, s);
    HIP_TRY(st, launch_rmsnorm(na, s));
  }
  EpiArgs e = epi_base(st, EPI_F32);
  e.out = logits;
  e.ldo = st->m.vocab;
  HIP_TRY(st, project(st, STAGE_KT_READOUT, n, nullptr, nullptr, st->xn, ps_xn(st), st->readout, st->m.vocab, d, e, s));
  return STAGE_OK;
}

int stage_mlp(stage_t* st, int global_block, int n, const float* hin, float* out, int accumulate, hipStream_t s) {
  if (!st || !hin || !out || n <= 0) return fail(st, STAGE_E_INVALID, "bad mlp arguments");
  if (global_block < st->s.block_begin || global_block >= st->s.block_end)
    return fail(st, STAGE_E_ROLE, "block outside the stage's range");
  if (n > st->s.max_tokens) return fail(st, STAGE_E_INVALID, "n > max_tokens");
  HIP_TRY(st, hipSetDevice(st->device));
  HIP_TRY(st, mlp_half(st, global_block - st->s.block_begin, n, hin, accumulate ? out : nullptr, out, s));
  return STAGE_OK;
}

int stage_kv_copy(stage_t* st, int src_slot, int dst_slot, int n_pos, hipStream_t s) {
  if (!st || n_pos < 0) return fail(st, STAGE_E_INVALID, "bad kv_copy arguments");
  if (src_slot < 0 || src_slot >= st->s.max_slots || dst_slot < 0 || dst_slot >= st->s.max_slots ||
      n_pos > st->s.max_ctx)
    return fail(st, STAGE_E_RANGE, "slot or positions out of range");
  if (n_pos == 0 || src_slot == dst_slot) return STAGE_OK;
  HIP_TRY(st, hipSetDevice(st->device));
  const int hkv = st->m.n_kv_heads, dh = st->m.head_dim, cap = st->L.ctx_cap;
  const size_t slot_elems = (size_t)hkv * cap * dh;
  const size_t vgroups = (size_t)(n_pos + 7) / 8;
  const size_t eb = st->kvb;
  for (int lb = 0; lb < st->nb; ++lb) {
    uint8_t* kc = st->kcache + (uint64_t)lb * st->L.kv_block_elems * eb;
    uint8_t* vc = st->vcache + (uint64_t)lb * st->L.kv_block_elems * eb;
    // per KV head: K rows [0, n_pos) and the V groups covering them are contiguous
    HIP_TRY(st, hipMemcpy2DAsync(kc + dst_slot * slot_elems * eb, (size_t)cap * dh * eb, kc + src_slot * slot_elems * eb,
                                 (size_t)cap * dh * eb, (size_t)n_pos * dh * eb, hkv, hipMemcpyDeviceToDevice, s));
    HIP_TRY(st, hipMemcpy2DAsync(vc + dst_slot * slot_elems * eb, (size_t)cap * dh * eb, vc + src_slot * slot_elems * eb,
                                 (size_t)cap * dh * eb, vgroups * dh * 8 * eb, hkv, hipMemcpyDeviceToDevice, s));
  }
  return STAGE_OK;
}

static int kv_io_check(stage_t* st, int global_block, int slot, int pos0, int n, const void* k, const void* v) {
  if (!st || !k || !v || n <= 0) return fail(st, STAGE_E_INVALID, "bad kv arguments");
  if (global_block < st->s.block_begin || global_block >= st->s.block_end)
    return fail(st, STAGE_E_ROLE, "block outside the stage's range");
  if (slot < 0 || slot >= st->s.max_slots || pos0 < 0 || (int64_t)pos0 + n > st->s.max_ctx)
    return fail(st, STAGE_E_RANGE, "slot or positions out of range");
  return STAGE_OK;
}

int stage_kv_import(stage_t* st, int global_block, int slot, int pos0, int n, const void* k, const void* v,
                    hipStream_t s) {
  const int rc = kv_io_check(st, global_block, slot, pos0, n, k, v);
  if (rc != STAGE_OK) return rc;
  HIP_TRY(st, hipSetDevice(st->device));
  const int lb = global_block - st->s.block_begin;
  HIP_TRY(st, launch_kv_import(st->kcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb,
                               st->vcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb, st->kv_fmt == KV_F32, st->m.n_kv_heads,
                               st->m.head_dim, st->L.ctx_cap, slot, pos0, n, k, v, s));
  return STAGE_OK;
}

int stage_kv_export(stage_t* st, int global_block, int slot, int pos0, int n, void* k, void* v,
                    hipStream_t s) {
  const int rc = kv_io_check(st, global_block, slot, pos0, n, k, v);
  if (rc != STAGE_OK) return rc;
  HIP_TRY(st, hipSetDevice(st->device));
  const int lb = global_block - st->s.block_begin;
  HIP_TRY(st, launch_kv_export(st->kcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb,
                               st->vcache + (uint64_t)lb * st->L.kv_block_elems * st->kvb, st->kv_fmt == KV_F32, st->m.n_kv_heads,
                               st->m.head_dim, st->L.ctx_cap, slot, pos0, n, k, v, s));
  return STAGE_OK;
}

int stage_device_errors(stage_t* st, int reset, uint32_t* count, hipStream_t s) {
  if (!st || !count) return fail(st, STAGE_E_INVALID, "bad arguments");
  HIP_TRY(st, hipSetDevice(st->device));
  HIP_TRY(st, hipMemcpyAsync(count, st->err, 4, hipMemcpyDeviceToHost, s));
  HIP_TRY(st, hipStreamSynchronize(s));
  if (reset) {
    HIP_TRY(st, hipMemsetAsync(st->err, 0, 4, s));
    HIP_TRY(st, hipStreamSynchronize(s));
  }
  return STAGE_OK;
}

}  // extern "C"
