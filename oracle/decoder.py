"""CPU oracle of one pipeline stage's decoder forward -- TEST INFRASTRUCTURE, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module.  It shares no code with the GPU path (``pipeline_stage_decoder_amd``) and
never imports it; the two meet only in the seeded inputs of ``fixtures``.

It is plain numpy: float64 for every sum, a library matmul (``@``) as the one primitive, no
blocking or fusion.  What it computes, by page title and section:

* "41. Many GPUs: tensor, pipeline, expert and data parallelism" (the book chapter), section
  "Pipeline parallelism": a stage embeds tokens when it is the first, then runs its blocks in
  order -- each block normalises the residual stream, adds the attention sublayer's output to it,
  normalises the new residual, adds the MLP's output -- and only the residual stream crosses a
  stage boundary; the last stage applies the final norm before the readout.
* same chapter, "Ring attention for very long contexts": causal attention with the score scale
  Dh^-1/2, a key visible to a query when its position is not after the query's, and partial
  results over disjoint key sets combined through their log-sum-exps.
* same chapter, "Tensor parallelism": weights are [out, in]; a column-parallel shard keeps output
  rows, a row-parallel shard keeps input columns and yields a partial sum; grouped-query attention
  gives each KV head an equal, contiguous group of query heads; the MLP multiplies SiLU of the
  gate projection by the up projection; the vocabulary is padded to a multiple of the shard count.
* "Multi-node layer splitting and tensor parallelism" (TensorSharp), "Supported stage executors":
  the dense pipeline hands F32 hidden activations between stages, the first stage embeds and the
  last computes logits; "Transport and tuning": partial sums are added in node order.
* "RFC: pipeline placement across multiple GPUs ...", "Numerical correctness proof": staged and
  single-device execution must agree bit for bit on logits, final features, KV state and tokens.

Readings where the pages are silent (each listed in the design notes):
RMSNorm is x * rsqrt(mean(x^2) + eps) * g (no mean subtraction, eps inside the root);
RoPE is the rotate-half form over the whole head, angle pos * theta^(-2i/Dh), absolute 0-based
positions; the residual stream is F32 inside a stage as well as across it; the readout is untied;
a sequence's keys are the positions its cache holds, so a query at position p attends to the held
positions <= p (for every call that keeps the stage contract -- positions before a prefill chunk
already written -- this is every position <= p).
Precision: weights are bf16 (the seeded inputs), the KV cache stores K (after RoPE) and V as bf16,
F16 or float32 values (the stage's cache format), and nothing else is rounded -- every activation,
score and sum is float64, and tensors the method hands over as F32 (stage output, final hidden,
logits, partial sums) are rounded to float32 once.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against brute-force loops,
closed forms and invariants the pages fix, and ``tests/test_oracle_mutations.py`` plants plausible
mistakes in a copy of this module and checks that some pin fails for each.  Absolute forward values
are not printed by any page; they are pinned by those invariants and brute-force cases.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# --------------------------------------------------------------------------------------------
# number formats
# --------------------------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> their exact float32 values."""
    b = np.asarray(bits, dtype=np.uint16)
    return (np.ascontiguousarray(b).astype(np.uint32) << 16).view(np.float32).reshape(b.shape)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    x = np.asarray(x, dtype=np.float32)
    u = np.ascontiguousarray(x).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16).reshape(x.shape)


def round_bf16(x) -> np.ndarray:
    """Round to float32 first (the GPU holds these values in f32), then to bf16; return float32."""
    return bf16_to_f32(f32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def round_f16(x) -> np.ndarray:
    """Round to float32 first, then to IEEE binary16 (nearest, ties to even); return float32."""
    return np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float32)


KV_FORMATS = {
    "bf16": round_bf16,
    "f16": round_f16,
    "f32": lambda t: np.asarray(t, dtype=np.float32),
}


def f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def f32_sum_in_order(parts) -> np.ndarray:
    """((p0 + p1) + p2) + ... with every partial sum rounded to float32 (node-order summation)."""
    total = np.asarray(parts[0], dtype=np.float32).copy()
    for p in parts[1:]:
        total = (total + np.asarray(p, dtype=np.float32)).astype(np.float32)
    return total


# --------------------------------------------------------------------------------------------
# the decoder's operations
# --------------------------------------------------------------------------------------------


def rms_norm(x: np.ndarray, gain: np.ndarray, eps: float) -> np.ndarray:
    """x * (1 / sqrt(mean(x^2) + eps)) * g per row, in float64 (reading: Llama RMSNorm)."""
    x = f64(x)
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return x * r * f64(gain)


def linear64(h: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """y = h W^T for W stored [out, in] (the chapter's nn.Linear layout), float64 throughout."""
    return f64(h) @ f64(bf16_to_f32(w_bits)).T


def linear(h: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """linear64 rounded once to float32 (an F32 output tensor)."""
    return linear64(h, w_bits).astype(np.float32)


def rope_angles(positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """angle[p, i] = p * theta^(-2i/Dh) for i < Dh/2, float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return f64(positions)[:, None] * inv_freq[None, :]


def rope(x: np.ndarray, positions: np.ndarray, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x [n, heads, Dh] at absolute positions [n]; f64 in, f64 out.

    For i < Dh/2 the pair (x_i, x_{i+Dh/2}) is rotated by angle[p, i]:
    y_i = x_i cos - x_{i+Dh/2} sin,  y_{i+Dh/2} = x_{i+Dh/2} cos + x_i sin.
    """
    x = f64(x)
    half = x.shape[-1] // 2
    a = rope_angles(positions, x.shape[-1], theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    lo, hi = x[..., :half], x[..., half:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def attend(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos, k_pos, scale: float):
    """Causal grouped-query attention with its log-sum-exp, from the definition.

    q [Tq, Hq, D]; k, v [Tk, Hkv, D], Hq a multiple of Hkv; query head h reads KV head
    h // (Hq / Hkv).  For query row t the visible keys J are those with k_pos[j] <= q_pos[t].
    With scores s_j = scale * <q_t, k_j> over J:
        lse = log sum_{j in J} exp(s_j),   out = sum_{j in J} exp(s_j - lse) v_j.
    An empty J gives lse = -inf and out = 0.  Float64.  The keys are put in position order once,
    so every J is a leading run of them; each (row, KV head) is then one small product.
    Returns (out [Tq, Hq, D], lse [Tq, Hq]).
    """
    q, k, v = f64(q), f64(k), f64(v)
    q_pos, k_pos = np.asarray(q_pos), np.asarray(k_pos)
    order = np.argsort(k_pos, kind="stable")
    k_pos = k_pos[order]
    k = np.ascontiguousarray(k[order].transpose(1, 0, 2))                # [Hkv, Tk, D]
    v = np.ascontiguousarray(v[order].transpose(1, 0, 2))
    n_q, hq, dd = q.shape
    hkv = k.shape[0]
    group = hq // hkv
    out = np.zeros((n_q, hq, dd))
    lse = np.full((n_q, hq), -np.inf)
    for t in range(n_q):
        n_vis = int(np.searchsorted(k_pos, q_pos[t], side="right"))     # |J|
        if n_vis == 0:
            continue
        for g in range(hkv):
            heads = slice(g * group, (g + 1) * group)                   # query heads reading KV head g
            s = (k[g, :n_vis] @ q[t, heads].T) * scale                 # [|J|, group]
            m = s.max(axis=0)
            l = m + np.log(np.sum(np.exp(s - m), axis=0))
            lse[t, heads] = l
            out[t, heads] = np.exp(s - l).T @ v[g, :n_vis]
    return out, lse


def lse_combine(partials):
    """Attention over a union of disjoint key sets from the partial results over each set.

    For partials (o_s, l_s), each the output and log-sum-exp of one key set:
        l = log sum_s exp(l_s),   o = sum_s exp(l_s - l) o_s,
    which is attend() over the union (the weights exp(s_j - l) of every key re-normalised to the
    whole set).  Partials with l_s = -inf (no visible key) weigh nothing; if every l_s is -inf the
    result is (0, -inf).  Float64.
    """
    ls = np.stack([f64(l) for _, l in partials])                        # [S, ...]
    with np.errstate(divide="ignore", invalid="ignore"):
        l_all = np.logaddexp.reduce(ls, axis=0)
    live = np.isfinite(l_all)
    out = np.zeros(np.shape(partials[0][0]))
    for o_s, l_s in partials:
        with np.errstate(invalid="ignore"):
            wgt = np.where(live, np.exp(np.where(live, f64(l_s) - l_all, -np.inf)), 0.0)
        out = out + wgt[..., None] * f64(o_s)
    return out, l_all


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """SwiGLU's product: silu(gate) * up = gate / (1 + e^-gate) * up, float64."""
    g = f64(gate)
    return g / (1.0 + np.exp(-g)) * f64(up)


def swiglu_act(h: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray) -> np.ndarray:
    """The MLP's inner activation of normed rows h: silu(h W_gate^T) * (h W_up^T), float64."""
    return silu_mul(linear64(h, w_gate), linear64(h, w_up))


def mlp_delta(x: np.ndarray, g_mlp, w_gate, w_up, w_down, eps: float):
    """The MLP sublayer of F32 rows x without its residual: W_down a with
    a = swiglu_act(RMSNorm(x) * g_mlp).  Returns (a, W_down a), both float64."""
    a = swiglu_act(rms_norm(x, bf16_to_f32(g_mlp), eps), w_gate, w_up)
    return a, linear64(a, w_down)


# --------------------------------------------------------------------------------------------
# one stage
# --------------------------------------------------------------------------------------------


@dataclass(frozen=True)
class Dims:
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4

    @staticmethod
    def of(shape) -> "Dims":
        return Dims(shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn,
                    shape.vocab, shape.rms_eps, shape.rope_theta)


class Stage:
    """A contiguous block range [begin, end) with its own weights and per-slot KV cache.

    ``weights`` maps (role, global_block) -> bf16 bits; the roles are embed, attn_norm, wq, wk, wv,
    wo, mlp_norm, wgate, wup, wdown (per block), final_norm, readout.  K (after RoPE) and V are
    cached per slot, block and absolute position in the stage's cache format ``kv_dtype``.
    """

    def __init__(self, dims: Dims, begin: int, end: int, first: bool, last: bool, weights: dict,
                 max_ctx: int, kv_dtype: str = "bf16"):
        assert kv_dtype in KV_FORMATS
        self.c, self.begin, self.end, self.first, self.last = dims, begin, end, first, last
        self.w, self.max_ctx = weights, max_ctx
        self.kv_dtype = kv_dtype
        self.kv = {}                      # slot -> (K, V) float32 [blocks, ctx, Hkv, Dh]
        self.held = {}                    # slot -> bool [blocks, ctx]: positions written

    def _cache(self, slot: int):
        if slot not in self.kv:
            shp = (self.end - self.begin, self.max_ctx, self.c.n_kv_heads, self.c.head_dim)
            self.kv[slot] = (np.zeros(shp, np.float32), np.zeros(shp, np.float32))
            self.held[slot] = np.zeros(shp[:2], bool)
        return self.kv[slot]

    def store(self, b: int, slot: int, pos: int, k_row: np.ndarray, v_row: np.ndarray) -> None:
        """Write one position's K and V (already in the cache format) of block b."""
        kc, vc = self._cache(slot)
        lb = b - self.begin
        kc[lb, pos], vc[lb, pos] = k_row, v_row
        self.held[slot][lb, pos] = True

    def import_kv(self, b: int, slot: int, pos0: int, k: np.ndarray, v: np.ndarray) -> None:
        """Write given K and V values [n, Hkv, Dh] of block b at positions pos0 .. pos0+n-1 (values
        taken as they are: the caller supplies them in the cache format)."""
        kc, vc = self._cache(slot)
        lb, n = b - self.begin, k.shape[0]
        kc[lb, pos0:pos0 + n], vc[lb, pos0:pos0 + n] = k, v
        self.held[slot][lb, pos0:pos0 + n] = True

    def embed(self, tokens: np.ndarray) -> np.ndarray:
        """First stage only: x_t = E[token_t] as F32 (exact)."""
        assert self.first
        return bf16_to_f32(self.w[("embed", -1)][np.asarray(tokens)])

    def qkv(self, b: int, x: np.ndarray, positions: np.ndarray):
        """q, k, v of F32 rows x at their positions: h = RMSNorm(x) g_attn, q = RoPE(h W_q^T)
        (f64), k = RoPE(h W_k^T) and v = h W_v^T in the cache format."""
        c, w = self.c, self.w
        n = x.shape[0]
        h = rms_norm(x, bf16_to_f32(w[("attn_norm", b)]), c.rms_eps)
        q = linear64(h, w[("wq", b)]).reshape(n, c.n_q_heads, c.head_dim)
        k = linear64(h, w[("wk", b)]).reshape(n, c.n_kv_heads, c.head_dim)
        v = linear64(h, w[("wv", b)]).reshape(n, c.n_kv_heads, c.head_dim)
        q = rope(q, positions, c.rope_theta)
        k = rope(k, positions, c.rope_theta)
        to_cache = KV_FORMATS[self.kv_dtype]
        return q, to_cache(k), to_cache(v)

    def attention(self, b: int, x: np.ndarray, slots: np.ndarray, positions: np.ndarray) -> np.ndarray:
        """The attention sublayer of block b without its residual (float64 [M, d]).  Every row's K
        and V are written to its slot first; row m then attends to its slot's held positions
        <= positions[m]; the heads' outputs, concatenated, go through W_o."""
        c = self.c
        q, k, v = self.qkv(b, x, positions)
        for m in range(x.shape[0]):
            self.store(b, int(slots[m]), int(positions[m]), k[m], v[m])
        lb = b - self.begin
        o = np.zeros(q.shape)
        for s in np.unique(slots):
            rows = np.nonzero(slots == s)[0]
            kc, vc = self._cache(int(s))
            key_pos = np.nonzero(self.held[int(s)][lb])[0]
            o[rows], _ = attend(q[rows], kc[lb, key_pos], vc[lb, key_pos], positions[rows], key_pos,
                                c.head_dim ** -0.5)
        return linear64(o.reshape(x.shape[0], -1), self.w[("wo", b)])

    def mlp(self, b: int, x1: np.ndarray) -> np.ndarray:
        """The MLP sublayer of block b on F32 rows x1 without its residual (float64)."""
        w = self.w
        _, y = mlp_delta(x1, w[("mlp_norm", b)], w[("wgate", b)], w[("wup", b)], w[("wdown", b)],
                         self.c.rms_eps)
        return y

    def block(self, b: int, x: np.ndarray, slots: np.ndarray, positions: np.ndarray) -> np.ndarray:
        """One decoder block on F32 rows x [M, d]; row m is slot slots[m] at positions[m].
        x1 = x + attention(x) and x2 = x1 + mlp(x1), each rounded once to F32."""
        x1 = (x + self.attention(b, x, slots, positions)).astype(np.float32)
        return (x1 + self.mlp(b, x1)).astype(np.float32)

    def forward(self, x: np.ndarray, slots, positions) -> np.ndarray:
        """All blocks of the stage; returns the F32 residual handed to the next stage."""
        x = np.asarray(x, dtype=np.float32)
        slots = np.asarray(slots, dtype=np.int64).reshape(-1)
        positions = np.asarray(positions, dtype=np.int64).reshape(-1)
        assert x.shape[0] == slots.shape[0] == positions.shape[0]
        assert positions.max(initial=0) < self.max_ctx
        for b in range(self.begin, self.end):
            x = self.block(b, x, slots, positions)
        return x

    def prefill(self, x, slot: int, pos0: int) -> np.ndarray:
        t = x.shape[0]
        return self.forward(x, np.full(t, slot), np.arange(pos0, pos0 + t))

    def readout(self, x: np.ndarray):
        """Last stage only: h_N = RMSNorm(x) g_final (returned as the F32 "final hidden") and the
        F32 logits h_N W_readout^T."""
        assert self.last
        g = bf16_to_f32(self.w[("final_norm", -1)])
        h_n = rms_norm(x, g, self.c.rms_eps)
        logits = linear(h_n, self.w[("readout", -1)])
        return logits, h_n.astype(np.float32)

    def kv_bits(self, slot: int, n_pos: int):
        """bf16 bits of the cached K and V of a slot, positions [0, n_pos): [blocks, n, Hkv, Dh]."""
        kc, vc = self._cache(slot)
        return f32_to_bf16_bits(kc[:, :n_pos]), f32_to_bf16_bits(vc[:, :n_pos])


def greedy(logits: np.ndarray) -> np.ndarray:
    """argmax per row, lowest index on ties."""
    return np.argmax(logits, axis=-1).astype(np.int32)


def top2_margin(logits: np.ndarray) -> np.ndarray:
    part = np.sort(logits, axis=-1)
    return part[..., -1] - part[..., -2]


# --------------------------------------------------------------------------------------------
# pipeline driver (split vs unsplit) and the sharded-MLP slices
# --------------------------------------------------------------------------------------------


def generate(stages: list, prompt: np.ndarray, n_new: int, slot: int = 0):
    """Greedy generation through an ordered list of stages, handing F32 rows between them.

    One token comes from the prompt's last logits row, then n_new - 1 decode steps (the
    chapter's "16 new tokens" are one prefill step plus fifteen decode steps).  Returns the tokens
    and, per step, the handoff rows, the final hidden rows and the logits.
    """
    trace = {"handoff": [], "final_hidden": [], "logits": [], "residual": []}
    x = stages[0].embed(prompt)
    pos0, t = 0, len(prompt)
    for st in stages:
        x = st.prefill(x, slot, pos0)
        trace["handoff"].append(x.copy())
    logits, h_n = stages[-1].readout(x)
    trace["residual"].append(x)
    trace["final_hidden"].append(h_n)
    trace["logits"].append(logits)
    toks = [int(greedy(logits[-1:])[0])]
    pos = t
    for _ in range(n_new - 1):
        x = stages[0].embed(np.array([toks[-1]]))
        for st in stages:
            x = st.forward(x, [slot], [pos])
            trace["handoff"].append(x.copy())
        logits, h_n = stages[-1].readout(x)
        trace["residual"].append(x)
        trace["final_hidden"].append(h_n)
        trace["logits"].append(logits)
        toks.append(int(greedy(logits)[0]))
        pos += 1
    return np.array(toks, dtype=np.int32), trace


def mlp_full(x: np.ndarray, g_mlp: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray,
             eps: float):
    """The whole SwiGLU MLP of F32 rows x: returns (activation a, f64; F32 output W_d a)."""
    a, y = mlp_delta(x, g_mlp, wg, wu, wd, eps)
    return a, y.astype(np.float32)


def mlp_slices(x, g_mlp, wg, wu, wd, eps: float, n_slices: int):
    """Megatron column/row split: slice i keeps rows [i*w, (i+1)*w) of W_gate and W_up (output
    rows, column parallel) and the same columns of W_down (input columns, row parallel), so its
    output is an F32 partial of the MLP; partials are summed in slice order in float32.
    Returns (slice activations, partials, f32 sum)."""
    width = wg.shape[0] // n_slices
    acts, parts = [], []
    for i in range(n_slices):
        rows = slice(i * width, (i + 1) * width)
        a_i, y_i = mlp_delta(x, g_mlp, wg[rows], wu[rows], np.ascontiguousarray(wd[:, rows]), eps)
        acts.append(a_i)
        parts.append(y_i.astype(np.float32))
    return acts, parts, f32_sum_in_order(parts)


# --------------------------------------------------------------------------------------------
# tensor-parallel shards of attention and of the vocabulary ("41. Many GPUs", Tensor parallelism)
# --------------------------------------------------------------------------------------------

def attn_stage(x_width: int, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float,
               kv_dtype: str, max_ctx: int) -> Stage:
    """A one-block Stage holding only the attention weights (block 0)."""
    dims = Dims(x_width, wq.shape[0] // head_dim, wk.shape[0] // head_dim, head_dim, 1, 1, eps, theta)
    w = {("attn_norm", 0): g_attn, ("wq", 0): wq, ("wk", 0): wk, ("wv", 0): wv, ("wo", 0): wo}
    return Stage(dims, 0, 1, False, False, w, max_ctx, kv_dtype)


def attn_sublayer(x: np.ndarray, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float,
                  kv_dtype: str = "bf16", pos0: int = 0):
    """The attention sublayer (Stage.attention) of F32 rows x [T, d] forming one sequence at
    positions pos0 .. pos0+T-1, without its residual; the f64 delta [T, d]."""
    t = x.shape[0]
    st = attn_stage(x.shape[1], g_attn, wq, wk, wv, wo, head_dim, eps, theta, kv_dtype, pos0 + t)
    return st.attention(0, np.asarray(x, np.float32), np.zeros(t, np.int64), np.arange(pos0, pos0 + t))


def head_shards(n_q_heads: int, n_kv_heads: int, n: int):
    """Attention split by heads over n shards: (q0, hq, kv0, hk) of each shard.

    Query heads are dealt out evenly and contiguously (hq = Hq / n per shard).  A shard keeps the
    KV heads its query heads read (query head h reads KV head h // (Hq / Hkv)).  The split is valid
    when every shard needs the same number of KV heads and either no KV head is needed by two
    shards (the KV heads are split too) or every shard needs exactly one (a KV head is replicated
    over the shards of its group); otherwise ValueError.
    """
    if n <= 0 or n_q_heads % n or n_q_heads % n_kv_heads:
        raise ValueError("query heads do not split evenly over the shards")
    per_shard, group = n_q_heads // n, n_q_heads // n_kv_heads
    needs = [sorted({h // group for h in range(i * per_shard, (i + 1) * per_shard)}) for i in range(n)]
    counts = {len(kv) for kv in needs}
    if len(counts) != 1:
        raise ValueError("shards would need different numbers of KV heads")
    hk = counts.pop()
    shared = len({h for kv in needs for h in kv}) < sum(len(kv) for kv in needs)
    if shared and hk != 1:
        raise ValueError("a KV head would be split across shards")
    return [(i * per_shard, per_shard, kv[0], hk) for i, kv in enumerate(needs)]


def attn_slices(x, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float, n_slices: int,
                kv_dtype: str = "bf16"):
    """Head-sharded attention: shard i keeps its query heads' rows of W_q, its KV heads' rows of
    W_k / W_v and the matching columns of W_o, and gives an F32 partial; partials are summed in
    shard order in float32.  Returns (partials, f32 sum)."""
    parts = []
    for q0, hq, kv0, hk in head_shards(wq.shape[0] // head_dim, wk.shape[0] // head_dim, n_slices):
        qr = slice(q0 * head_dim, (q0 + hq) * head_dim)
        kr = slice(kv0 * head_dim, (kv0 + hk) * head_dim)
        part = attn_sublayer(x, g_attn, wq[qr], wk[kr], wv[kr], np.ascontiguousarray(wo[:, qr]), head_dim,
                             eps, theta, kv_dtype)
        parts.append(part.astype(np.float32))
    return parts, f32_sum_in_order(parts)


def vocab_shards(vocab: int, n: int):
    """An n-way split of a vocabulary padded with zero rows to n * ceil(V / n): every shard holds
    rows = ceil(V / n) rows, shard i the ids [i * rows, (i + 1) * rows) (ids >= V are padding).
    Returns (rows, [first id of each shard])."""
    rows = (vocab + n - 1) // n
    return rows, [i * rows for i in range(n)]


def vocab_shard(table_bits: np.ndarray, n: int, i: int) -> np.ndarray:
    """Shard i of a [V, d] bf16 table split as vocab_shards says (zero rows past V)."""
    rows, _ = vocab_shards(table_bits.shape[0], n)
    padded = np.zeros((rows * n, table_bits.shape[1]), table_bits.dtype)
    padded[:table_bits.shape[0]] = table_bits
    return padded.reshape(n, rows, -1)[i]


def embed_shards(table_bits: np.ndarray, tokens: np.ndarray, n: int) -> np.ndarray:
    """Vocabulary-parallel embedding.  A lookup E[t] is the product onehot(t) E; splitting E's rows
    into shards splits that product's inner dimension, so shard i contributes onehot_i(t) E_i -- its
    row t - first_i when t falls inside the shard and a zero row otherwise -- and the shards'
    contributions are summed in shard order (F32; each is exact, one product per element)."""
    rows, firsts = vocab_shards(table_bits.shape[0], n)
    tokens = np.asarray(tokens, dtype=np.int64)
    parts = []
    for i in range(n):
        onehot = (tokens[:, None] - firsts[i]) == np.arange(rows)[None, :]
        parts.append(onehot.astype(np.float64) @ f64(bf16_to_f32(vocab_shard(table_bits, n, i))))
    return f32_sum_in_order(parts)


def readout_shards(h_final: np.ndarray, readout_bits: np.ndarray, n: int) -> np.ndarray:
    """Vocabulary-parallel head: every shard scores its rows (padding rows score 0), the scores are
    concatenated in shard order and cut back to V (F32 logits)."""
    cols = [linear(h_final, vocab_shard(readout_bits, n, i)) for i in range(n)]
    return np.concatenate(cols, axis=1)[:, :readout_bits.shape[0]]


# --------------------------------------------------------------------------------------------
# context parallelism: ring attention ("41. Many GPUs", Ring attention for very long contexts)
# --------------------------------------------------------------------------------------------

def ring_chunks(T: int, n_ranks: int, zigzag: bool):
    """Query/KV position ranges each rank holds: rank r gets [rT, (r+1)T) of n equal chunks, or
    with zigzag the 2n chunks r and 2n - 1 - r (which evens out causal work)."""
    if zigzag:
        c = T // (2 * n_ranks)
        return [[(r * c, (r + 1) * c), ((2 * n_ranks - 1 - r) * c, (2 * n_ranks - r) * c)] for r in range(n_ranks)]
    c = T // n_ranks
    return [[(r * c, (r + 1) * c)] for r in range(n_ranks)]


def ring_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_ranks: int, zigzag: bool = False):
    """Causal GQA attention of a whole sequence (positions 0..T-1; q [T, Hq, D], k / v [T, Hkv, D])
    computed the ring way: rank r holds its chunks' queries and keys; at hop h it holds the K/V of
    rank (r - h) mod n, and each of its query chunks takes the partial attention over that K/V
    (attend); a query chunk's partials over the n hops cover every key once and are combined by
    lse_combine (associative: the hop order the GPU merges in changes only rounding).  Returns the
    f64 output [T, Hq, D]."""
    t, hq, dd = q.shape
    chunks = ring_chunks(t, n_ranks, zigzag)
    out = np.zeros((t, hq, dd))
    for r in range(n_ranks):
        for qa, qb in chunks[r]:
            partials = []
            for hop in range(n_ranks):
                for ka, kb in chunks[(r - hop) % n_ranks]:
                    partials.append(attend(q[qa:qb], k[ka:kb], v[ka:kb], np.arange(qa, qb), np.arange(ka, kb),
                                           dd ** -0.5))
            out[qa:qb], _ = lse_combine(partials)
    return out


def attn_sublayer_ring(x: np.ndarray, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float,
                       n_ranks: int, zigzag: bool, kv_dtype: str = "bf16"):
    """attn_sublayer over positions 0..T-1 with the attention taken by ring_attention (f64 delta)."""
    t = x.shape[0]
    st = attn_stage(x.shape[1], g_attn, wq, wk, wv, wo, head_dim, eps, theta, kv_dtype, t)
    q, k, v = st.qkv(0, np.asarray(x, np.float32), np.arange(t))
    o = ring_attention(q, k, v, n_ranks, zigzag)
    return linear64(o.reshape(t, -1), wo)
