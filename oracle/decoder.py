"""CPU oracle of one pipeline stage's decoder forward -- TEST INFRASTRUCTURE, not the product.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import this module.  It shares no code with the GPU path (``pipeline_stage_decoder_amd``) and
never imports it; the two meet only in the seeded inputs of ``fixtures``.

It is plain numpy: float64 for every sum, a library matmul (``@``) as the one primitive, no
blocking or fusion.  Sources, cited by page title and section:

* "41. Many GPUs: tensor, pipeline, expert and data parallelism" (the book chapter), section
  "Pipeline parallelism": ``PipelineStage.forward`` fixes the stage semantics -- embed on the first
  stage, then per block ``add_norm`` -> attention -> ``add_norm`` -> MLP, and only the residual
  stream ``x + delta`` crosses a stage boundary; the final norm follows the last block.
* same chapter, "Ring attention for very long contexts": ``attention_partial`` (causal scores
  ``q.k * scale``, keys with ``k_pos > q_pos`` masked, log-sum-exp, rows with no key get lse -inf)
  and ``merge_partials`` (the split-KV merge by log-sum-exp).
* same chapter, "Tensor parallelism": weights are ``[out, in]``; ``take_rows`` keeps output rows
  (column parallel), ``take_cols`` keeps input columns (row parallel, a partial sum); GQA maps
  query head h to KV head ``h // (Hq / Hkv)``; the MLP is ``down(silu(gate(x)) * up(x))``.
* "Multi-node layer splitting and tensor parallelism" (TensorSharp), "Supported stage executors":
  the dense pipeline hands F32 hidden activations between stages, the first stage embeds and the
  last computes logits; "Transport and tuning": sums of partials in node order ((v0+v1)+v2)+...
* "RFC: pipeline placement across multiple GPUs ...", "Numerical correctness proof": staged and
  single-device execution must agree bit-for-bit on logits, final features, KV state and tokens.

Readings where the pages are silent (each listed in the design notes):
RMSNorm is x * rsqrt(mean(x^2) + eps) * g (no mean subtraction, eps inside the root);
RoPE is the rotate-half form over the whole head, angle pos * theta^(-2i/Dh), absolute 0-based
positions; the residual stream is F32 inside a stage as well as across it; the readout is untied.
Precision: weights are bf16 (the seeded inputs), the KV cache stores K (after RoPE) and V as bf16
(or, for a stage built with an F32 cache, as float32), and nothing else is rounded -- every
activation, score and sum is float64, and tensors the method hands over as F32 (stage output, final
hidden, logits, MLP partials) are rounded to float32 once.

Pins: every function here is checked by ``tests/test_oracle_pins.py`` against brute-force loops,
closed forms and invariants the pages fix (see that file).  Absolute forward values are not
printed by any page ("parity unpinned" by page numbers); they are pinned by those invariants.
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


def f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


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


def attention_partial(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray,
                      k_pos: np.ndarray, scale: float):
    """Causal attention of q [Tq, H, D] over k, v [Tk, H, D] -> (out [Tq, H, D], lse [Tq, H]).

    Same definition as the chapter's ``attention_partial``: scores = q.k * scale, keys with
    k_pos > q_pos masked to -inf, probabilities exp(score - lse); a row that sees no key has
    lse = -inf and output 0.  Float64 throughout.
    """
    q, k, v = f64(q), f64(k), f64(v)
    scores = np.einsum("qhd,khd->hqk", q, k) * scale
    masked = k_pos[None, None, :] > q_pos[None, :, None]
    scores = np.where(masked, -np.inf, scores)
    top = scores.max(axis=-1, keepdims=True)
    top_safe = np.where(np.isinf(top), 0.0, top)
    with np.errstate(divide="ignore"):
        lse = (np.log(np.exp(scores - top_safe).sum(axis=-1, keepdims=True)) + top_safe)[..., 0]
    probs = np.exp(scores - np.where(np.isinf(lse), 0.0, lse)[..., None])
    return np.einsum("hqk,khd->qhd", probs, v), lse.T


def merge_partials(out, lse, new_out, new_lse):
    """The chapter's split-KV merge of two partial attentions by their log-sum-exps (f64)."""
    top = np.maximum(lse, new_lse)
    top = np.where(np.isinf(top), 0.0, top)
    a, b = np.exp(lse - top), np.exp(new_lse - top)
    total = a + b
    merged = (out * a[..., None] + new_out * b[..., None]) / np.where(total > 0, total, 1)[..., None]
    with np.errstate(divide="ignore"):
        return merged, top + np.log(total)


def gqa_expand(kv: np.ndarray, n_q_heads: int) -> np.ndarray:
    """[T, Hkv, D] -> [T, Hq, D]: query head h reads KV head h // (Hq / Hkv)."""
    group = n_q_heads // kv.shape[1]
    return np.repeat(kv, group, axis=1)


def attention_gqa(q: np.ndarray, k: np.ndarray, v: np.ndarray, q_pos: np.ndarray, k_pos: np.ndarray,
                  scale: float) -> np.ndarray:
    """attention_partial's output for GQA without repeating K/V: q [Tq, Hq, D] over k, v
    [Tk, Hkv, D], query head h reading KV head h // (Hq / Hkv).  Float64 throughout."""
    tq, hq, dd = q.shape
    hkv = k.shape[1]
    qg = f64(q).reshape(tq, hkv, hq // hkv, dd)                    # [Tq, Hkv, G, D]
    scores = np.einsum("qcgd,kcd->cgqk", qg, f64(k)) * scale       # [Hkv, G, Tq, Tk]
    masked = k_pos[None, None, None, :] > q_pos[None, None, :, None]
    scores = np.where(masked, -np.inf, scores)
    top = scores.max(axis=-1, keepdims=True)
    top = np.where(np.isinf(top), 0.0, top)
    w = np.exp(scores - top)
    z = w.sum(axis=-1, keepdims=True)
    out = np.einsum("cgqk,kcd->qcgd", w / np.where(z > 0, z, 1.0), f64(v))
    return out.reshape(tq, hq, dd)


def silu_mul(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """silu(gate) * up in float64 (the chapter's ``F.silu(gate) * up``)."""
    g = f64(gate)
    return g / (1.0 + np.exp(-g)) * f64(up)


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
    wo, mlp_norm, wgate, wup, wdown (per block), final_norm, readout.  K and V are cached as the
    bf16 values the attention reads, per slot, block and absolute position.
    """

    def __init__(self, dims: Dims, begin: int, end: int, first: bool, last: bool, weights: dict,
                 max_ctx: int, kv_dtype: str = "bf16"):
        assert kv_dtype in ("bf16", "f32")
        self.c, self.begin, self.end, self.first, self.last = dims, begin, end, first, last
        self.w, self.max_ctx = weights, max_ctx
        self.kv_dtype = kv_dtype
        self.kv = {}                      # slot -> (K, V) float32 [blocks, ctx, Hkv, Dh]

    def _cache(self, slot: int):
        if slot not in self.kv:
            shp = (self.end - self.begin, self.max_ctx, self.c.n_kv_heads, self.c.head_dim)
            self.kv[slot] = (np.zeros(shp, np.float32), np.zeros(shp, np.float32))
        return self.kv[slot]

    def embed(self, tokens: np.ndarray) -> np.ndarray:
        """First stage only: x_t = E[token_t] as F32 (exact)."""
        assert self.first
        return bf16_to_f32(self.w[("embed", -1)][np.asarray(tokens)])

    def block(self, b: int, x: np.ndarray, slots: np.ndarray, positions: np.ndarray) -> np.ndarray:
        """One decoder block on F32 rows x [M, d]; row m is slot slots[m] at positions[m]."""
        c, w = self.c, self.w
        hq, hkv, dh = c.n_q_heads, c.n_kv_heads, c.head_dim
        m_rows = x.shape[0]
        h = rms_norm(x, bf16_to_f32(w[("attn_norm", b)]), c.rms_eps)
        q = linear64(h, w[("wq", b)]).reshape(m_rows, hq, dh)
        k = linear64(h, w[("wk", b)]).reshape(m_rows, hkv, dh)
        v = linear64(h, w[("wv", b)]).reshape(m_rows, hkv, dh)
        q = rope(q, positions, c.rope_theta)
        store = round_bf16 if self.kv_dtype == "bf16" else (lambda t: np.asarray(t, np.float32))
        k = store(rope(k, positions, c.rope_theta))                           # the KV cache's format
        v = store(v)
        lb = b - self.begin
        for m in range(m_rows):                                                # write KV first
            kc, vc = self._cache(int(slots[m]))
            kc[lb, positions[m]] = k[m]
            vc[lb, positions[m]] = v[m]
        attn = np.empty((m_rows, hq * dh), np.float64)
        scale = dh ** -0.5
        for s in np.unique(slots):
            rows = np.nonzero(slots == s)[0]
            kc, vc = self._cache(int(s))
            n_keys = int(positions[rows].max()) + 1
            o = attention_gqa(q[rows], kc[lb, :n_keys], vc[lb, :n_keys], positions[rows].astype(np.int64),
                              np.arange(n_keys), scale)
            attn[rows] = o.reshape(len(rows), hq * dh)
        x1 = (x + linear64(attn, w[("wo", b)])).astype(np.float32)
        h2 = rms_norm(x1, bf16_to_f32(w[("mlp_norm", b)]), c.rms_eps)
        a = silu_mul(linear64(h2, w[("wgate", b)]), linear64(h2, w[("wup", b)]))
        return (x1 + linear64(a, w[("wdown", b)])).astype(np.float32)

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
        """Last stage only: final RMSNorm (F32 "final hidden") and F32 logits of bf16(h_N)."""
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
    h = rms_norm(x, bf16_to_f32(g_mlp), eps)
    a = silu_mul(linear64(h, wg), linear64(h, wu))
    return a, linear(a, wd)


def mlp_slices(x, g_mlp, wg, wu, wd, eps: float, n_slices: int):
    """Megatron column/row split: slice i keeps rows [i*w, (i+1)*w) of W_gate and W_up and the
    same columns of W_down, giving an F32 partial; partials are summed in slice order
    ((p0 + p1) + p2) + ... in float32.  Returns (slice activations, partials, f32 sum)."""
    f = wg.shape[0]
    w = f // n_slices
    h = rms_norm(x, bf16_to_f32(g_mlp), eps)
    acts, parts = [], []
    for i in range(n_slices):
        lo, hi = i * w, (i + 1) * w
        a_i = silu_mul(linear64(h, wg[lo:hi]), linear64(h, wu[lo:hi]))
        acts.append(a_i)
        parts.append(linear(a_i, np.ascontiguousarray(wd[:, lo:hi])))
    total = parts[0].copy()
    for p in parts[1:]:
        total = (total + p).astype(np.float32)
    return acts, parts, total


# --------------------------------------------------------------------------------------------
# tensor-parallel slices of attention and of the vocabulary ("41. Many GPUs", Tensor parallelism)
# --------------------------------------------------------------------------------------------

def attn_sublayer(x: np.ndarray, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float,
                  kv_dtype: str = "bf16"):
    """The attention sublayer of F32 rows x [T, d] at positions 0..T-1 of a fresh sequence, without
    its residual: W_o . attention(q, K, V), q/k/v from h = RMSNorm(x) * g, K and V stored in the
    cache format (bf16 or F32) as in Stage.block.  Returns the f64 delta [T, d]."""
    t = x.shape[0]
    hq, hkv = wq.shape[0] // head_dim, wk.shape[0] // head_dim
    pos = np.arange(t)
    h = rms_norm(x, bf16_to_f32(g_attn), eps)
    q = rope(linear64(h, wq).reshape(t, hq, head_dim), pos, theta)
    store = round_bf16 if kv_dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    k = store(rope(linear64(h, wk).reshape(t, hkv, head_dim), pos, theta))
    v = store(linear64(h, wv).reshape(t, hkv, head_dim))
    o = attention_gqa(q, k, v, pos, pos, head_dim ** -0.5)
    return linear64(o.reshape(t, hq * head_dim), wo)


def head_slices(n_q_heads: int, n_kv_heads: int, n_slices: int):
    """Slice i's query heads [q0, q0 + hq) and KV heads [kv0, kv0 + hk): query heads split evenly,
    KV heads split while there are at least as many as slices and otherwise replicated, slice i
    keeping the KV head its query heads read (kv0 = q0 // (Hq / Hkv))."""
    if n_q_heads % n_slices or (n_kv_heads % n_slices and n_slices % n_kv_heads):
        raise ValueError("heads do not split over the slices")
    hq, hk = n_q_heads // n_slices, max(n_kv_heads // n_slices, 1)
    out = []
    for i in range(n_slices):
        kv0 = i * hk if n_kv_heads >= n_slices else (i * hq) // (n_q_heads // n_kv_heads)
        out.append((i * hq, hq, kv0, hk))
    return out


def attn_slices(x, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float, n_slices: int,
                kv_dtype: str = "bf16"):
    """Head-sharded attention: slice i keeps its query heads' rows of W_q, its KV heads' rows of
    W_k / W_v and the matching columns of W_o, and gives an F32 partial; partials are summed in
    slice order in float32.  Returns (partials, f32 sum)."""
    hq_all, hkv_all = wq.shape[0] // head_dim, wk.shape[0] // head_dim
    parts = []
    for q0, hq, kv0, hk in head_slices(hq_all, hkv_all, n_slices):
        qr = slice(q0 * head_dim, (q0 + hq) * head_dim)
        kr = slice(kv0 * head_dim, (kv0 + hk) * head_dim)
        part = attn_sublayer(x, g_attn, wq[qr], wk[kr], wv[kr], np.ascontiguousarray(wo[:, qr]), head_dim, eps,
                             theta, kv_dtype)
        parts.append(part.astype(np.float32))
    total = parts[0].copy()
    for p in parts[1:]:
        total = (total + p).astype(np.float32)
    return parts, total


def vocab_range(vocab: int, n_slices: int, i: int):
    """(rows per slice, first id, end id) of slice i: the vocabulary padded to a multiple of the
    slice count, every slice holding the same number of rows."""
    per = -(-vocab // n_slices)
    return per, i * per, min(vocab, (i + 1) * per)


def vocab_slice(table_bits: np.ndarray, n_slices: int, i: int) -> np.ndarray:
    """Slice i of a [V, d] bf16 table: its rows, zero rows past V (the padding)."""
    per, lo, hi = vocab_range(table_bits.shape[0], n_slices, i)
    out = np.zeros((per, table_bits.shape[1]), table_bits.dtype)
    out[:hi - lo] = table_bits[lo:hi]
    return out


def embed_slices(table_bits: np.ndarray, tokens: np.ndarray, n_slices: int) -> np.ndarray:
    """Vocabulary-parallel embedding: slice i looks up its own ids and zeros for the rest; the
    slices' rows are summed in slice order (F32)."""
    total = np.zeros((len(tokens), table_bits.shape[1]), np.float32)
    for i in range(n_slices):
        per, lo, hi = vocab_range(table_bits.shape[0], n_slices, i)
        mine = (tokens >= lo) & (tokens < hi)
        rows = bf16_to_f32(vocab_slice(table_bits, n_slices, i))[np.where(mine, tokens - lo, 0)]
        total = (total + rows * mine[:, None]).astype(np.float32)
    return total


def readout_slices(h_final: np.ndarray, readout_bits: np.ndarray, n_slices: int) -> np.ndarray:
    """Vocabulary-parallel head: every slice scores its rows, the scores are concatenated in slice
    order and cut back to V (F32 logits)."""
    cols = [linear(h_final, vocab_slice(readout_bits, n_slices, i)) for i in range(n_slices)]
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
    rank (r - h) mod n and attends its queries to it (attention_partial), merging the partials in
    hop order by log-sum-exp (merge_partials).  Returns the f64 output [T, Hq, D]."""
    t, hq, dd = q.shape
    kx, vx = gqa_expand(k, hq), gqa_expand(v, hq)
    chunks = ring_chunks(t, n_ranks, zigzag)
    out = np.zeros((t, hq, dd))
    for r in range(n_ranks):
        for qa, qb in chunks[r]:
            qp = np.arange(qa, qb)
            acc, lse = np.zeros((qb - qa, hq, dd)), np.full((qb - qa, hq), -np.inf)
            for hop in range(n_ranks):
                owner = (r - hop) % n_ranks
                for ka, kb in chunks[owner]:
                    o, l = attention_partial(q[qa:qb], kx[ka:kb], vx[ka:kb], qp, np.arange(ka, kb), dd ** -0.5)
                    acc, lse = merge_partials(acc, lse, o, l)
            out[qa:qb] = acc
    return out


def attn_sublayer_ring(x: np.ndarray, g_attn, wq, wk, wv, wo, head_dim: int, eps: float, theta: float,
                       n_ranks: int, zigzag: bool, kv_dtype: str = "bf16"):
    """attn_sublayer with the attention taken by ring_attention (f64 delta [T, d])."""
    t = x.shape[0]
    hq, hkv = wq.shape[0] // head_dim, wk.shape[0] // head_dim
    pos = np.arange(t)
    h = rms_norm(x, bf16_to_f32(g_attn), eps)
    q = rope(linear64(h, wq).reshape(t, hq, head_dim), pos, theta)
    store = round_bf16 if kv_dtype == "bf16" else (lambda a: np.asarray(a, np.float32))
    k = store(rope(linear64(h, wk).reshape(t, hkv, head_dim), pos, theta))
    v = store(linear64(h, wv).reshape(t, hkv, head_dim))
    o = ring_attention(q, k, v, n_ranks, zigzag)
    return linear64(o.reshape(t, hq * head_dim), wo)
