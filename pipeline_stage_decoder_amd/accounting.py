"""Algorithmic bytes and flops of the stage forward, for throughput against the HBM / MFMA rooflines.

Conventions:
* Decode reads every weight once per step ("41. Many GPUs", When one GPU isn't enough: decode
  reads every weight once per step), so a decode step's bytes are the bf16 weights of the stage,
  the bf16 K and V of every attended position, the K/V rows written, the F32 hidden rows in and
  out, and the F32 logits on a last stage.
* Prefill flops are 2 * (linear parameters) * tokens (the chapter's estimate of prefill cost, from
  its section on disaggregated prefill and decode: 32 TFLOP for 2,000 tokens of an 8B model) plus
  attention 4 * Hq * Dh * (keys attended, summed over queries).
* Elementwise work (norms, RoPE, SiLU, softmax) is not counted.

The page-traffic helpers reproduce the arithmetic the chapter prints for its CPU engine runs and
are pinned by tests against those printed numbers.
"""
from __future__ import annotations

BF16 = 2
F32 = 4


# ---------------------------------------------------------------------------------------------
# per-block shapes
# ---------------------------------------------------------------------------------------------

def block_linear_params(s) -> int:
    d, dh = s.d_model, s.head_dim
    qkv = (s.n_q_heads + 2 * s.n_kv_heads) * dh * d
    o = d * s.n_q_heads * dh
    mlp = 3 * s.d_ffn * d
    return qkv + o + mlp


def block_weight_bytes(s) -> int:
    """bf16 matrices of one block (the F32 norm gains, 2 * d * 4 bytes, are not counted)."""
    return block_linear_params(s) * BF16


def kv_bytes_per_token_block(s, kv_elem_bytes: int = BF16) -> int:
    return 2 * s.n_kv_heads * s.head_dim * kv_elem_bytes


def projection_shapes(s) -> dict:
    """(N, K) of every projection: output rows N, input width K."""
    d, dh = s.d_model, s.head_dim
    return {"qkv": ((s.n_q_heads + 2 * s.n_kv_heads) * dh, d), "o": (d, s.n_q_heads * dh),
            "gateup": (2 * s.d_ffn, d), "down": (d, s.d_ffn), "readout": (s.vocab, d)}


def projection_bytes(s, kind: str, rows: int) -> int:
    """Algorithmic bytes of one launch of a projection over `rows` rows: the bf16 weight read once,
    the input rows (F32 for the normalised projections, which read the residual; a bf16 hi+lo pair,
    4 bytes, for the others) and the outputs (F32 residual / logits, 4-byte pair activations, bf16
    K/V rows + pair q for QKV)."""
    n, k = projection_shapes(s)[kind]
    w = n * k * BF16
    if kind == "qkv":
        qw, kvw = s.n_q_heads * s.head_dim, 2 * s.n_kv_heads * s.head_dim
        return w + rows * (k * F32 + qw * 4 + kvw * BF16)
    if kind == "gateup":
        return w + rows * (k * F32 + s.d_ffn * 4)
    if kind == "readout":
        return w + rows * (k * 4 + n * F32)
    # o, down: pair input, F32 residual read + write
    return w + rows * (k * 4 + 2 * n * F32)


def projection_flops(s, kind: str, rows: int) -> int:
    """Algorithmic flops of one launch of a projection over `rows` rows: 2 * rows * N * K."""
    n, k = projection_shapes(s)[kind]
    return 2 * rows * n * k


def projection_gemm_bytes(s, kind: str, rows: int, kv_elem_bytes: int = BF16) -> int:
    """Bytes a prefill projection launch must move at least once: the bf16 weight, its activation
    operand as the planes the GEMM multiplies (2 planes of bf16, 3 for QKV over a 2-byte cache),
    and its outputs (F32 residual read + write for O/down, a 4-byte pair per SwiGLU output, pair q
    and the K/V rows for QKV)."""
    n, k = projection_shapes(s)[kind]
    w = n * k * BF16
    if kind == "qkv":
        planes = 2 if kv_elem_bytes == F32 else 3
        qw, kvw = s.n_q_heads * s.head_dim, 2 * s.n_kv_heads * s.head_dim
        return w + rows * (planes * k * BF16 + qw * 4 + kvw * kv_elem_bytes)
    if kind == "gateup":
        return w + rows * (2 * k * BF16 + s.d_ffn * 4)
    if kind == "readout":
        return w + rows * (2 * k * BF16 + n * F32)
    return w + rows * (2 * k * BF16 + 2 * n * F32)


# ---------------------------------------------------------------------------------------------
# whole steps
# ---------------------------------------------------------------------------------------------

def decode_step_bytes(s, n_blocks: int, ctxs, first: bool = False, last: bool = False,
                      kv_elem_bytes: int = BF16) -> int:
    """One decode step of B = len(ctxs) rows; row b attends ctxs[b] + 1 keys (ctxs[b] cached)."""
    B = len(ctxs)
    kv_tok = kv_bytes_per_token_block(s, kv_elem_bytes)
    per_block = block_weight_bytes(s) + sum(c + 1 for c in ctxs) * kv_tok
    total = n_blocks * per_block
    total += 2 * B * s.d_model * F32                       # hidden in, hidden out
    if first:
        total += B * s.d_model * BF16                      # embedding rows
    if last:
        total += s.vocab * s.d_model * BF16 + B * s.vocab * F32
    return total


def prefill_flops(s, n_blocks: int, T: int, pos0: int = 0, last: bool = False, attn: bool = True) -> int:
    """Linear flops 2 * params * T plus (attn=True) 4 * Hq * Dh * keys attended."""
    lin = 2 * block_linear_params(s) * T
    keys = sum(pos0 + t + 1 for t in range(T))
    attn = 4 * s.n_q_heads * s.head_dim * keys if attn else 0
    total = n_blocks * (lin + attn)
    if last:
        total += 2 * s.vocab * s.d_model * T
    return total


def mlp_slice_bytes(d: int, width: int, T: int) -> int:
    """bf16 gate/up [width, d] and down [d, width] of one slice, F32 rows in and partial out."""
    return 3 * width * d * BF16 + 2 * T * d * F32


def mlp_slice_flops(d: int, width: int, T: int) -> int:
    return 2 * 3 * width * d * T


# ---------------------------------------------------------------------------------------------
# the chapter's CPU-engine traffic arithmetic ("41. Many GPUs", Measured)
# ---------------------------------------------------------------------------------------------

def pp_send_bytes(prompts: int, prompt_tokens: int, new_tokens: int, hidden: int, dtype_bytes: int) -> int:
    """Pipeline sends: one hidden row per token per step -- the prompt step, then one row per
    sequence for each of the remaining new_tokens - 1 decode steps."""
    return (prompts * prompt_tokens + (new_tokens - 1) * prompts) * hidden * dtype_bytes


def tp_all_reduce(layers: int, prompts: int, prompt_tokens: int, new_tokens: int, hidden: int,
                  dtype_bytes: int):
    """(calls, bytes) of tensor-parallel all-reduces: two per layer plus one for the vocabulary-
    parallel embedding per step, plus one int64 to agree on the KV pool size."""
    per_step = 2 * layers + 1
    calls = new_tokens * per_step + 1
    prefill = per_step * prompts * prompt_tokens * hidden * dtype_bytes
    decode = (new_tokens - 1) * per_step * prompts * hidden * dtype_bytes
    return calls, prefill + decode + 8


def tp_all_gather_bytes(new_tokens: int, rows: int, vocab: int, ranks: int, dtype_bytes: int) -> int:
    """Logit all-gathers: one per step, this rank's vocabulary slice of every sampled row."""
    return new_tokens * rows * (vocab // ranks) * dtype_bytes


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    return 2 * layers * kv_heads * head_dim * dtype_bytes
