"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a copy of the oracle's source (a textual change to one
statement, applied to a fresh module; the oracle itself is untouched) and runs the pins named for
it against that copy: every named pin must fail.  This shows that the pins are not a retyping of
the oracle -- a dropped term, a swapped operand, a wrong index or a missing rotation is caught.
"""
import itertools
import os
import sys
import types

import pytest

from tests import test_oracle_pins as pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "decoder.py")

# (name, [(statement, planted statement)], [pins that must fail])
MUTATIONS = [
    ("query RoPE dropped (block and attention sublayer)",
     [("q = rope(q, positions, c.rope_theta)", "q = q")],
     ["test_attention_sublayer_bruteforce_relative_rotation", "test_prefill_is_invariant_to_a_shift_of_all_positions"]),
    ("key RoPE dropped",
     [("k = rope(k, positions, c.rope_theta)", "k = k")],
     ["test_attention_sublayer_bruteforce_relative_rotation", "test_kv_cache_holds_rotated_keys_in_the_cache_format"]),
    ("both RoPEs dropped",
     [("q = rope(q, positions, c.rope_theta)", "q = q"), ("k = rope(k, positions, c.rope_theta)", "k = k")],
     ["test_attention_sublayer_bruteforce_relative_rotation"]),
    ("MLP norm reads x instead of the new residual x1",
     [("return (x1 + self.mlp(b, x1)).astype(np.float32)", "return (x1 + self.mlp(b, x)).astype(np.float32)")],
     ["test_block_composes_attention_then_mlp_of_the_new_residual"]),
    ("gate and up swapped in the SwiGLU activation",
     [("return silu_mul(linear64(h, w_gate), linear64(h, w_up))", "return silu_mul(linear64(h, w_up), linear64(h, w_gate))")],
     ["test_mlp_bruteforce_gate_and_up_named", "test_block_with_zero_attention_output_is_x_plus_mlp_of_x"]),
    ("gate and up swapped in the block's MLP only",
     [('w[("wgate", b)], w[("wup", b)]', 'w[("wup", b)], w[("wgate", b)]')],
     ["test_block_with_zero_attention_output_is_x_plus_mlp_of_x", "test_block_composes_attention_then_mlp_of_the_new_residual"]),
    ("final-norm gain dropped in the readout",
     [("h_n = rms_norm(x, g, self.c.rms_eps)", "h_n = rms_norm(x, np.ones_like(g), self.c.rms_eps)")],
     ["test_readout_bruteforce_with_gains"]),
    ("attention residual dropped",
     [("x1 = (x + self.attention(b, x, slots, positions)).astype(np.float32)",
       "x1 = (0 * x + self.attention(b, x, slots, positions)).astype(np.float32)")],
     ["test_attn_sublayer_is_the_blocks_attention_half", "test_block_composes_attention_then_mlp_of_the_new_residual"]),
    ("MLP residual dropped",
     [("return (x1 + self.mlp(b, x1)).astype(np.float32)", "return (0 * x1 + self.mlp(b, x1)).astype(np.float32)")],
     ["test_block_with_zero_attention_output_is_x_plus_mlp_of_x"]),
    ("score scale dropped",
     [("positions[rows], key_pos,\n                                c.head_dim ** -0.5)", "positions[rows], key_pos,\n                                1.0)")],
     ["test_attention_sublayer_bruteforce_relative_rotation"]),
    ("a query does not see its own key",
     [('n_vis = int(np.searchsorted(k_pos, q_pos[t], side="right"))', 'n_vis = int(np.searchsorted(k_pos, q_pos[t], side="left"))')],
     ["test_attention_bruteforce", "test_attention_special_cases"]),
    ("query heads mapped to KV heads modulo Hkv",
     [("heads = slice(g * group, (g + 1) * group)", "heads = slice(g, hq, hkv)")],
     ["test_attention_bruteforce", "test_attention_gqa_map_pin_catches_modulo_mapping"]),
    ("partials combined without renormalising to the whole key set",
     [("f64(l_s) - l_all, -np.inf", "f64(l_s), -np.inf")],
     ["test_split_kv_merge_identity", "test_lse_combine_closed_form_two_keys"]),
    ("RoPE pairs interleaved instead of rotate-half",
     [("lo, hi = x[..., :half], x[..., half:]", "lo, hi = x[..., 0::2], x[..., 1::2]")],
     ["test_rope_worked_example"]),
    ("RMSNorm epsilon outside the square root",
     [("r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)",
       "r = 1.0 / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps)")],
     ["test_rms_norm_closed_form_constant_row", "test_rms_norm_bruteforce_and_gain_matters"]),
    ("vocabulary shards sized by floor instead of padding up",
     [("rows = (vocab + n - 1) // n", "rows = max(vocab // n, 1)")],
     ["test_vocab_shards_reassemble_embedding_and_logits"]),
    ("embedding shard ignores its first id",
     [("onehot = (tokens[:, None] - firsts[i]) == np.arange(rows)[None, :]",
       "onehot = tokens[:, None] == np.arange(rows)[None, :]")],
     ["test_vocab_shards_reassemble_embedding_and_logits"]),
    ("head shard keeps KV heads by shard index instead of the heads its queries read",
     [("return [(i * per_shard, per_shard, kv[0], hk) for i, kv in enumerate(needs)]",
       "return [(i * per_shard, per_shard, (i * hk) % n_kv_heads, hk) for i, kv in enumerate(needs)]")],
     ["test_head_shards_exhaustive"]),
    ("MLP slices take W_down rows' first columns instead of the slice's columns",
     [("np.ascontiguousarray(wd[:, rows])", "np.ascontiguousarray(wd[:, :rows.stop - rows.start])")],
     ["test_mlp_slices_sum_to_full_mlp"]),
    ("K/V stored unrounded in a bf16 cache",
     [('"bf16": round_bf16,', '"bf16": lambda t: np.asarray(t, dtype=np.float32),')],
     ["test_kv_cache_holds_rotated_keys_in_the_cache_format"]),
]


def mutant_module(replacements):
    src = open(ORACLE_SRC).read()
    for old, new in replacements:
        assert src.count(old) == 1, f"statement to mutate not found exactly once: {old!r}"
        src = src.replace(old, new)
    mod = types.ModuleType("oracle_mutant")
    sys.modules["oracle_mutant"] = mod
    try:
        exec(compile(src, "oracle_mutant", "exec"), mod.__dict__)
    finally:
        del sys.modules["oracle_mutant"]
    return mod


def pin_calls(name):
    """Every parametrisation of one pin as a list of kwargs dicts."""
    fn = getattr(pins, name)
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    grids = []
    for m in marks:
        names = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
        vals = [v if isinstance(v, tuple) and len(names) > 1 else ((v,) if len(names) == 1 else v) for v in m.args[1]]
        grids.append([dict(zip(names, v)) for v in vals])
    if not grids:
        return fn, [{}]
    return fn, [dict(kv for d in combo for kv in d.items()) for combo in itertools.product(*grids)]


def fails(name, mod, monkeypatch) -> bool:
    """True if the pin fails (any exception) under some parametrisation with the oracle `mod`."""
    fn, calls = pin_calls(name)
    with monkeypatch.context() as m:
        m.setattr(pins, "o", mod)
        for kw in calls:
            try:
                fn(**kw)
            except Exception:
                return True
    return False


def test_pins_pass_on_the_unmutated_copy(monkeypatch):
    mod = mutant_module([])
    for name in sorted({p for _, _, ps in MUTATIONS for p in ps}):
        assert not fails(name, mod, monkeypatch), name


@pytest.mark.parametrize("name,replacements,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_its_pins(name, replacements, catchers, monkeypatch):
    mod = mutant_module(replacements)
    survived = [p for p in catchers if not fails(p, mod, monkeypatch)]
    assert not survived, f"mutation '{name}' passed pins {survived}"
