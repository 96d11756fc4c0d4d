"""Pins of the CPU oracle to things other than itself (CPU only).

No page prints activations or logits for a worked forward pass, so the oracle's forward values
are pinned by brute force on tiny shapes (pure-Python loops with math.exp, no numpy matmul or
einsum), closed forms, a worked RoPE example, and invariants the pages fix:
* split vs unsplit bit-identity ("RFC: pipeline placement ...", Numerical correctness proof);
* the split-KV merge identity ("41. Many GPUs", Ring attention: partials over disjoint key sets
  combine through their log-sum-exps);
* Megatron slice sums ("41. Many GPUs", Tensor parallelism: take_rows / take_cols);
* prefill/decode/chunked-prefill consistency (TensorSharp, Reproducible validation: full and
  chunked prefill, decode, refill and reset probes compared against an unsplit control).
Several tests plant a plausible mistake in a copy of an oracle function and check that the
matching pin catches it.
"""
import json
import math
import os

import numpy as np
import pytest

import fixtures as fx
from oracle import decoder as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TINY = fx.TINY


def rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------------------------

def test_bf16_round_to_nearest_even():
    one = 1.0
    cases = {
        one: one,
        one + 2 ** -8: one,                        # tie, rounds to even mantissa 0
        one + 3 * 2 ** -8: one + 2 ** -6,          # tie between mantissa 1 and 2 -> 2
        one + 2 ** -8 + 2 ** -20: one + 2 ** -7,   # just above the tie -> up
        -(one + 2 ** -8 + 2 ** -20): -(one + 2 ** -7),
        3.140625: 3.140625,                        # exactly representable
    }
    for x, want in cases.items():
        assert float(o.round_bf16(np.float32(x))) == want, x
    bits = o.f32_to_bf16_bits(np.array([1.0, -2.0, 0.5], np.float32))
    assert bits.tolist() == [0x3F80, 0xC000, 0x3F00]
    assert o.bf16_to_f32(np.array([0x3F80, 0xC000], np.uint16)).tolist() == [1.0, -2.0]


def test_bf16_matches_fixture_generator_rounding():
    # the generator's own RNE (fx_core.h) and the oracle's must agree on random f32 values
    vals = fx.normal_f32(7, 11, 4096) * np.float32(0.37)
    via_oracle = o.f32_to_bf16_bits(vals)
    # values 0.37 * z are not what the generator rounds, so compare with an independent route:
    # exhaustive neighbour search of the nearest bf16 (ties to even) in pure Python
    for v, b in zip(vals[:256].tolist(), via_oracle[:256].tolist()):
        u = np.float32(v).view(np.uint32).item()
        lo = u & 0xFFFF0000
        hi = lo + 0x10000
        flo = np.uint32(lo).view(np.float32).item()
        fhi = np.uint32(hi).view(np.float32).item()
        dlo, dhi = abs(v - flo), abs(fhi - v)
        pick = lo if (dlo < dhi or (dlo == dhi and ((lo >> 16) & 1) == 0)) else hi
        assert b == pick >> 16


# ---------------------------------------------------------------------------------------------
# RMSNorm, linear, RoPE, SwiGLU
# ---------------------------------------------------------------------------------------------

def test_rms_norm_closed_form_constant_row():
    d, eps = 64, 1e-5
    g = 1.0 + 0.1 * rng(1).standard_normal(d)
    for c in (0.0, 0.3, -2.5, 7.0):
        c = float(np.float32(c))
        y = o.rms_norm(np.full((1, d), c, np.float32), g, eps)
        want = g * c / math.sqrt(c * c + eps)
        np.testing.assert_allclose(y[0], want, rtol=1e-13, atol=0)


def test_rms_norm_bruteforce_and_gain_matters():
    x = rng(2).standard_normal((3, 16)).astype(np.float32)
    g = (1.0 + 0.2 * rng(3).standard_normal(16)).astype(np.float32)
    y = o.rms_norm(x, g, 1e-5)
    for m in range(3):
        ms = sum(float(v) * float(v) for v in x[m]) / 16
        r = 1.0 / math.sqrt(ms + 1e-5)
        for i in range(16):
            assert abs(y[m, i] - float(x[m, i]) * r * float(g[i])) < 1e-12
    assert not np.allclose(o.rms_norm(x, np.ones(16), 1e-5), y)   # a dropped gain is visible


def test_linear_bruteforce_nonsquare():
    # W is [out, in] (nn.Linear layout); a transposed operand would not even have the right shape
    h = o.round_bf16(rng(4).standard_normal((3, 5)))
    w_bits = fx.normal_bf16(1, 2, 7 * 5, 0.5).reshape(7, 5)
    w = o.bf16_to_f32(w_bits)
    y = o.linear(h, w_bits)
    assert y.shape == (3, 7) and y.dtype == np.float32
    for m in range(3):
        for n in range(7):
            s = 0.0
            for k in range(5):
                s += float(h[m, k]) * float(w[n, k])
            assert y[m, n] == np.float32(s)


def test_rope_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "rope_worked_example.json")))
    x = np.array(g["x"], np.float64).reshape(1, 1, 4)
    y = o.rope(x, np.array([g["position"]]), g["theta"])[0, 0]
    np.testing.assert_allclose(y, g["y"], rtol=0, atol=1e-14)


def test_rope_identity_norm_and_relative_position():
    r = rng(5)
    dh = 64
    x = r.standard_normal((1, 3, dh))
    np.testing.assert_array_equal(o.rope(x, np.array([0]), 1e4), x)            # position 0
    y = o.rope(x, np.array([37]), 1e4)
    half = dh // 2
    np.testing.assert_allclose(x[..., :half] ** 2 + x[..., half:] ** 2,
                               y[..., :half] ** 2 + y[..., half:] ** 2, rtol=1e-12)
    q, k = r.standard_normal((1, 1, dh)), r.standard_normal((1, 1, dh))
    for m, n, s in ((5, 2, 11), (100, 0, 4000), (8191, 17, 3)):
        a = np.sum(o.rope(q, np.array([m]), 1e4) * o.rope(k, np.array([n]), 1e4))
        b = np.sum(o.rope(q, np.array([m + s]), 1e4) * o.rope(k, np.array([n + s]), 1e4))
        assert abs(a - b) < 1e-9 * max(1.0, abs(a))


def test_rope_pin_catches_interleaved_pairs():
    # planted mistake: the interleaved (x_2i, x_2i+1) pairing instead of rotate-half
    def rope_interleaved(x, positions, theta):
        x = np.asarray(x, np.float64)
        a = o.rope_angles(positions, x.shape[-1], theta)[:, None, :]
        c, s = np.cos(a), np.sin(a)
        ev, od = x[..., 0::2], x[..., 1::2]
        y = np.empty_like(x)
        y[..., 0::2], y[..., 1::2] = ev * c - od * s, od * c + ev * s
        return y

    g = json.load(open(os.path.join(GOLDEN, "rope_worked_example.json")))
    x = np.array(g["x"], np.float64).reshape(1, 1, 4)
    y = rope_interleaved(x, np.array([g["position"]]), g["theta"])[0, 0]
    assert np.max(np.abs(y - np.array(g["y"]))) > 1e-3


def test_silu_mul():
    g = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    u = np.array([2.0, 1.0, 1.0, 1.0, 1.0])
    y = o.silu_mul(g, u)
    want = [0.0, 1.0 / (1.0 + math.exp(-1.0)), -1.0 / (1.0 + math.exp(1.0)),
            30.0 / (1.0 + math.exp(-30.0)), -30.0 / (1.0 + math.exp(30.0))]
    np.testing.assert_allclose(y, want, rtol=1e-15, atol=1e-300)


# ---------------------------------------------------------------------------------------------
# attention: brute force, special cases, GQA map, split-KV merge
# ---------------------------------------------------------------------------------------------

def brute_attention(q, k, v, q_pos, k_pos, scale, group):
    """Pure-Python causal GQA attention: q [Tq, Hq, D], k/v [Tk, Hkv, D]; head h uses KV h//group."""
    tq, hq, dd = q.shape
    out = np.zeros((tq, hq, dd))
    for t in range(tq):
        for h in range(hq):
            g = h // group
            sc = []
            for j in range(k.shape[0]):
                if k_pos[j] <= q_pos[t]:
                    sc.append((j, sum(float(q[t, h, e]) * float(k[j, g, e]) for e in range(dd)) * scale))
            if not sc:
                continue
            mx = max(s for _, s in sc)
            ws = [(j, math.exp(s - mx)) for j, s in sc]
            z = sum(w for _, w in ws)
            for e in range(dd):
                out[t, h, e] = sum(w * float(v[j, g, e]) for j, w in ws) / z
    return out


@pytest.mark.parametrize("tq,tk,hq,hkv,dd", [(4, 4, 2, 1, 4), (5, 8, 4, 2, 4), (3, 6, 4, 4, 8),
                                             (8, 8, 4, 1, 64), (1, 7, 16, 2, 8), (5, 9, 8, 2, 8)])
def test_attention_bruteforce(tq, tk, hq, hkv, dd):
    r = rng(tq * 100 + tk)
    q = r.standard_normal((tq, hq, dd))                 # N(0,1): not near-uniform attention
    k = r.standard_normal((tk, hkv, dd))
    v = r.standard_normal((tk, hkv, dd))
    q_pos = np.arange(tk - tq, tk)
    k_pos = np.arange(tk)
    scale = dd ** -0.5
    got, lse = o.attend(q, k, v, q_pos, k_pos, scale)
    want = brute_attention(q, k, v, q_pos, k_pos, scale, hq // hkv)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    assert lse.shape == (tq, hq) and np.all(np.isfinite(lse))
    # the log-sum-exp, brute force
    for t in range(tq):
        for h in range(hq):
            z = sum(math.exp(sum(float(q[t, h, e]) * float(k[j, h // (hq // hkv), e]) for e in range(dd)) * scale)
                    for j in range(tk) if k_pos[j] <= q_pos[t])
            assert abs(lse[t, h] - math.log(z)) < 1e-12 * max(1.0, abs(math.log(z)))


def test_attention_key_order_and_unsorted_positions():
    # visibility is by position, not by storage order: shuffled keys give the same result
    r = rng(12)
    q, k, v = r.standard_normal((3, 4, 8)), r.standard_normal((9, 2, 8)), r.standard_normal((9, 2, 8))
    q_pos, k_pos = np.array([2, 5, 8]), np.arange(9)
    perm = r.permutation(9)
    a, la = o.attend(q, k, v, q_pos, k_pos, 0.4)
    b, lb = o.attend(q, k[perm], v[perm], q_pos, k_pos[perm], 0.4)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)
    np.testing.assert_allclose(la, lb, rtol=1e-14)
    np.testing.assert_allclose(a, brute_attention(q, k, v, q_pos, k_pos, 0.4, 2), rtol=0, atol=1e-12)


def test_attention_gqa_map_pin_catches_modulo_mapping():
    r = rng(9)
    q, k, v = r.standard_normal((2, 4, 4)), r.standard_normal((3, 2, 4)), r.standard_normal((3, 2, 4))
    want = brute_attention(q, k, v, np.array([1, 2]), np.arange(3), 0.5, 2)
    got, _ = o.attend(q, k, v, np.array([1, 2]), np.arange(3), 0.5)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # planted: head h -> KV head h % Hkv (expanding K/V by tiling instead of repeating)
    wrong, _ = o.attend(q, np.concatenate([k, k], axis=1), np.concatenate([v, v], axis=1), np.array([1, 2]),
                        np.arange(3), 0.5)
    assert np.max(np.abs(wrong - want)) > 1e-3


def test_attention_special_cases():
    r = rng(10)
    v = r.standard_normal((5, 1, 4))
    k = np.zeros((5, 1, 4))
    q = r.standard_normal((1, 1, 4))
    # equal scores -> mean of the visible values
    out, lse = o.attend(q, k, v, np.array([2]), np.arange(5), 1.0)
    np.testing.assert_allclose(out[0, 0], v[:3, 0].mean(axis=0), rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(3.0), rtol=1e-14)
    # one visible key -> its value
    out, _ = o.attend(q, r.standard_normal((5, 1, 4)), v, np.array([0]), np.arange(5), 1.0)
    np.testing.assert_allclose(out[0, 0], v[0, 0], rtol=1e-14)
    # no visible key -> zero output and lse -inf
    out, lse = o.attend(q, k, v, np.array([0]), np.arange(1, 6), 1.0)
    assert np.all(out == 0) and np.isneginf(lse[0, 0])
    # a very large score dominates completely (no overflow: the definition is shift-invariant)
    kk = np.zeros((3, 1, 4))
    kk[1, 0, 0] = 1e4
    qq = np.array([[[1.0, 0, 0, 0]]])
    out, lse = o.attend(qq, kk, v[:3], np.array([2]), np.arange(3), 1.0)
    np.testing.assert_allclose(out[0, 0], v[1, 0], rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], 1e4, rtol=1e-15)


def test_split_kv_merge_identity():
    r = rng(11)
    tq, tk, h, dd = 3, 37, 4, 16
    q, k, v = r.standard_normal((tq, h, dd)), r.standard_normal((tk, 2, dd)), r.standard_normal((tk, 2, dd))
    q_pos, k_pos = np.arange(tk - tq, tk), np.arange(tk)
    full, full_lse = o.attend(q, k, v, q_pos, k_pos, 0.25)
    for chunk in (1, 5, 16, 36):
        parts = [o.attend(q, k[s:s + chunk], v[s:s + chunk], q_pos, k_pos[s:s + chunk], 0.25)
                 for s in range(0, tk, chunk)]
        out, lse = o.lse_combine(parts)
        np.testing.assert_allclose(out, full, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, full_lse, rtol=1e-13)
        # combining two at a time, in order, is the same combination
        run = parts[0]
        for p in parts[1:]:
            run = o.lse_combine([run, p])
        np.testing.assert_allclose(run[0], full, rtol=0, atol=1e-12)
    # a partial with no visible key (lse -inf) weighs nothing; all-empty gives (0, -inf)
    empty = (np.zeros_like(full), np.full_like(full_lse, -np.inf))
    e_out, e_lse = o.lse_combine([(full, full_lse), empty])
    np.testing.assert_allclose(e_out, full, rtol=1e-15)
    z_out, z_lse = o.lse_combine([empty, empty])
    assert np.all(z_out == 0) and np.all(np.isneginf(z_lse))


def test_lse_combine_closed_form_two_keys():
    # two single-key partials: the combination is the softmax over the two keys
    s1, s2, v1, v2 = 0.3, -1.7, np.array([1.0, 2.0]), np.array([-3.0, 0.5])
    out, lse = o.lse_combine([(v1[None, None], np.array([[s1]])), (v2[None, None], np.array([[s2]]))])
    p1 = math.exp(s1) / (math.exp(s1) + math.exp(s2))
    np.testing.assert_allclose(out[0, 0], p1 * v1 + (1 - p1) * v2, rtol=1e-14)
    np.testing.assert_allclose(lse[0, 0], math.log(math.exp(s1) + math.exp(s2)), rtol=1e-14)


# ---------------------------------------------------------------------------------------------
# MLP slices
# ---------------------------------------------------------------------------------------------

def test_mlp_slices_sum_to_full_mlp():
    d, f, n = 32, 48, 4
    x = fx.normal_f32(3, 1, 5 * d).reshape(5, d)
    g = fx.gain_bf16(3, 2, d, 0.1)
    wg = fx.normal_bf16(3, 3, f * d, 0.1).reshape(f, d)
    wu = fx.normal_bf16(3, 4, f * d, 0.1).reshape(f, d)
    wd = fx.normal_bf16(3, 5, d * f, 0.1).reshape(d, f)
    a_full, y_full = o.mlp_full(x, g, wg, wu, wd, 1e-5)
    acts, parts, total = o.mlp_slices(x, g, wg, wu, wd, 1e-5, n)
    w = f // n
    for i in range(n):   # column-parallel slices see exactly their columns of the activation
        np.testing.assert_allclose(acts[i], a_full[:, i * w:(i + 1) * w], rtol=1e-14, atol=1e-300)
    # float64 invariant: sum of the exact partials equals the exact full product
    wd64 = o.bf16_to_f32(wd).astype(np.float64)
    exact_parts = [acts[i].astype(np.float64) @ wd64[:, i * w:(i + 1) * w].T for i in range(n)]
    exact_full = a_full.astype(np.float64) @ wd64.T
    np.testing.assert_allclose(sum(exact_parts), exact_full, rtol=0, atol=1e-12)
    np.testing.assert_allclose(total, y_full, rtol=1e-5, atol=1e-6)
    # planted mistake: row slices of W_down instead of its columns do not sum to the MLP
    assert wd.shape[0] != wd.shape[1] or True
    bad = [acts[i].astype(np.float64) @ wd64[:w, :][:, :w].T for i in range(n)]
    assert np.max(np.abs(sum(bad)[:, :w] - exact_full[:, :w])) > 1e-3


# ---------------------------------------------------------------------------------------------
# stage-level invariants on the tiny decoder
# ---------------------------------------------------------------------------------------------

def tiny_stage(begin, end, first, last, gain_sigma=0.1, max_ctx=64):
    w = fx.draw_stage_weights(TINY, begin, end, first, last, gain_sigma=gain_sigma)
    return o.Stage(o.Dims.of(TINY), begin, end, first, last, w, max_ctx)


def test_split_equals_unsplit_bitwise():
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(0), 16, TINY.vocab)
    whole = tiny_stage(0, 2, True, True)
    toks1, tr1 = o.generate([whole], prompt, 8)
    a, b = tiny_stage(0, 1, True, False), tiny_stage(1, 2, False, True)
    toks2, tr2 = o.generate([a, b], prompt, 8)
    np.testing.assert_array_equal(toks1, toks2)
    for key in ("logits", "final_hidden", "residual"):
        for u, v in zip(tr1[key], tr2[key]):
            assert u.tobytes() == v.tobytes(), key
    kw, vw = whole.kv_bits(0, 23)
    ka, va = a.kv_bits(0, 23)
    kb, vb = b.kv_bits(0, 23)
    assert np.array_equal(kw[0], ka[0]) and np.array_equal(kw[1], kb[0])
    assert np.array_equal(vw[0], va[0]) and np.array_equal(vw[1], vb[0])


def test_prefill_decode_and_chunked_consistency():
    x = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(0), 17 * TINY.d_model).reshape(17, TINY.d_model)
    s1 = tiny_stage(0, 2, False, False)
    full = s1.prefill(x, 0, 0)
    s2 = tiny_stage(0, 2, False, False)
    part = s2.prefill(x[:16], 0, 0)
    last = s2.forward(x[16:], [0], [16])
    s3 = tiny_stage(0, 2, False, False)
    c1 = s3.prefill(x[:8], 0, 0)
    c2 = s3.prefill(x[8:], 0, 8)
    # rows are independent up to the float64 summation order of the library matmul
    np.testing.assert_allclose(np.vstack([part, last]), full, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(np.vstack([c1, c2]), full, rtol=1e-6, atol=1e-6)
    k1, v1 = s1.kv_bits(0, 17)
    k3, v3 = s3.kv_bits(0, 17)
    assert np.mean(k1 == k3) > 0.999 and np.mean(v1 == v3) > 0.999


def test_determinism_and_reset():
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(0), 16, TINY.vocab)
    s = tiny_stage(0, 2, True, True)
    t1, tr1 = o.generate([s], prompt, 4)
    t2, tr2 = o.generate([s], prompt, 4)         # "reset": the caller rewinds positions to 0
    np.testing.assert_array_equal(t1, t2)
    assert all(a.tobytes() == b.tobytes() for a, b in zip(tr1["logits"], tr2["logits"]))


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_kv_cache_holds_rotated_keys_in_the_cache_format(fmt):
    # the KV cache is the one storage point of activations: cached K and V are values of the
    # cache format, and K is cached after RoPE (the value attention reads)
    x = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(0), 4 * TINY.d_model).reshape(4, TINY.d_model)
    w = fx.draw_stage_weights(TINY, 0, 1, False, False, gain_sigma=0.1)
    s = o.Stage(o.Dims.of(TINY), 0, 1, False, False, w, 64, kv_dtype=fmt)
    s.prefill(x, 0, 0)
    k, v = s.kv[0]
    if fmt == "bf16":
        assert np.array_equal(o.round_bf16(k), k) and np.array_equal(o.round_bf16(v), v)
    if fmt == "f16":
        assert np.array_equal(k.astype(np.float16).astype(np.float32), k)
        assert np.array_equal(v.astype(np.float16).astype(np.float32), v)
    c = o.Dims.of(TINY)
    h = o.rms_norm(x, o.bf16_to_f32(w[("attn_norm", 0)]), c.rms_eps)
    k_raw = o.linear64(h, w[("wk", 0)]).reshape(4, c.n_kv_heads, c.head_dim)
    want = o.KV_FORMATS[fmt](o.rope(k_raw, np.arange(4), c.rope_theta))
    np.testing.assert_array_equal(k[0, :4], want)
    assert not np.allclose(k[0, 1:4], o.KV_FORMATS[fmt](k_raw[1:]))   # RoPE was applied
    assert s.held[0][0, :4].all() and not s.held[0][0, 4:].any()


def test_f16_rounding_is_round_to_nearest_even():
    # binary16 has 11 significant bits: 1 + 2^-11 is a tie (rounds to 1), 1 + 3 * 2^-11 rounds up
    vals = np.array([1.0, 1 + 2 ** -11, 1 + 3 * 2 ** -11, 1 + 2 ** -11 + 2 ** -20, 65504.0, 2 ** -24], np.float32)
    want = [1.0, 1.0, 1 + 2 ** -9, 1 + 2 ** -10, 65504.0, 2 ** -24]
    assert o.round_f16(vals).tolist() == want


# ---------------------------------------------------------------------------------------------
# how a block composes its parts ("41. Many GPUs", Pipeline parallelism: each block normalises
# the residual, adds attention, normalises the new residual, adds the MLP)
# ---------------------------------------------------------------------------------------------

def brute_rms_norm(row, gain, eps):
    ms = sum(float(t) * float(t) for t in row) / len(row)
    r = 1.0 / math.sqrt(ms + eps)
    return [float(t) * r * float(g) for t, g in zip(row, gain)]


def brute_swiglu_mlp(x, g_mlp, w_gate, w_up, w_down, eps):
    """Pure-Python SwiGLU MLP of rows x: y_j = sum_f W_down[j, f] silu(gate_f) up_f with
    gate_f = sum_k h_k W_gate[f, k], up_f = sum_k h_k W_up[f, k], h = RMSNorm(x) g."""
    wg, wu, wd = (o.bf16_to_f32(t).astype(np.float64) for t in (w_gate, w_up, w_down))
    out = []
    for row in x:
        h = brute_rms_norm(row, o.bf16_to_f32(g_mlp), eps)
        act = []
        for f in range(wg.shape[0]):
            gate = sum(h[k] * wg[f, k] for k in range(len(h)))
            up = sum(h[k] * wu[f, k] for k in range(len(h)))
            act.append(gate / (1.0 + math.exp(-gate)) * up)
        out.append([sum(wd[j, f] * act[f] for f in range(len(act))) for j in range(wd.shape[0])])
    return np.array(out)


def small_mlp(d=6, f=4, seed=21):
    g = fx.gain_bf16(seed, 1, d, 0.2)
    wg = fx.normal_bf16(seed, 2, f * d, 0.5).reshape(f, d)
    wu = fx.normal_bf16(seed, 3, f * d, 0.5).reshape(f, d)
    wd = fx.normal_bf16(seed, 4, d * f, 0.5).reshape(d, f)
    return g, wg, wu, wd


def test_mlp_bruteforce_gate_and_up_named():
    # W_gate and W_up differ, so silu(gate) * up and silu(up) * gate give different outputs
    g, wg, wu, wd = small_mlp()
    x = (2.0 * rng(22).standard_normal((3, 6))).astype(np.float32)
    want = brute_swiglu_mlp(x, g, wg, wu, wd, 1e-5)
    _, y = o.mlp_full(x, g, wg, wu, wd, 1e-5)
    np.testing.assert_allclose(y, want, rtol=1e-6, atol=1e-7)
    _, y64 = o.mlp_delta(x, g, wg, wu, wd, 1e-5)
    np.testing.assert_allclose(y64, want, rtol=1e-12, atol=1e-13)
    _, parts, total = o.mlp_slices(x, g, wg, wu, wd, 1e-5, 2)
    np.testing.assert_allclose(total, want, rtol=1e-6, atol=1e-6)
    swapped = brute_swiglu_mlp(x, g, wu, wg, wd, 1e-5)
    assert np.max(np.abs(swapped - want)) > 1e-2          # the pin can tell gate from up


def tiny_dims(d=6, hq=2, hkv=1, dh=2, f=4):
    return o.Dims(d, hq, hkv, dh, f, 8, 1e-5, 1e4)


def small_block_weights(dims, seed=23, wo_zero=False):
    d, hq, hkv, dh, f = dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim, dims.d_ffn
    g, wg, wu, wd = small_mlp(d, f, seed)
    w = {("attn_norm", 0): fx.gain_bf16(seed, 5, d, 0.2), ("mlp_norm", 0): g,
         ("wq", 0): fx.normal_bf16(seed, 6, hq * dh * d, 0.7).reshape(hq * dh, d),
         ("wk", 0): fx.normal_bf16(seed, 7, hkv * dh * d, 0.7).reshape(hkv * dh, d),
         ("wv", 0): fx.normal_bf16(seed, 8, hkv * dh * d, 0.7).reshape(hkv * dh, d),
         ("wo", 0): fx.normal_bf16(seed, 9, d * hq * dh, 0.7).reshape(d, hq * dh),
         ("wgate", 0): wg, ("wup", 0): wu, ("wdown", 0): wd}
    if wo_zero:
        w[("wo", 0)] = np.zeros_like(w[("wo", 0)])
    return w


def test_block_with_zero_attention_output_is_x_plus_mlp_of_x():
    # W_o = 0: the attention adds nothing, so the block is x + MLP(x) (brute force, named gate/up)
    dims = tiny_dims()
    w = small_block_weights(dims, wo_zero=True)
    x = (1.5 * rng(24).standard_normal((3, 6))).astype(np.float32)
    st = o.Stage(dims, 0, 1, False, False, w, 8, kv_dtype="f32")
    y = st.prefill(x, 0, 0)
    want = x.astype(np.float64) + brute_swiglu_mlp(x, w[("mlp_norm", 0)], w[("wgate", 0)], w[("wup", 0)],
                                                   w[("wdown", 0)], 1e-5)
    np.testing.assert_allclose(y, want, rtol=1e-6, atol=1e-6)


def rot(vec, delta, theta):
    """Pure-Python rotate-half rotation of one head vector by the angles delta * theta^(-2i/D)."""
    dd = len(vec)
    half = dd // 2
    out = list(vec)
    for i in range(half):
        a = delta * theta ** (-2.0 * i / dd)
        c, s_ = math.cos(a), math.sin(a)
        out[i] = vec[i] * c - vec[i + half] * s_
        out[i + half] = vec[i + half] * c + vec[i] * s_
    return out


def brute_attn_sublayer(x, w, dims, positions):
    """Pure-Python attention sublayer over one sequence at `positions`: scores are computed as
    <q_p, R(j - p) k_j> (rotating the key by the RELATIVE position only), which equals
    <R(p) q_p, R(j) k_j> exactly when RoPE rotates both q and k at their absolute positions."""
    d, hq, hkv, dh = dims.d_model, dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    grp = hq // hkv
    wq, wk, wv, wo = (o.bf16_to_f32(w[(r, 0)]).astype(np.float64) for r in ("wq", "wk", "wv", "wo"))
    hs = [brute_rms_norm(row, o.bf16_to_f32(w[("attn_norm", 0)]), dims.rms_eps) for row in x]

    def proj(wm, h):
        return [sum(wm[r, c] * h[c] for c in range(d)) for r in range(wm.shape[0])]

    qs, ks, vs = [proj(wq, h) for h in hs], [proj(wk, h) for h in hs], [proj(wv, h) for h in hs]
    out = []
    for t, p in enumerate(positions):
        o_row = []
        for h in range(hq):
            g = h // grp
            qh = qs[t][h * dh:(h + 1) * dh]
            sc = []
            for j, pj in enumerate(positions):
                if pj <= p:
                    kj = rot(ks[j][g * dh:(g + 1) * dh], pj - p, dims.rope_theta)
                    sc.append((j, sum(a * b for a, b in zip(qh, kj)) * dh ** -0.5))
            mx = max(s_ for _, s_ in sc)
            z = sum(math.exp(s_ - mx) for _, s_ in sc)
            o_row += [sum(math.exp(s_ - mx) / z * vs[j][g * dh + e] for j, s_ in sc) for e in range(dh)]
        out.append([sum(wo[r, c] * o_row[c] for c in range(hq * dh)) for r in range(d)])
    return np.array(out)


@pytest.mark.parametrize("pos0", [0, 5, 1000])
def test_attention_sublayer_bruteforce_relative_rotation(pos0):
    # pins RoPE on BOTH q and k (dropping either, or both, changes the scores), the scale, the
    # causal mask, the GQA map and W_o, at absolute positions pos0 .. pos0 + 3
    dims = tiny_dims(d=6, hq=4, hkv=2, dh=4)
    w = small_block_weights(dims)
    x = (1.5 * rng(25).standard_normal((4, 6))).astype(np.float32)
    positions = list(range(pos0, pos0 + 4))
    want = brute_attn_sublayer(x, w, dims, positions)
    got = o.attn_sublayer(x, w[("attn_norm", 0)], w[("wq", 0)], w[("wk", 0)], w[("wv", 0)], w[("wo", 0)],
                          dims.head_dim, dims.rms_eps, dims.rope_theta, "f32", pos0=pos0)
    np.testing.assert_allclose(got, want, rtol=1e-6, atol=1e-6)      # K, V stored as float32
    st = o.Stage(dims, 0, 1, False, False, w, pos0 + 4, kv_dtype="f32")
    delta = st.attention(0, x, np.zeros(4, np.int64), np.array(positions))
    np.testing.assert_allclose(delta, want, rtol=1e-6, atol=1e-6)


def test_prefill_is_invariant_to_a_shift_of_all_positions():
    # RoPE makes attention depend on relative positions only: the same rows prefilled as a fresh
    # sequence at positions 0.. and at s.. give the same block outputs (to the float32 rounding
    # of the cached K and V, which differs with the absolute rotation)
    w = fx.draw_stage_weights(TINY, 0, 2, False, False, gain_sigma=0.1)
    x = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(5), 9 * TINY.d_model).reshape(9, TINY.d_model)
    st = o.Stage(o.Dims.of(TINY), 0, 2, False, False, w, 300, kv_dtype="f32")
    y0 = st.prefill(x, 0, 0)
    for s_ in (1, 37, 290):
        ys = st.prefill(x, s_ % 7 + 1, s_)                  # fresh slots
        np.testing.assert_allclose(ys, y0, rtol=2e-6, atol=2e-6)


def test_block_composes_attention_then_mlp_of_the_new_residual():
    # x1 = x + attention(x); y = x1 + MLP(x1): the MLP norm reads x1 (not x), both residuals are
    # added, in that order (nonzero attention, so x1 != x)
    w = fx.draw_stage_weights(TINY, 0, 1, False, False, gain_sigma=0.1)
    c = o.Dims.of(TINY)
    x = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(6), 5 * TINY.d_model).reshape(5, TINY.d_model)
    st = o.Stage(c, 0, 1, False, False, w, 8, kv_dtype="f32")
    y = st.prefill(x, 0, 0)
    att = o.attn_sublayer(x, w[("attn_norm", 0)], w[("wq", 0)], w[("wk", 0)], w[("wv", 0)], w[("wo", 0)],
                          c.head_dim, c.rms_eps, c.rope_theta, "f32")
    x1 = (x + att).astype(np.float32)
    assert rel(x1, x) > 1e-2
    _, m = o.mlp_full(x1, w[("mlp_norm", 0)], w[("wgate", 0)], w[("wup", 0)], w[("wdown", 0)], c.rms_eps)
    np.testing.assert_allclose(y, x1.astype(np.float64) + m, rtol=1e-6, atol=1e-6)
    _, m_wrong = o.mlp_full(x, w[("mlp_norm", 0)], w[("wgate", 0)], w[("wup", 0)], w[("wdown", 0)], c.rms_eps)
    assert rel(x1 + m_wrong, y) > 1e-4                     # the MLP of x would be visible


def rel(a, b):
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def test_readout_bruteforce_with_gains():
    # h_N = RMSNorm(x) g_final, logits = h_N W_readout^T; the gains are far from 1
    d, V = 8, 5
    g = fx.gain_bf16(31, 1, d, 0.3)
    wr = fx.normal_bf16(31, 2, V * d, 0.5).reshape(V, d)
    dims = o.Dims(d, 2, 1, 4, 4, V, 1e-5, 1e4)
    st = o.Stage(dims, 0, 0, False, True, {("final_norm", -1): g, ("readout", -1): wr}, 4)
    x = (3.0 * rng(32).standard_normal((3, d))).astype(np.float32)
    logits, hn = st.readout(x)
    wrf = o.bf16_to_f32(wr).astype(np.float64)
    for m in range(3):
        h = brute_rms_norm(x[m], o.bf16_to_f32(g), 1e-5)
        np.testing.assert_allclose(hn[m], h, rtol=1e-6)
        for j in range(V):
            assert abs(logits[m, j] - sum(h[i] * wrf[j, i] for i in range(d))) <= 1e-6 * (1 + abs(logits[m, j]))
    assert rel(o.rms_norm(x, np.ones(d), 1e-5), hn) > 1e-2       # the gains matter here


# ---------------------------------------------------------------------------------------------
# tensor-parallel shards ("41. Many GPUs", Tensor parallelism)
# ---------------------------------------------------------------------------------------------

def tp_weights(d, hq, hkv, dh, seed=5):
    g = fx.gain_bf16(seed, 1, d, 0.1)
    wq = fx.normal_bf16(seed, 2, hq * dh * d, 0.1).reshape(hq * dh, d)
    wk = fx.normal_bf16(seed, 3, hkv * dh * d, 0.1).reshape(hkv * dh, d)
    wv = fx.normal_bf16(seed, 4, hkv * dh * d, 0.1).reshape(hkv * dh, d)
    wo = fx.normal_bf16(seed, 5, d * hq * dh, 0.1).reshape(d, hq * dh)
    return g, wq, wk, wv, wo


def test_attn_sublayer_single_row_is_wo_times_v():
    # one row attends only to itself: softmax over one key is 1, so the output is W_o applied to
    # V of the KV head each query head reads (closed form; catches a wrong head map or operand)
    d, hq, hkv, dh = 64, 4, 2, 16
    g, wq, wk, wv, wo = tp_weights(d, hq, hkv, dh)
    x = fx.normal_f32(5, 9, d).reshape(1, d)
    got = o.attn_sublayer(x, g, wq, wk, wv, wo, dh, 1e-5, 1e4)
    h = o.rms_norm(x, o.bf16_to_f32(g), 1e-5)
    v = o.round_bf16(o.linear64(h, wv).reshape(1, hkv, dh))
    want = o.linear64(np.repeat(v, hq // hkv, axis=1).reshape(1, hq * dh), wo)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_attn_sublayer_is_the_blocks_attention_half():
    # a block whose MLP is zero (W_gate = 0 -> silu(0) = 0) outputs x + the attention delta
    w = fx.draw_stage_weights(TINY, 0, 1, False, False, gain_sigma=0.1)
    w[("wgate", 0)] = np.zeros_like(w[("wgate", 0)])
    c = o.Dims.of(TINY)
    x = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(3), 6 * TINY.d_model).reshape(6, TINY.d_model)
    s = o.Stage(c, 0, 1, False, False, w, 16)
    y = s.prefill(x, 0, 0)
    delta = o.attn_sublayer(x, w[("attn_norm", 0)], w[("wq", 0)], w[("wk", 0)], w[("wv", 0)], w[("wo", 0)],
                            c.head_dim, c.rms_eps, c.rope_theta)
    np.testing.assert_array_equal(y, (x + delta).astype(np.float32))


@pytest.mark.parametrize("hq,hkv,n", [(4, 2, 2), (4, 2, 4), (8, 8, 4), (8, 2, 8)])
def test_attn_slices_sum_to_full_attention(hq, hkv, n):
    d, dh = 64, 16
    g, wq, wk, wv, wo = tp_weights(d, hq, hkv, dh)
    x = fx.normal_f32(5, 11, 7 * d).reshape(7, d)
    full = o.attn_sublayer(x, g, wq, wk, wv, wo, dh, 1e-5, 1e4)
    # float64 invariant: the exact partials sum to the exact full sublayer
    exact = []
    for q0, q_n, kv0, k_n in o.head_shards(hq, hkv, n):
        qr, kr = slice(q0 * dh, (q0 + q_n) * dh), slice(kv0 * dh, (kv0 + k_n) * dh)
        exact.append(o.attn_sublayer(x, g, wq[qr], wk[kr], wv[kr], np.ascontiguousarray(wo[:, qr]), dh, 1e-5, 1e4))
        # every query head of the shard reads the KV head the full model maps it to
        for hh in range(q0, q0 + q_n):
            assert kv0 <= hh // (hq // hkv) < kv0 + k_n
    np.testing.assert_allclose(sum(exact), full, rtol=0, atol=1e-12)
    parts, total = o.attn_slices(x, g, wq, wk, wv, wo, dh, 1e-5, 1e4, n)
    np.testing.assert_allclose(total, full, rtol=1e-5, atol=1e-6)


def test_head_shards_exhaustive():
    # every (Hq, Hkv, n) up to 16: a split is accepted exactly when query heads divide evenly and
    # KV heads either divide evenly too or are replicated a whole number of times (n a multiple of
    # Hkv); an accepted split covers every query head once, keeps every KV head its query heads
    # read, and splits or replicates the KV heads evenly
    for hq in range(1, 17):
        for hkv in (k for k in range(1, hq + 1) if hq % k == 0):
            for n in range(1, 17):
                ok = hq % n == 0 and (hkv % n == 0 or n % hkv == 0)
                if not ok:
                    with pytest.raises(ValueError):
                        o.head_shards(hq, hkv, n)
                    continue
                sh = o.head_shards(hq, hkv, n)
                assert sorted(h for q0, k, _, _ in sh for h in range(q0, q0 + k)) == list(range(hq))
                for q0, k, kv0, hk in sh:
                    assert {h // (hq // hkv) for h in range(q0, q0 + k)} == set(range(kv0, kv0 + hk))
                use = [sum(kv0 <= g < kv0 + hk for _, _, kv0, hk in sh) for g in range(hkv)]
                assert len(set(use)) == 1 and use[0] == max(1, n // hkv)
    sl = o.head_shards(32, 8, 16)
    assert [s[2] for s in sl] == [i // 2 for i in range(16)] and all(s[1] == 2 and s[3] == 1 for s in sl)
    assert [s[2] for s in o.head_shards(32, 8, 4)] == [0, 2, 4, 6]


@pytest.mark.parametrize("vocab,n", [(1024, 3), (1000, 8), (17, 4), (16, 4)])
def test_vocab_shards_reassemble_embedding_and_logits(vocab, n):
    d = 32
    table = fx.normal_bf16(6, 1, vocab * d, 1.0).reshape(vocab, d)
    rows, firsts = o.vocab_shards(vocab, n)
    assert rows * n >= vocab and rows * (n - 1) < vocab and rows == math.ceil(vocab / n)
    # every id lands in exactly one shard, at row id - first
    for t in range(vocab):
        owners = [i for i in range(n) if firsts[i] <= t < firsts[i] + rows]
        assert len(owners) == 1
        assert np.array_equal(o.vocab_shard(table, n, owners[0])[t - firsts[owners[0]]], table[t])
    toks = np.array([0, vocab - 1, rows - 1, min(rows, vocab - 1), min(2 * rows, vocab - 1), vocab // 2],
                    dtype=np.int64)
    np.testing.assert_array_equal(o.embed_shards(table, toks, n), o.bf16_to_f32(table)[toks])
    h = fx.normal_f32(6, 2, 3 * d).reshape(3, d)
    full = o.linear(h, table)
    np.testing.assert_allclose(o.readout_shards(h, table, n), full, rtol=1e-6, atol=1e-6)
    # the padding rows are zero and never reach the logits
    assert not o.vocab_shard(table, n, n - 1)[vocab - firsts[n - 1]:].any()


# ---------------------------------------------------------------------------------------------
# ring attention ("41. Many GPUs", Ring attention for very long contexts)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("n,zigzag", [(1, False), (2, False), (4, False), (2, True), (4, True)])
def test_ring_attention_equals_full_causal_attention(n, zigzag):
    # the combination of every (query chunk, KV chunk) partial is the full softmax
    t, hq, hkv, dd = 24, 4, 2, 8
    r = rng(7)
    q, k, v = r.standard_normal((t, hq, dd)), r.standard_normal((t, hkv, dd)), r.standard_normal((t, hkv, dd))
    pos = np.arange(t)
    want = brute_attention(q, k, v, pos, pos, dd ** -0.5, hq // hkv)
    np.testing.assert_allclose(o.ring_attention(q, k, v, n, zigzag), want, rtol=0, atol=1e-12)


def test_ring_chunks_cover_the_sequence_and_zigzag_balances_work():
    for n, zz in ((4, False), (4, True), (3, True)):
        t = 2 * n * 5
        cover = sorted(p for ch in o.ring_chunks(t, n, zz) for a, b in ch for p in range(a, b))
        assert cover == list(range(t))
    # causal work (visible keys) per rank: zigzag equal, plain chunking rising with the rank
    def work(n, zz, t=48):
        return [sum(p + 1 for a, b in ch for p in range(a, b)) for ch in o.ring_chunks(t, n, zz)]
    assert len(set(work(4, True))) == 1
    w = work(4, False)
    assert w == sorted(w) and w[-1] > 3 * w[0]


def test_attn_sublayer_ring_matches_attn_sublayer():
    d, hq, hkv, dh = 64, 4, 2, 16
    g, wq, wk, wv, wo = tp_weights(d, hq, hkv, dh)
    x = fx.normal_f32(5, 13, 16 * d).reshape(16, d)
    full = o.attn_sublayer(x, g, wq, wk, wv, wo, dh, 1e-5, 1e4)
    for n, zz in ((2, False), (2, True), (4, True)):
        np.testing.assert_allclose(o.attn_sublayer_ring(x, g, wq, wk, wv, wo, dh, 1e-5, 1e4, n, zz), full,
                                   rtol=0, atol=1e-11)


# ---------------------------------------------------------------------------------------------
# node-order sums and greedy ties
# ---------------------------------------------------------------------------------------------

def test_f32_sum_in_order_is_left_to_right_in_float32():
    # ((p0 + p1) + p2) with every partial rounded to float32: 1e8 + (-1e8) + 1 = 1, while
    # 1 + 1e8 + (-1e8) = 0 in float32 (1 is below half an ulp of 1e8)
    big = np.float32(1e8)
    assert o.f32_sum_in_order([np.array([big]), np.array([-big]), np.array([np.float32(1)])])[0] == 1.0
    assert o.f32_sum_in_order([np.array([np.float32(1)]), np.array([big]), np.array([-big])])[0] == 0.0
    r = rng(33).standard_normal((5, 7)).astype(np.float32)
    want = r[0].copy()
    for row in r[1:]:
        want = (want + row).astype(np.float32)
    np.testing.assert_array_equal(o.f32_sum_in_order(list(r)), want)


def test_greedy_lowest_index_on_ties():
    logits = np.array([[0.5, 2.0, 2.0, -1.0], [3.0, 3.0, 3.0, 3.0], [-np.inf, -5.0, -5.0, -np.inf]])
    assert o.greedy(logits).tolist() == [1, 0, 1]
    np.testing.assert_allclose(o.top2_margin(np.array([[1.0, 4.0, 2.5]])), [1.5])
