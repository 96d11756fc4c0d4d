"""GPU parity on the tiny decoder (2 blocks, d 256, 4 q / 2 KV heads, Dh 64, F 688, V 1024).

Compares the HIP path (through the C ABI) with the CPU oracle on the same seeded weights and
inputs: relative L2 <= 1e-3 on hidden rows and logits, identical greedy tokens, and bit-identical
split-vs-unsplit results on the GPU itself ("RFC: pipeline placement ...", Numerical correctness
proof: logits, final features, KV state and generated tokens must match bit for bit).
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from oracle import decoder as o
from tests.gpu_util import gpu_generate, hidden_rows, kv_bits, kv_values, make_stage, rel_l2, rel_l2_kv, say

pytestmark = pytest.mark.gpu

TINY = fx.TINY
TOL = 1e-3


@pytest.fixture(scope="module")
def weights():
    return fx.draw_stage_weights(TINY, 0, 2, True, True, gain_sigma=0.1)


def oracle_stage(w, begin, end, first, last, max_ctx=64, kv_dtype="bf16"):
    return o.Stage(o.Dims.of(TINY), begin, end, first, last, w, max_ctx, kv_dtype=kv_dtype)


@pytest.mark.parametrize("kv", ["bf16", "f32", "f16"])
def test_tiny_greedy_parity(weights, kv):
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(0), 16, TINY.vocab)
    say("tiny greedy: oracle")
    want_toks, want = o.generate([oracle_stage(weights, 0, 2, True, True, kv_dtype=kv)],
                                 prompt, 8)
    say("tiny greedy: gpu")
    st = make_stage(TINY, 0, 2, True, True, weights, max_slots=2, max_ctx=64, max_tokens=16, kv=kv)
    got_toks, got = gpu_generate([st], prompt, 8)
    for step in range(8):
        for key in ("logits", "final_hidden", "residual"):
            e = rel_l2(got[key][step], want[key][step])
            assert e <= TOL, (step, key, e)
    margins = [float(o.top2_margin(l[-1:])[0]) for l in want["logits"]]
    say("tokens", got_toks.tolist(), "oracle", want_toks.tolist(), "margins", [round(m, 4) for m in margins])
    np.testing.assert_array_equal(got_toks, want_toks)
    assert st.device_errors() == 0


@pytest.mark.parametrize("kv", ["bf16", "f32", "f16"])
def test_tiny_split_equals_unsplit_on_gpu(weights, kv):
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(1), 16, TINY.vocab)
    kw = dict(max_slots=1, max_ctx=64, max_tokens=16, kv=kv)
    whole = make_stage(TINY, 0, 2, True, True, weights, **kw)
    t1, tr1 = gpu_generate([whole], prompt, 8)
    a = make_stage(TINY, 0, 1, True, False, weights, **kw)
    b = make_stage(TINY, 1, 2, False, True, weights, **kw)
    t2, tr2 = gpu_generate([a, b], prompt, 8)
    np.testing.assert_array_equal(t1, t2)
    for key in ("logits", "final_hidden", "residual"):
        for u, v in zip(tr1[key], tr2[key]):
            assert u.tobytes() == v.tobytes(), key
    kw0, vw0 = kv_bits(whole, 0, 0, 23)
    kw1, vw1 = kv_bits(whole, 1, 0, 23)
    ka, va = kv_bits(a, 0, 0, 23)
    kb, vb = kv_bits(b, 1, 0, 23)
    assert np.array_equal(kw0, ka) and np.array_equal(vw0, va)
    assert np.array_equal(kw1, kb) and np.array_equal(vw1, vb)


def test_tiny_kv_matches_oracle(weights):
    x = hidden_rows(0, 16, TINY.d_model)
    ost = oracle_stage(weights, 0, 2, False, False)
    want = ost.prefill(x, 0, 0)
    st = make_stage(TINY, 0, 2, False, False, weights, max_slots=1, max_ctx=64, max_tokens=16)
    got = st.prefill(torch.from_numpy(x).cuda(), 0, 0).cpu().numpy()
    assert rel_l2(got, want) <= TOL
    kw, vw = ost.kv_bits(0, 16)
    for blk in range(2):
        kg, vg = kv_bits(st, blk, 0, 16)
        for g_bits, w_bits in ((kg, kw[blk]), (vg, vw[blk])):
            gv, wv = o.bf16_to_f32(g_bits), o.bf16_to_f32(w_bits)
            assert rel_l2_kv(gv, wv) <= TOL
            assert np.mean(g_bits == w_bits) > 0.99      # bf16 rounding flips are rare


@pytest.mark.parametrize("T", [1, 3, 4, 5, 16, 40])
def test_tiny_prefill_row_counts(weights, T):
    # T <= 4 runs the GEMV kernels, larger T the MFMA GEMM; 40 leaves a ragged GEMM tile
    x = hidden_rows(1, T, TINY.d_model)
    want = oracle_stage(weights, 0, 2, False, False).prefill(x, 0, 0)
    st = make_stage(TINY, 0, 2, False, False, weights, max_slots=1, max_ctx=64, max_tokens=64)
    got = st.prefill(torch.from_numpy(x).cuda(), 0, 0).cpu().numpy()
    assert rel_l2(got, want) <= TOL, T


def test_tiny_chunked_prefill_and_decode(weights):
    x = hidden_rows(2, 20, TINY.d_model)
    ost = oracle_stage(weights, 0, 2, False, False)
    w1 = ost.prefill(x[:8], 0, 0)
    w2 = ost.prefill(x[8:19], 0, 8)
    w3 = ost.forward(x[19:], [0], [19])
    st = make_stage(TINY, 0, 2, False, False, weights, max_slots=1, max_ctx=64, max_tokens=16)
    xt = torch.from_numpy(x).cuda()
    g1 = st.prefill(xt[:8], 0, 0).cpu().numpy()
    g2 = st.prefill(xt[8:19], 0, 8).cpu().numpy()
    dev = xt.device
    g3 = st.decode(xt[19:], torch.tensor([0], dtype=torch.int32, device=dev),
                   torch.tensor([19], dtype=torch.int32, device=dev)).cpu().numpy()
    for g, w in ((g1, w1), (g2, w2), (g3, w3)):
        assert rel_l2(g, w) <= TOL


@pytest.mark.parametrize("B,kv", [(2, "bf16"), (4, "bf16"), (6, "bf16"), (9, "bf16"), (3, "f32"), (9, "f32"),
                                  (1, "f16"), (3, "f16"), (9, "f16")])
def test_tiny_batched_decode(weights, B, kv):
    # slots prefilled to different lengths, then one decode step for all rows at once
    ost = oracle_stage(weights, 0, 2, False, False, kv_dtype=kv)
    st = make_stage(TINY, 0, 2, False, False, weights, max_slots=B, max_ctx=64, max_tokens=64, kv=kv)
    lens = [3 + 5 * b for b in range(B)]
    for b, n in enumerate(lens):
        x = hidden_rows(10 + b, n, TINY.d_model)
        ost.prefill(x, b, 0)
        st.prefill(torch.from_numpy(x).cuda(), b, 0)
    xd = np.vstack([hidden_rows(10 + b, 1, TINY.d_model, offset_pos=n) for b, n in enumerate(lens)])
    slots = np.arange(B)[::-1].copy()
    xd = xd[slots]
    pos = np.array(lens)[slots]
    want = ost.forward(xd, slots, pos)
    dev = torch.device("cuda")
    got = st.decode(torch.from_numpy(xd).to(dev), torch.tensor(slots, dtype=torch.int32, device=dev),
                    torch.tensor(pos, dtype=torch.int32, device=dev)).cpu().numpy()
    assert rel_l2(got, want) <= TOL
    assert st.device_errors() == 0


def test_tiny_determinism(weights):
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(3), 16, TINY.vocab)
    st = make_stage(TINY, 0, 2, True, True, weights, max_slots=1, max_ctx=64, max_tokens=16)
    t1, tr1 = gpu_generate([st], prompt, 6)
    t2, tr2 = gpu_generate([st], prompt, 6)       # the caller rewinds positions: "reset"
    np.testing.assert_array_equal(t1, t2)
    assert all(a.tobytes() == b.tobytes() for a, b in zip(tr1["logits"], tr2["logits"]))


@pytest.mark.parametrize("bad", ["slot", "position"])
def test_device_side_range_checks(weights, bad):
    # the documented per-row contract: an out-of-range token id embeds a zero row (one error); a
    # decode row with an out-of-range slot or position writes no K/V and gets a zero attention
    # output, so each block passes it on as x + MLP(x) (one error per block); the other rows are
    # exactly what they are in a call where every row is valid
    dev = torch.device("cuda")
    kw = dict(max_slots=2, max_ctx=64, max_tokens=4)
    st = make_stage(TINY, 0, 2, True, False, weights, **kw)
    ref = make_stage(TINY, 0, 2, True, False, weights, **kw)
    st.device_errors(reset=True)
    rows = st.embed(torch.tensor([5, TINY.vocab, -1], dtype=torch.int32, device=dev)).cpu().numpy()
    assert st.device_errors(reset=True) == 2
    assert not rows[1:].any()
    np.testing.assert_array_equal(rows[0], o.bf16_to_f32(weights[("embed", -1)][5]))
    x = hidden_rows(7, 2, TINY.d_model)
    xt = torch.from_numpy(x).to(dev)
    good = ref.decode(xt, torch.tensor([0, 1], dtype=torch.int32, device=dev),
                      torch.tensor([3, 1], dtype=torch.int32, device=dev)).cpu().numpy()
    slots, pos = ([0, 7], [3, 1]) if bad == "slot" else ([0, 1], [3, 128])   # 128: past the cache
    got = st.decode(xt, torch.tensor(slots, dtype=torch.int32, device=dev),
                    torch.tensor(pos, dtype=torch.int32, device=dev)).cpu().numpy()
    assert st.device_errors(reset=True) == 2                  # one per block
    assert ref.device_errors() == 0
    assert got[0].tobytes() == good[0].tobytes()
    ost = oracle_stage(weights, 0, 2, True, False)
    want = x[1:2]
    for b in range(2):                                        # x <- x + MLP_b(x), block by block
        want = (want + ost.mlp(b, want)).astype(np.float32)
    assert rel_l2(got[1:2], want) <= TOL
    # the bad row wrote nothing: slot 1's cache is still empty where the row would have gone
    if bad == "position":
        k, v = kv_bits(st, 0, 1, 2)
        assert not k.any() and not v.any()


@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_wide_decode_batch_splits_the_qkv_rows(kv):
    # 1024 decode rows in 1024 slots of a 2-block stage with 64 query heads of 128 (16 per KV head)
    # at d 256: the q rows alone make 8 x 32 = 256 GEMM tiles of 128 x 256, so over a 2-byte cache the
    # QKV projection runs as two GEMMs over row ranges of the fused weight (q over two activation
    # planes, K/V over three), with per-row slots and positions.  Two steps, so every row attends to
    # two keys and q matters; in the second, three rows are out of range: one error per bad row and
    # block (not one per GEMM), no K/V written for them, their outputs x + MLP(x) block by block,
    # and every other row bit-identical to a call whose rows are all valid
    B, ctx, dev = 1024, 16, torch.device("cuda")
    shape = fx.Shape(256, 64, 4, 128, 64, 1024, 2)
    w = fx.draw_stage_weights(shape, 0, 2, False, False, gain_sigma=0.1)
    say(f"{B}-row decode, 64 q / 4 KV heads of 128, {kv} cache")
    kw = dict(max_slots=B, max_ctx=ctx, max_tokens=B, kv=kv)
    st = make_stage(shape, 0, 2, False, False, w, **kw)
    ref = make_stage(shape, 0, 2, False, False, w, **kw)
    ost = o.Stage(o.Dims.of(shape), 0, 2, False, False, w, ctx, kv_dtype=kv)

    def i32(a):
        return torch.tensor(np.asarray(a), dtype=torch.int32, device=dev)

    slots = np.arange(B)
    x0, x1 = hidden_rows(11, B, shape.d_model), hidden_rows(12, B, shape.d_model)
    want0 = ost.forward(x0, slots, np.zeros(B, np.int64))
    for s_ in (st, ref):
        got0 = s_.decode(torch.from_numpy(x0).to(dev), i32(slots), i32(np.zeros(B))).cpu().numpy()
        e = rel_l2(got0, want0)
        say(f"  step 1 vs oracle: {e:.2e}")
        assert e <= TOL
    st.device_errors(reset=True)
    sl, ps = slots.copy(), np.ones(B, np.int64)
    sl[7], ps[600], sl[1023] = B, 100000, -1              # slot past the cache, position past it, negative slot
    bad = np.array([7, 600, 1023])
    ok = np.setdiff1d(slots, bad)
    got = st.decode(torch.from_numpy(x1).to(dev), i32(sl), i32(ps)).cpu().numpy()
    assert st.device_errors(reset=True) == len(bad) * 2      # per bad row and block
    good = ref.decode(torch.from_numpy(x1).to(dev), i32(slots), i32(np.ones(B))).cpu().numpy()
    assert ref.device_errors() == 0
    assert got[ok].tobytes() == good[ok].tobytes()
    want1 = ost.forward(x1[ok], slots[ok], np.ones(len(ok), np.int64))
    e = rel_l2(got[ok], want1)
    say(f"  step 2, {len(ok)} valid rows vs oracle: {e:.2e}")
    assert e <= TOL
    want_bad = x1[bad]
    for b in range(2):
        want_bad = (want_bad + ost.mlp(b, want_bad)).astype(np.float32)
    assert rel_l2(got[bad], want_bad) <= TOL
    # the K/V rows of the fused weight's second range land at the right heads and positions
    for b in range(2):
        for slot in (0, 599, 600, 1022):
            k, v = kv_bits(st, b, slot, 2)
            kc, vc = ost.kv[slot]
            n = 1 if slot == 600 else 2                        # row 600's second step wrote nothing
            assert rel_l2_kv(kv_values(kv, k[:n]), kc[b, :n]) <= TOL
            assert rel_l2_kv(kv_values(kv, v[:n]), vc[b, :n]) <= TOL
            if n == 1:
                assert not k[1].any() and not v[1].any()


@pytest.mark.parametrize("hq,hkv,dh", [(4, 4, 64), (16, 1, 128), (8, 2, 128)])
def test_gqa_group_sizes_prefill_and_decode(hq, hkv, dh):
    # query heads per KV head from 1 (every head its own K/V) to 16 (the largest group the kernels
    # take: one wave's 16 columns are one query's heads); prefill, then B = 2 decode over two slots
    d = hq * dh if hq * dh >= 256 else 256
    s = fx.Shape(d, hq, hkv, dh, 128, 512, 1)
    w = fx.draw_stage_weights(s, 0, 1, False, False, gain_sigma=0.1)
    T = 40
    ost = o.Stage(o.Dims.of(s), 0, 1, False, False, w, T + 4)
    st = make_stage(s, 0, 1, False, False, w, max_slots=2, max_ctx=64, max_tokens=64)
    dev = torch.device("cuda")
    for slot in range(2):
        x = hidden_rows(60 + slot, T - 8 * slot, d)
        want = ost.prefill(x, slot, 0)
        got = st.prefill(torch.from_numpy(x).to(dev), slot, 0).cpu().numpy()
        assert rel_l2(got, want) <= TOL, (slot, "prefill")
    for step in range(2):
        pos = np.array([T + step, T - 8 + step])
        x = np.vstack([hidden_rows(70 + b, 1, d, int(pos[b])) for b in range(2)])
        want = ost.forward(x, [0, 1], pos)
        got = st.decode(torch.from_numpy(x).to(dev), torch.tensor([0, 1], dtype=torch.int32, device=dev),
                        torch.tensor(pos, dtype=torch.int32, device=dev)).cpu().numpy()
        assert rel_l2(got, want) <= TOL, (step, "decode")
    assert st.device_errors() == 0


def test_context_end_and_ragged_capacity(weights):
    # max_ctx 77, so the cache holds 128 positions per slot: a two-chunk prefill of positions
    # 0 .. 75, a decode step at the last position 76, a prefill past max_ctx refused on the host, and
    # a decode row past the cache counted by the device and not computed
    from pipeline_stage_decoder_amd import stage as S
    max_ctx, T = 77, 60
    ost = oracle_stage(weights, 0, 2, False, False, max_ctx=max_ctx)
    st = make_stage(TINY, 0, 2, False, False, weights, max_slots=1, max_ctx=max_ctx, max_tokens=64)
    dev = torch.device("cuda")
    x = hidden_rows(5, max_ctx - 1, TINY.d_model)
    want = [ost.prefill(x[:T], 0, 0), ost.prefill(x[T:], 0, T)]
    got = [st.prefill(torch.from_numpy(x[:T]).to(dev), 0, 0).cpu().numpy(),
           st.prefill(torch.from_numpy(x[T:]).to(dev), 0, T).cpu().numpy()]
    for g, wv in zip(got, want):
        assert rel_l2(g, wv) <= TOL
    xd = hidden_rows(6, 1, TINY.d_model, max_ctx - 1)
    wd = ost.forward(xd, [0], [max_ctx - 1])
    gd = st.decode(torch.from_numpy(xd).to(dev), torch.tensor([0], dtype=torch.int32, device=dev),
                   torch.tensor([max_ctx - 1], dtype=torch.int32, device=dev)).cpu().numpy()
    assert rel_l2(gd, wd) <= TOL
    with pytest.raises(S.StageError) as e:
        st.prefill(torch.from_numpy(x[:2]).to(dev), 0, max_ctx - 1)
    assert e.value.code == S.STAGE_E_RANGE
    assert st.device_errors(reset=True) == 0
    st.decode(torch.from_numpy(xd).to(dev), torch.tensor([0], dtype=torch.int32, device=dev),
              torch.tensor([128], dtype=torch.int32, device=dev))       # past the cache: refused per row
    assert st.device_errors(reset=True) > 0


def test_empty_calls_are_refused_and_enqueue_nothing(weights):
    # a row count of zero is a non-positive size: every entry point returns STAGE_E_INVALID with
    # real buffers passed, and neither the cache nor the output buffer changes
    from pipeline_stage_decoder_amd import stage as S
    st = make_stage(TINY, 0, 2, True, True, weights, max_slots=2, max_ctx=64, max_tokens=16)
    dev = torch.device("cuda")
    x = torch.from_numpy(hidden_rows(7, 4, TINY.d_model)).to(dev)
    st.prefill(x, 0, 0)
    torch.cuda.synchronize()
    k0, v0 = kv_bits(st, 0, 0, 8)
    out = torch.full((4, TINY.d_model), 7.0, device=dev)
    logits = torch.full((4, TINY.vocab), 7.0, device=dev)
    idx = torch.zeros(4, dtype=torch.int32, device=dev)
    L, h, p = S.lib(), st._h, S._ptr
    calls = {
        "stage_embed": lambda: L.stage_embed(h, 0, p(idx), p(out), 0),
        "stage_prefill": lambda: L.stage_prefill(h, 0, 4, 0, p(x), p(out), 0),
        "stage_decode": lambda: L.stage_decode(h, 0, p(idx), p(idx), p(x), p(out), 0),
        "stage_readout": lambda: L.stage_readout(h, 0, p(x), p(logits), p(out), 0),
        "stage_mlp": lambda: L.stage_mlp(h, 0, 0, p(x), p(out), 0, 0),
        "stage_attn": lambda: L.stage_attn(h, 0, 0, 4, 0, p(x), p(out), 0, 0),
    }
    for name, call in calls.items():
        assert call() == S.STAGE_E_INVALID, name
    torch.cuda.synchronize()
    k1, v1 = kv_bits(st, 0, 0, 8)
    assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
    assert bool((out == 7.0).all()) and bool((logits == 7.0).all())
    assert st.device_errors() == 0
