"""GPU parity at the workloads' real shapes (relative L2 <= 1e-3 against the float64 oracle).

The oracle cannot run a whole 16- or 20-block stage at these widths in seconds, so each case runs
the stage's kernels at their real shapes on a slice the oracle can follow:
* 8B-shaped first stage: embedding + blocks 0..1 at d 4096, prefill T = 512 (the benchmark's
  launch shapes) and a ragged T = 72, then B = 1 decode steps (the benchmark's decode kernels);
* 8B-shaped last stage: block 16 + final norm + readout, B = 64 decode at context 4096 over a
  seeded KV cache imported into both sides;
* 70B-shaped middle stage: block 20 at d 8192, T = 64 prefill, then B = 128 decode at context
  8192 over a seeded KV cache; and a 4096-token chunk (the large-grid GEMM schedule for every
  projection), its first 64 rows and their KV against the oracle's 64-token prefill;
* sharded MLP: 8 column/row slices of a d 8192 / F 28672 MLP summed in slice order against the full
  MLP at T in {1, 64, 4096} (the T = 4096 oracle check on 64 sampled rows; MLP rows are
  independent);
* 8B blocks [0, 2) against [0, 1) + [1, 2): bit-identical hidden rows and KV after a 300-row
  prefill, two B = 1 decode steps and a B = 64 decode step, bf16 and F32 caches;
* 8B MLP at T in {40, 100, 257, 300, 512, 2600}: every GEMM tiling with a ragged last row tile,
  the oracle on sampled rows and the tail rows;
* an irregular shape off the benchmark grid (d 2560, 20 q / 4 KV heads, SwiGLU 6912): a 160-row
  prefill and B = 3 and B = 70 decode steps over fresh and continuing slots.
Inputs: seeded bf16 N(0, 0.02) weights with norm gains 1 + N(0, 0.1^2), uniform tokens, F32 N(0,1)
hidden rows, bf16 N(0,1) cached K/V.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from oracle import decoder as o
from pipeline_stage_decoder_amd.stage import Stage
from tests.gpu_util import (hidden_rows, kv_bits, kv_bits_of, kv_values, make_stage, rel_l2, rel_l2_kv, rel_l2_rows,
                            rel_l2_whole, say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

TOL = 1e-3
SEED_KV = 0x5EED0004


def seeded_kv(shape, slot: int, n: int, kv: str = "bf16"):
    """Seeded N(0,1) K and V [n, Hkv, Dh] of one slot (K stands for post-RoPE keys) as values of
    the cache format kv (bf16 draws, rounded to binary16 for an F16 cache)."""
    per = shape.n_kv_heads * shape.head_dim
    k = fx.normal_bf16(SEED_KV, 2 * slot, n * per, 1.0).reshape(n, shape.n_kv_heads, shape.head_dim)
    v = fx.normal_bf16(SEED_KV, 2 * slot + 1, n * per, 1.0).reshape(n, shape.n_kv_heads, shape.head_dim)
    k, v = o.bf16_to_f32(k), o.bf16_to_f32(v)
    if kv == "f16":
        k, v = k.astype(np.float16).astype(np.float32), v.astype(np.float16).astype(np.float32)
    return k, v


def import_kv(st, ost, block, slots, n):
    """Write the same seeded KV (positions 0..n-1) into the GPU stage and the oracle stage."""
    dt = torch.float32 if st.kv == "f32" else torch.int16
    for s in slots:
        k, v = seeded_kv(st.shape, s, n, st.kv)
        kb, vb = kv_bits_of(st.kv, k), kv_bits_of(st.kv, v)
        st.kv_import(block, s, 0, torch.from_numpy(kb).view(dt).cuda(), torch.from_numpy(vb).view(dt).cuda())
        ost.import_kv(block, s, 0, k, v)
    torch.cuda.synchronize()


@pytest.fixture(scope="module")
def w8b_first():
    return fx.draw_stage_weights(fx.LLAMA8B, 0, 2, True, False, gain_sigma=0.1)


@pytest.mark.parametrize("T,kv", [(72, "bf16"), (512, "f32"), (72, "f32"), (512, "f16"), (72, "f16")])
def test_8b_first_stage_prefill_and_decode(w8b_first, T, kv):
    # with an F32 cache the QKV projection takes two activation planes instead of three
    s = fx.LLAMA8B
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(0), T, s.vocab)
    say(f"8B first stage: oracle prefill T={T}, {kv} cache")
    ost = o.Stage(o.Dims.of(s), 0, 2, True, False, w8b_first, T + 4, kv_dtype=kv)
    want = ost.prefill(ost.embed(prompt), 0, 0)
    st = make_stage(s, 0, 2, True, False, w8b_first, max_slots=1, max_ctx=2048, max_tokens=512, kv=kv)
    dev = torch.device("cuda")
    x = st.embed(torch.tensor(prompt, dtype=torch.int32, device=dev))
    got = st.prefill(x, 0, 0).cpu().numpy()
    e = rel_l2(got, want)
    say(f"  prefill rel L2 {e:.2e}")
    assert e <= TOL
    toks = fx.tokens(fx.SEED_TOKENS, fx.token_stream(1), 2, s.vocab)
    for i, tok in enumerate(toks):
        w = ost.forward(ost.embed(np.array([tok])), [0], [T + i])
        xg = st.embed(torch.tensor([tok], dtype=torch.int32, device=dev))
        g = st.decode(xg, torch.tensor([0], dtype=torch.int32, device=dev),
                      torch.tensor([T + i], dtype=torch.int32, device=dev)).cpu().numpy()
        e = rel_l2(g, w)
        say(f"  decode step {i} rel L2 {e:.2e}")
        assert e <= TOL


def test_8b_bf16_cache_outside_the_row_bound(w8b_first):
    # bf16 KV storage is offered but is not inside the parity envelope.  A K/V value that the GPU's
    # f32 sums and the float64 oracle put on different sides of a bf16 rounding boundary is stored
    # 2^-8 apart, and over a 512-token prompt of the 8B-shaped first stage (two blocks) that moves
    # single rows past 1e-3 (measured 1.18e-3 on MI355X) although the whole tensor stays well below
    # it; the F16 and F32-grade caches hold the row bound at full depth.  What this checks of the
    # bf16 format itself: the rounding (bits equal to the oracle's bf16 rounding for > 99% of the
    # cached values of the first block), the whole-tensor bound, and a worst row under 2e-3 as a
    # regression guard.
    s, T = fx.LLAMA8B, 512
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(0), T, s.vocab)
    ost = o.Stage(o.Dims.of(s), 0, 2, True, False, w8b_first, T, kv_dtype="bf16")
    want = ost.prefill(ost.embed(prompt), 0, 0)
    st = make_stage(s, 0, 2, True, False, w8b_first, max_slots=1, max_ctx=T, max_tokens=T, kv="bf16")
    got = st.prefill(st.embed(torch.tensor(prompt, dtype=torch.int32, device="cuda")), 0, 0).cpu().numpy()
    e_whole, e_row = rel_l2_whole(got, want), rel_l2_rows(got, want)
    say(f"8B first stage, bf16 cache, T={T}: whole {e_whole:.2e}, worst row {e_row:.2e}")
    assert e_whole <= TOL and e_row <= 2e-3
    # block 0's K/V come from exact inputs (embedding rows), so they show the rounding itself;
    # block 1's inputs already carry block 0's differences
    kg, vg = kv_bits(st, 0, 0, T)
    kc, vc = ost.kv[0]
    for g_bits, w_vals in ((kg, kc[0, :T]), (vg, vc[0, :T])):
        assert np.mean(g_bits == kv_bits_of("bf16", w_vals)) > 0.99


@pytest.mark.parametrize("kv", ["bf16", "f16"])
def test_8b_last_stage_batched_decode_and_readout(kv):
    s, blk, B, ctx = fx.LLAMA8B, 16, 64, 4096
    w = fx.draw_stage_weights(s, blk, blk + 1, False, True, gain_sigma=0.1)
    ost = o.Stage(o.Dims.of(s), blk, blk + 1, False, True, w, ctx + 1, kv_dtype=kv)
    st = make_stage(s, blk, blk + 1, False, True, w, max_slots=B, max_ctx=ctx + 1, max_tokens=B, kv=kv)
    say("8B last stage: importing KV")
    import_kv(st, ost, blk, range(B), ctx)
    slots = np.arange(B)[::-1].copy()
    x = np.vstack([hidden_rows(100 + int(b), 1, s.d_model, offset_pos=ctx) for b in slots])
    pos = np.full(B, ctx)
    say("8B last stage: oracle")
    want = ost.forward(x, slots, pos)
    want_logits, want_hn = ost.readout(want)
    dev = torch.device("cuda")
    got = st.decode(torch.from_numpy(x).to(dev), torch.tensor(slots, dtype=torch.int32, device=dev),
                    torch.tensor(pos, dtype=torch.int32, device=dev))
    logits, hn = st.readout(got)
    for name, g, wv in (("hidden", got.cpu().numpy(), want), ("final hidden", hn.cpu().numpy(), want_hn),
                        ("logits", logits.cpu().numpy(), want_logits)):
        e = rel_l2(g, wv)
        say(f"  {name} rel L2 {e:.2e}")
        assert e <= TOL, name
    assert st.device_errors() == 0


@pytest.fixture(scope="module")
def w70b_block():
    return fx.draw_stage_weights(fx.LLAMA70B, 20, 21, False, False, gain_sigma=0.1)


@pytest.mark.parametrize("kv", ["bf16", "f16"])
def test_70b_mid_stage_prefill_and_batched_decode(w70b_block, kv):
    s, blk, B, ctx = fx.LLAMA70B, 20, 128, 8192
    w = w70b_block
    st = make_stage(s, blk, blk + 1, False, False, w, max_slots=B + 1, max_ctx=ctx + 1, max_tokens=B, kv=kv)
    # prefill T = 64 into the extra slot B
    ost = o.Stage(o.Dims.of(s), blk, blk + 1, False, False, w, ctx + 1, kv_dtype=kv)
    xp = hidden_rows(7, 64, s.d_model)
    say("70B block: oracle prefill")
    want = ost.prefill(xp, B, 0)
    got = st.prefill(torch.from_numpy(xp).cuda(), B, 0).cpu().numpy()
    e = rel_l2(got, want)
    say(f"  prefill rel L2 {e:.2e}")
    assert e <= TOL
    say("70B block: importing KV")
    import_kv(st, ost, blk, range(B), ctx)
    slots = np.arange(B)
    x = np.vstack([hidden_rows(300 + b, 1, s.d_model, offset_pos=ctx) for b in slots])
    pos = np.full(B, ctx)
    say("70B block: oracle decode")
    want = ost.forward(x, slots, pos)
    dev = torch.device("cuda")
    got = st.decode(torch.from_numpy(x).to(dev), torch.tensor(slots, dtype=torch.int32, device=dev),
                    torch.tensor(pos, dtype=torch.int32, device=dev)).cpu().numpy()
    e = rel_l2(got, want)
    say(f"  decode B=128 rel L2 {e:.2e}")
    assert e <= TOL
    assert st.device_errors() == 0


@pytest.mark.parametrize("kv", ["bf16", "f32", "f16"])
def test_70b_prefill_chunk_4096_all_kv_rows_and_late_rows(w70b_block, kv):
    # a 4096-token chunk runs every projection of the block on the large-grid GEMM schedule (QKV +
    # RoPE + KV write, O + residual, gate/up + SwiGLU, down + residual).  Every row's K and V
    # depend only on that row's input, so the oracle's K/V of all 4096 rows are compared with the
    # exported cache, per KV head; then the oracle's attention (over its own K/V of every earlier
    # row), O projection and MLP give the exact outputs of rows spread over the chunk -- the first
    # GEMM row tile, middle tiles and the last 64 rows, which attend to up to 4096 keys.
    s, blk, T = fx.LLAMA70B, 20, 4096
    st = make_stage(s, blk, blk + 1, False, False, w70b_block, max_slots=1, max_ctx=T, max_tokens=T, kv=kv)
    x = hidden_rows(9, T, s.d_model)
    say(f"70B block, {kv} cache: gpu prefill T={T}")
    got = st.prefill(torch.from_numpy(x).cuda(), 0, 0).cpu().numpy()
    assert np.isfinite(got).all()
    kg, vg = kv_bits(st, blk, 0, T)
    say("  oracle K/V of all rows")
    ost = o.Stage(o.Dims.of(s), blk, blk + 1, False, False, w70b_block, T, kv_dtype=kv)
    pos = np.arange(T)
    _, k_all, v_all = ost.qkv(blk, x, pos)
    for name, g_bits, want_kv in (("K", kg, k_all), ("V", vg, v_all)):
        e = rel_l2_kv(kv_values(kv, g_bits), want_kv)
        say(f"  {name} of rows 0..{T - 1}: rel L2 (worst head) {e:.2e}")
        assert e <= TOL
        if kv != "f32":                            # rounding flips are rare
            assert np.mean(g_bits == kv_bits_of(kv, want_kv)) > 0.99
    ost.import_kv(blk, 0, 0, k_all, v_all)        # the oracle's own cache, every row held
    rows = np.concatenate([np.arange(0, 64), np.arange(1000, 1032), np.arange(2500, 2532), np.arange(T - 64, T)])
    say(f"  oracle block output of {len(rows)} rows")
    want = ost.forward(x[rows], np.zeros(len(rows), np.int64), rows)
    e = rel_l2(got[rows], want)
    say(f"  rows 0..63, 1000..1031, 2500..2531, {T - 64}..{T - 1}: rel L2 (worst row) {e:.2e}")
    assert e <= TOL
    assert st.device_errors() == 0


@pytest.fixture(scope="module")
def mlp70b():
    s = fx.LLAMA70B
    g = fx.draw_weight(s, "mlp_norm", 0, gain_sigma=0.1)
    wg = fx.draw_weight(s, "wgate", 0)
    wu = fx.draw_weight(s, "wup", 0)
    wd = fx.draw_weight(s, "wdown", 0)
    return g, wg, wu, wd


def slice_stage(mlp, n_slices):
    """A stage whose n blocks hold the MLP slices (block i = rows/columns [i w, (i+1) w))."""
    g, wg, wu, wd = mlp
    s = fx.LLAMA70B
    width = s.d_ffn // n_slices
    sh = fx.Shape(s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, width, s.vocab, n_slices)
    st = make_stage(sh, 0, n_slices, False, False, {}, max_slots=1, max_ctx=64, max_tokens=4096)
    for i in range(n_slices):
        lo, hi = i * width, (i + 1) * width
        st.load_weight("mlp_norm", i, g)
        st.load_weight("wgate", i, np.ascontiguousarray(wg[lo:hi]))
        st.load_weight("wup", i, np.ascontiguousarray(wu[lo:hi]))
        st.load_weight("wdown", i, np.ascontiguousarray(wd[:, lo:hi]))
    torch.cuda.synchronize()
    return st


@pytest.mark.parametrize("T", [1, 64, 4096])
def test_mlp_slices_sum_to_full_mlp(mlp70b, T):
    g, wg, wu, wd = mlp70b
    s = fx.LLAMA70B
    x = hidden_rows(40, T, s.d_model)
    xt = torch.from_numpy(x).cuda()
    sl = slice_stage(mlp70b, 8)
    acc = torch.empty_like(xt)
    for i in range(8):                                   # ((p0 + p1) + p2) + ... in slice order
        sl.mlp(i, xt, out=acc, accumulate=i > 0)
    full = make_stage(s, 0, 1, False, False, {("mlp_norm", 0): g, ("wgate", 0): wg, ("wup", 0): wu,
                                              ("wdown", 0): wd}, max_slots=1, max_ctx=64, max_tokens=4096)
    y_full = full.mlp(0, xt).cpu().numpy()
    y_sum = acc.cpu().numpy()
    # on the GPU the slice sum differs from the full MLP only by F32 reassociation
    e_gpu = rel_l2(y_sum, y_full)
    rows = np.arange(T) if T <= 64 else np.linspace(0, T - 1, 64).astype(int)
    say(f"MLP slices T={T}: oracle on {len(rows)} rows")
    _, _, want_sum = o.mlp_slices(x[rows], g, wg, wu, wd, s.rms_eps, 8)
    _, want_full = o.mlp_full(x[rows], g, wg, wu, wd, s.rms_eps)
    e_sum = rel_l2(y_sum[rows], want_sum)
    e_full = rel_l2(y_full[rows], want_full)
    say(f"  slices vs full (gpu) {e_gpu:.2e}; slices vs oracle {e_sum:.2e}; full vs oracle {e_full:.2e}")
    assert e_gpu <= 1e-5
    assert e_sum <= TOL and e_full <= TOL


@pytest.mark.parametrize("kv", ["bf16", "f32", "f16"])
def test_8b_split_equals_unsplit_on_gpu(w8b_first, kv):
    # blocks [0, 2) in one stage against [0, 1) + [1, 2) with the F32 handoff, at the real 8B shape:
    # a 300-row prefill (LDS-direct GEMMs, split-K sums; in one stage block 0's down projection
    # also normalises for block 1, in two stages block 1 normalises its input itself), two B = 1
    # decode steps (GEMVs, split-KV attention), then one B = 64 decode step over 64 slots holding
    # copies of that context (64-row GEMM tiles, split-K sums fused with the next norm); hidden rows
    # and both blocks' KV bit for bit
    s, T, B = fx.LLAMA8B, 300, 64
    dev = torch.device("cuda")
    kw = dict(max_slots=B, max_ctx=512, max_tokens=512, kv=kv)
    whole = make_stage(s, 0, 2, True, False, w8b_first, **kw)
    a = make_stage(s, 0, 1, True, False, w8b_first, **kw)
    b = make_stage(s, 1, 2, False, False, w8b_first, **kw)
    prompt = torch.tensor(fx.tokens(fx.SEED_TOKENS, fx.token_stream(2), T, s.vocab), dtype=torch.int32, device=dev)
    y1 = whole.prefill(whole.embed(prompt), 0, 0)
    y2 = b.prefill(a.prefill(a.embed(prompt), 0, 0), 0, 0)
    assert torch.equal(y1, y2)
    toks = fx.tokens(fx.SEED_TOKENS, fx.token_stream(3), 2, s.vocab)
    for i, tok in enumerate(toks):
        t = torch.tensor([tok], dtype=torch.int32, device=dev)
        sl, ps = torch.tensor([0], dtype=torch.int32, device=dev), torch.tensor([T + i], dtype=torch.int32, device=dev)
        d1 = whole.decode(whole.embed(t), sl, ps)
        d2 = b.decode(a.decode(a.embed(t), sl, ps), sl, ps)
        assert torch.equal(d1, d2)
    n = T + len(toks)
    for st in (whole, a, b):
        for slot in range(1, B):
            st.kv_copy(0, slot, n)
    tb = torch.tensor(fx.tokens(fx.SEED_TOKENS, fx.token_stream(4), B, s.vocab), dtype=torch.int32, device=dev)
    sl = torch.arange(B, dtype=torch.int32, device=dev)
    ps = torch.full((B,), n, dtype=torch.int32, device=dev)
    d1 = whole.decode(whole.embed(tb), sl, ps)
    d2 = b.decode(a.decode(a.embed(tb), sl, ps), sl, ps)
    assert torch.equal(d1, d2)
    assert whole.device_errors() == 0 and a.device_errors() == 0 and b.device_errors() == 0
    for blk, part in ((0, a), (1, b)):
        for slot in (0, 1, B - 1):
            kw_, vw_ = kv_bits(whole, blk, slot, n + 1)
            kp, vp = kv_bits(part, blk, slot, n + 1)
            assert np.array_equal(kw_, kp) and np.array_equal(vw_, vp)
    say(f"8B split [0,1)+[1,2) == [0,2), {kv} cache: prefill {T} rows, 2 decode steps, "
        f"B={B} decode step, KV")


@pytest.mark.parametrize("T", [40, 100, 257, 300, 512, 2600])
def test_8b_mlp_gemm_tiles_ragged_rows(w8b_first, T):
    # each row count takes another GEMM plan: 40 the 64 x 128 LDS-direct tiles (M <= 64), 100 one
    # row of 128 x 256 tiles (64 < M <= 128, non-temporal weight loads), 257 / 300 / 512 / 2600 the
    # 128 x 256 tiles with three weight buffers -- gate/up unsplit, down split along K into 4 at
    # 257 / 300 / 512 rows and unsplit at 2600; the last row tile is ragged in every case (clamped
    # reads that must never be stored).  MLP rows are independent: the oracle checks the first rows, a spread,
    # and the tail rows.
    s = fx.LLAMA8B
    w = {(r, 0): w8b_first[(r, 0)] for r in ("mlp_norm", "wgate", "wup", "wdown")}
    st = make_stage(s, 0, 1, False, False, w, max_slots=1, max_ctx=64, max_tokens=max(T, 512))
    x = hidden_rows(41, T, s.d_model)
    got = st.mlp(0, torch.from_numpy(x).cuda()).cpu().numpy()
    tail = np.arange(max(0, T - 24), T)
    rows = np.unique(np.concatenate([np.arange(4), np.linspace(0, T - 1, 16).astype(int), tail]))
    say(f"8B MLP T={T}: oracle on {len(rows)} rows")
    _, want = o.mlp_full(x[rows], w[("mlp_norm", 0)], w[("wgate", 0)], w[("wup", 0)], w[("wdown", 0)], s.rms_eps)
    e = rel_l2(got[rows], want)
    say(f"  rel L2 {e:.2e}")
    assert e <= TOL
    assert np.isfinite(got).all()


def oracle_layer_major(shape, begin, end, kv, x_rows, draw_block):
    """Oracle output of blocks [begin, end) for one sequence whose rows x_rows sit at positions
    0, 1, ...: a prefill of the first rows followed by decode steps of the rest gives, row for row,
    the values of one prefill of every row (each row attends the keys at or before its position,
    and every row's K/V is written first), so the oracle runs block by block over all rows at once
    and holds one block's weights at a time (draw_block(b) -> that block's weights)."""
    c = o.Dims.of(shape)
    x = np.asarray(x_rows, np.float32)
    for b in range(begin, end):
        st = o.Stage(c, b, b + 1, False, False, draw_block(b), x.shape[0], kv_dtype=kv)
        x = st.prefill(x, 0, 0)
        say(f"    oracle block {b} done")
    return x


def fill_weights_on_gpu(st, shape, blocks, first, last, gain_sigma):
    """Draw a stage's weights with the device generator (bit-identical to the host draws of
    fixtures.draw_weight) and load them; no host copy of the whole stage."""
    roles = fx.stage_roles(blocks[0], blocks[1], first, last)
    biggest = max(int(np.prod(fx.role_shape(shape, r))) for r, _ in roles)
    scratch = torch.empty(biggest, dtype=torch.int16, device="cuda")
    for role, b in roles:
        t = scratch[:int(np.prod(fx.role_shape(shape, role)))]
        if role in fx.GAIN_ROLES:
            fx.gain_bf16_gpu(t, fx.SEED_WEIGHTS, fx.weight_stream(role, b), gain_sigma)
        else:
            fx.normal_bf16_gpu(t, fx.SEED_WEIGHTS, fx.weight_stream(role, b), 0.02)
        st.load_weight(role, b, t)
    torch.cuda.synchronize()


@pytest.mark.parametrize("kv", ["f32", "f16"])
def test_8b_first_stage_all_16_blocks_decode_kernels(kv):
    # the whole first stage (embedding + 16 blocks) with a short prompt, then B = 1 decode steps:
    # the decode launches are the benchmark's (GEMV kernels, split-KV attention over max_ctx 2048).
    # F32-grade and binary16 caches hold 1e-3 at this depth; bf16 storage does not (its rounding
    # flips cascade through the blocks) and is covered block by block above.
    s = fx.LLAMA8B
    T, n_dec = 24, 2
    prompt = fx.tokens(fx.SEED_TOKENS, fx.token_stream(2), T, s.vocab)
    toks = fx.tokens(fx.SEED_TOKENS, fx.token_stream(3), n_dec, s.vocab)
    emb = fx.draw_weight(s, "embed")
    x_rows = o.bf16_to_f32(emb[np.concatenate([prompt, toks])])
    say(f"8B first stage, 16 blocks, {kv} cache: oracle")
    want = oracle_layer_major(s, 0, 16, kv, x_rows,
                              lambda b: {(r, b): fx.draw_weight(s, r, b, gain_sigma=0.1) for r in fx.BLOCK_ROLES})
    st = Stage(s, 0, 16, True, False, max_slots=1, max_ctx=2048, max_tokens=512, kv=kv)
    fill_weights_on_gpu(st, s, (0, 16), True, False, 0.1)
    dev = torch.device("cuda")
    got = [st.prefill(st.embed(torch.tensor(prompt, dtype=torch.int32, device=dev)), 0, 0).cpu().numpy()]
    for i, tok in enumerate(toks):
        xg = st.embed(torch.tensor([tok], dtype=torch.int32, device=dev))
        got.append(st.decode(xg, torch.tensor([0], dtype=torch.int32, device=dev),
                             torch.tensor([T + i], dtype=torch.int32, device=dev)).cpu().numpy())
    wants = [want[:T]] + [want[T + i:T + i + 1] for i in range(n_dec)]
    for i, (g, wv) in enumerate(zip(got, wants)):
        e = rel_l2(g, wv)
        say(f"  step {i} rel L2 (worst row) {e:.2e}")
        assert e <= TOL
    assert st.device_errors() == 0


def test_70b_stage_all_20_blocks_f16_cache():
    # the 70B-shaped middle stage at full depth (blocks 20..39, d 8192, 64 q / 8 KV heads, SwiGLU
    # 28672) on the binary16 cache its benchmark runs: a 16-row prefill (GEMM path) and two B = 1
    # decode steps (GEMV path), against the oracle through all 20 blocks
    s = fx.LLAMA70B
    T, n_dec, kv = 16, 2, "f16"
    x_rows = hidden_rows(11, T + n_dec, s.d_model)
    say("70B-shaped stage, 20 blocks, f16 cache: oracle")
    want = oracle_layer_major(s, 20, 40, kv, x_rows,
                              lambda b: {(r, b): fx.draw_weight(s, r, b, gain_sigma=0.1) for r in fx.BLOCK_ROLES})
    st = Stage(s, 20, 40, False, False, max_slots=1, max_ctx=64, max_tokens=64, kv=kv)
    fill_weights_on_gpu(st, s, (20, 40), False, False, 0.1)
    dev = torch.device("cuda")
    got = [st.prefill(torch.from_numpy(x_rows[:T]).to(dev), 0, 0).cpu().numpy()]
    for i in range(n_dec):
        got.append(st.decode(torch.from_numpy(x_rows[T + i:T + i + 1]).to(dev),
                             torch.tensor([0], dtype=torch.int32, device=dev),
                             torch.tensor([T + i], dtype=torch.int32, device=dev)).cpu().numpy())
    wants = [want[:T]] + [want[T + i:T + i + 1] for i in range(n_dec)]
    for i, (g, wv) in enumerate(zip(got, wants)):
        e = rel_l2(g, wv)
        say(f"  step {i} rel L2 (worst row) {e:.2e}")
        assert e <= TOL
    assert st.device_errors() == 0


IRREG = fx.Shape(2560, 20, 4, 128, 6912, 1024, 2)


@pytest.mark.parametrize("kv", ["f16", "f32"])
def test_irregular_shape_prefill_and_decode(kv):
    # a model off the benchmark grid: d 2560 and SwiGLU 6912 (neither a multiple of 2048, so the
    # B <= 4 decode takes the general GEMV, and the down projection, too wide for its input
    # staging, the skinny MFMA tiles), 20 query heads over 4 KV heads (groups of 5), a QKV width of
    # 3584 and 54 gate/up tiles of 256.  A 160-row prefill of slot 0 (the register-staged GEMMs
    # with a ragged second row tile, the 64-column attention kernel), then a B = 3 decode step
    # (slot 0 continuing, slots 1 and 2 starting) and a B = 70 step (70 slots at mixed positions).
    s, T, ctx = IRREG, 160, 256
    w = fx.draw_stage_weights(s, 0, 2, False, False, gain_sigma=0.1)
    say(f"irregular shape (d 2560, 20q/4kv, F 6912), {kv} cache: prefill {T}")
    st = make_stage(s, 0, 2, False, False, w, max_slots=70, max_ctx=ctx, max_tokens=T, kv=kv)
    ost = o.Stage(o.Dims.of(s), 0, 2, False, False, w, ctx, kv_dtype=kv)
    dev = torch.device("cuda")
    x = hidden_rows(51, T, s.d_model)
    got = st.prefill(torch.from_numpy(x).to(dev), 0, 0).cpu().numpy()
    want = ost.prefill(x, 0, 0)
    e = rel_l2(got, want)
    say(f"  prefill vs oracle: {e:.2e}")
    assert e <= TOL
    steps = [(np.array([0, 1, 2]), np.array([T, 0, 0])),
             (np.arange(70), np.concatenate([[T + 1, 1, 1], np.zeros(67, np.int64)]))]
    for i, (slots, pos) in enumerate(steps):
        xd = hidden_rows(52 + i, len(slots), s.d_model)
        got = st.decode(torch.from_numpy(xd).to(dev), torch.tensor(slots, dtype=torch.int32, device=dev),
                        torch.tensor(pos, dtype=torch.int32, device=dev)).cpu().numpy()
        want = ost.forward(xd, slots, pos)
        e = rel_l2(got, want)
        say(f"  B = {len(slots)} decode vs oracle: {e:.2e}")
        assert e <= TOL
    for b in range(2):
        k, v = kv_bits(st, b, 0, T + 2)
        kc, vc = ost.kv[0]
        assert rel_l2_kv(kv_values(kv, k), kc[b, :T + 2]) <= TOL
        assert rel_l2_kv(kv_values(kv, v), vc[b, :T + 2]) <= TOL
    assert st.device_errors() == 0
