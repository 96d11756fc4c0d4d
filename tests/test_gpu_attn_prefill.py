"""Prefill attention on its wide kernel: 2-byte caches (binary16, bf16) with at least 512
work-groups of 128 (query, head) columns, each wave owning 32 columns on 32 x 32 x 16 MFMAs.

The attention sublayer (stage_attn, no residual) of a seeded one-block stage is compared with the
oracle's ("41. Many GPUs", Pipeline parallelism: the block's attention half) on rows taken from
the start, the middle and the end of the sequence -- the last ones attend to every key -- with the
oracle attending over its own K/V of every row.  The shapes reach the kernel with GQA groups of 1,
4 and 16 and head dims 64 and 128; the ring-attention form ("41. Many GPUs", Ring attention for
very long contexts) runs it in partial mode, one key range per hop.  Smaller grids take the
64-column kernel, which the other attention tests cover.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from oracle import decoder as o
from pipeline_stage_decoder_amd.stage import Stage
from tests.gpu_util import hidden_rows, kv_bits, kv_values, rel_l2, rel_l2_kv, say

pytestmark = pytest.mark.gpu
TOL = 1e-3

# (Hq, Hkv, Dh, T): ceil(T * G / 128) * Hkv >= 512 work-groups in every case
CASES = [(8, 8, 64, 8192), (32, 8, 128, 2048), (128, 8, 64, 512)]


def setup(hq, hkv, dh, T, kv, seed):
    d = hq * dh
    s = fx.Shape(d, hq, hkv, dh, 64, 512, 1)
    w = {r: fx.draw_weight(s, r, 0, gain_sigma=0.1) for r in ("attn_norm", "wq", "wk", "wv", "wo")}
    st = Stage(s, 0, 1, False, False, max_slots=1, max_ctx=T, max_tokens=T, kv=kv)
    for r, t in w.items():
        st.load_weight(r, 0, t)
    torch.cuda.synchronize()
    x = hidden_rows(seed, T, d)
    c = o.Dims.of(s)
    ost = o.attn_stage(d, w["attn_norm"], w["wq"], w["wk"], w["wv"], w["wo"], dh, c.rms_eps, c.rope_theta, kv, T)
    _, k, v = ost.qkv(0, x, np.arange(T))
    ost.import_kv(0, 0, 0, k, v)                   # the oracle's own cache, every row held
    return st, ost, x


def sample_rows(T):
    return np.unique(np.concatenate([np.arange(0, 32), np.arange(T // 2 - 16, T // 2 + 16), np.arange(T - 32, T)]))


@pytest.mark.parametrize("kv", ["f16", "bf16"])
@pytest.mark.parametrize("hq,hkv,dh,T", CASES)
def test_wide_prefill_attention_matches_the_oracle(hq, hkv, dh, T, kv):
    say(f"wide prefill attention: Hq {hq}, Hkv {hkv}, Dh {dh}, T {T}, {kv} cache")
    st, ost, x = setup(hq, hkv, dh, T, kv, 80)
    got = st.attn(0, torch.from_numpy(x).cuda(), 0, 0).cpu().numpy()
    assert np.isfinite(got).all()
    rows = sample_rows(T)
    want = ost.attention(0, x[rows], np.zeros(len(rows), np.int64), rows)
    e = rel_l2(got[rows], want)
    say(f"  {len(rows)} rows vs the oracle: rel L2 (worst row) {e:.2e}")
    assert e <= TOL
    assert st.device_errors() == 0


@pytest.mark.parametrize("zigzag", [False, True])
def test_wide_prefill_attention_in_ring_mode(zigzag):
    # 4096 tokens over 2 ranks: each hop attends a 2048-row query chunk to one key range in partial
    # mode on the wide kernel (zigzag: two 1024-row chunks per rank, 256 work-groups each, on the
    # 64-column kernel); the hops' partials merged in order must give the oracle's attention
    hq, hkv, dh, T = 32, 8, 64, 4096
    say(f"ring attention over 2 ranks, zigzag {zigzag}: Hq {hq}, Hkv {hkv}, Dh {dh}, T {T}, f16 cache")
    st, ost, x = setup(hq, hkv, dh, T, "f16", 81)
    xt = torch.from_numpy(x).cuda()
    got = st.attn_ring(0, xt, 0, 2, zigzag).cpu().numpy()
    plain = st.attn(0, xt, 0, 0).cpu().numpy()
    rows = sample_rows(T)
    want = ost.attention(0, x[rows], np.zeros(len(rows), np.int64), rows)
    e, e_plain = rel_l2(got[rows], want), rel_l2(got, plain)
    say(f"  ring vs oracle {e:.2e}; ring vs the plain sublayer on the GPU {e_plain:.2e}")
    assert e <= TOL and e_plain <= TOL
    assert st.device_errors() == 0


@pytest.mark.parametrize("kv", ["f16", "bf16"])
def test_second_chunk_splits_the_qkv_rows_at_an_offset(kv):
    # one sequence through the attention sublayer in two prefill chunks: 1024 tokens at position 0
    # (their q rows make 128 GEMM tiles of 128 x 256: the fused three-plane QKV projection), then
    # 2048 at position 1024 (256 tiles: the q rows over two activation planes and the K/V rows over
    # three, as two GEMMs over row ranges of the fused weight).  The second chunk's K/V must land at
    # positions 1024..3071 and its rows attend to both chunks' keys.
    hq, hkv, dh, T1, T2 = 32, 8, 128, 1024, 2048
    say(f"two prefill chunks ({T1} at 0, {T2} at {T1}), Hq {hq}, Hkv {hkv}, Dh {dh}, {kv} cache")
    st, ost, x = setup(hq, hkv, dh, T1 + T2, kv, 82)
    xt = torch.from_numpy(x).cuda()
    st.attn(0, xt[:T1], 0, 0)
    got = st.attn(0, xt[T1:], 0, T1).cpu().numpy()
    assert np.isfinite(got).all()
    rows = sample_rows(T2)
    want = ost.attention(0, x[T1 + rows], np.zeros(len(rows), np.int64), T1 + rows)
    e = rel_l2(got[rows], want)
    say(f"  second chunk, {len(rows)} rows vs the oracle: rel L2 (worst row) {e:.2e}")
    assert e <= TOL
    k, v = kv_bits(st, 0, 0, T1 + T2)
    kc, vc = ost.kv[0]
    for name, g, w in (("K", k, kc), ("V", v, vc)):
        for lo, hi in ((0, T1), (T1, T1 + T2)):
            ek = rel_l2_kv(kv_values(kv, g[lo:hi]), w[0, lo:hi])
            say(f"  {name} positions {lo}..{hi - 1} vs the oracle's cache: {ek:.2e}")
            assert ek <= TOL
    assert st.device_errors() == 0
