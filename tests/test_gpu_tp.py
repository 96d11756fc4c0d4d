"""GPU checks of the tensor-parallel slices on one GPU ("41. Many GPUs", Tensor parallelism).

* Attention by heads: slice stages hold their query heads' rows of W_q, their KV heads' rows of
  W_k / W_v (replicated when there are fewer KV heads than slices) and the matching columns of
  W_o; stage_attn over the slices in order (accumulate) must match the oracle's slice sum and full
  sublayer (rel L2 <= 1e-3).  With an F32 cache the slice sum must also equal the GPU's full
  sublayer up to F32 reassociation (rel L2 <= 1e-5).  With a bf16 cache it need not: the slice and
  full projections sum in different orders, so a few K/V values round to neighbouring bf16 values
  (measured up to 2.7e-4 on one 8B slice), the cache-rounding effect the oracle bound covers; the
  same holds for a binary16 cache.
  The sublayer itself plus stage_mlp reproduces stage_prefill's block bit for bit.
* Vocabulary: slices of the embedding (zero-padded to a multiple of the slice count) summed by
  stage_embed_range reproduce the full embedding bit for bit; readout slices concatenated and cut
  to V reproduce the full logits (bit for bit on the GEMV path, within F32 reassociation on the
  GEMM path) and the oracle.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from oracle import decoder as o
from pipeline_stage_decoder_amd.stage import Stage
from tests.gpu_util import hidden_rows, make_stage, rel_l2, say

pytestmark = pytest.mark.gpu


def slice_shape(s, hq, hk, vocab=None, n_blocks=1):
    """The per-slice shape; the MLP width is irrelevant to these checks and kept small."""
    return fx.Shape(s.d_model, hq, hk, s.head_dim, 64, vocab or s.vocab, n_blocks)


def attn_weights(s, block=0):
    w = {r: fx.draw_weight(s, r, block, gain_sigma=0.1) for r in ("attn_norm", "wq", "wk", "wv", "wo")}
    return w


@pytest.mark.parametrize("kv", ["bf16", "f32", "f16"])
@pytest.mark.parametrize("name,n,T", [("tiny", 2, 24), ("tiny", 4, 24), ("8b", 8, 64), ("8b", 16, 20)])
def test_attention_head_slices_sum_to_full(name, n, T, kv):
    s = fx.TINY if name == "tiny" else fx.LLAMA8B
    w = attn_weights(s)
    dh = s.head_dim
    x = hidden_rows(50, T, s.d_model)
    xt = torch.from_numpy(x).cuda()
    sl = o.head_shards(s.n_q_heads, s.n_kv_heads, n)
    hq, hk = sl[0][1], sl[0][3]
    st = Stage(slice_shape(s, hq, hk, n_blocks=n), 0, n, False, False, max_slots=1, max_ctx=64, max_tokens=64,
               kv=kv)
    for i, (q0, _, kv0, _) in enumerate(sl):
        qr, kr = slice(q0 * dh, (q0 + hq) * dh), slice(kv0 * dh, (kv0 + hk) * dh)
        st.load_weight("attn_norm", i, w["attn_norm"])
        st.load_weight("wq", i, np.ascontiguousarray(w["wq"][qr]))
        st.load_weight("wk", i, np.ascontiguousarray(w["wk"][kr]))
        st.load_weight("wv", i, np.ascontiguousarray(w["wv"][kr]))
        st.load_weight("wo", i, np.ascontiguousarray(w["wo"][:, qr]))
    acc = torch.empty_like(xt)
    for i in range(n):                                   # ((p0 + p1) + p2) + ... in slice order
        st.attn(i, xt, 0, 0, out=acc, accumulate=i > 0)
    full_st = Stage(slice_shape(s, s.n_q_heads, s.n_kv_heads), 0, 1, False, False, max_slots=1, max_ctx=64,
                    max_tokens=64, kv=kv)
    for r, t in w.items():
        full_st.load_weight(r, 0, t)
    full = full_st.attn(0, xt, 0, 0).cpu().numpy()
    got = acc.cpu().numpy()
    c = o.Dims.of(s)
    kvd = kv
    want = o.attn_sublayer(x, w["attn_norm"], w["wq"], w["wk"], w["wv"], w["wo"], dh, c.rms_eps, c.rope_theta, kvd)
    _, want_sum = o.attn_slices(x, w["attn_norm"], w["wq"], w["wk"], w["wv"], w["wo"], dh, c.rms_eps,
                                c.rope_theta, n, kvd)
    e_gpu, e_full, e_sum = rel_l2(got, full), rel_l2(full, want), rel_l2(got, want_sum)
    say(f"{name} attention over {n} head slices, T={T}, {kvd} cache: slices vs full (gpu) {e_gpu:.2e}; "
        f"full vs oracle {e_full:.2e}; slices vs oracle {e_sum:.2e}")
    assert e_full <= 1e-3 and e_sum <= 1e-3
    if kv == "f32":
        assert e_gpu <= 1e-5


def test_attention_and_mlp_halves_reproduce_the_block():
    s = fx.TINY
    w = fx.draw_stage_weights(s, 0, 1, False, False, gain_sigma=0.1)
    st = make_stage(s, 0, 1, False, False, w, max_slots=2, max_ctx=64, max_tokens=32)
    x = torch.from_numpy(hidden_rows(51, 20, s.d_model)).cuda()
    y = st.prefill(x, 0, 0)
    h = x.clone()
    st.attn(0, x, 1, 0, out=h, accumulate=True)         # x1 = x + attention(x), slot 1
    st.mlp(0, h, out=h, accumulate=True)                # x1 + MLP(x1)
    assert torch.equal(h, y)
    assert torch.equal(st.kv_export(0, 0, 0, 20)[0], st.kv_export(0, 1, 0, 20)[0])


@pytest.mark.parametrize("name,n", [("tiny", 3), ("tiny", 8), ("8b", 8)])
def test_vocab_slices_embedding_and_readout(name, n):
    s = fx.TINY if name == "tiny" else fx.LLAMA8B
    V, d = s.vocab, s.d_model
    emb = fx.draw_weight(s, "embed")
    ro = fx.draw_weight(s, "readout")
    g = fx.draw_weight(s, "final_norm", gain_sigma=0.1)
    per, firsts = o.vocab_shards(V, n)
    toks = np.concatenate([fx.tokens(fx.SEED_TOKENS, fx.token_stream(40), 13, V),
                           [0, V - 1, per - 1, per, min(2 * per, V - 1)]]).astype(np.int32)
    tt = torch.from_numpy(toks).cuda()
    full = Stage(slice_shape(s, s.n_q_heads, s.n_kv_heads, n_blocks=1), 0, 0, True, True, max_slots=1,
                 max_ctx=64, max_tokens=32)
    full.load_weight("embed", -1, emb)
    full.load_weight("readout", -1, ro)
    full.load_weight("final_norm", -1, g)
    want_rows = full.embed(tt)
    acc = torch.empty_like(want_rows)
    slices = []
    for i in range(n):
        sh = slice_shape(s, s.n_q_heads, s.n_kv_heads, vocab=per, n_blocks=1)
        st = Stage(sh, 0, 0, True, True, max_slots=1, max_ctx=64, max_tokens=32)
        st.load_weight("embed", -1, o.vocab_shard(emb, n, i))
        st.load_weight("readout", -1, o.vocab_shard(ro, n, i))
        st.load_weight("final_norm", -1, g)
        st.embed_range(tt, firsts[i], out=acc, accumulate=i > 0)
        slices.append(st)
    assert torch.equal(acc, want_rows)
    np.testing.assert_array_equal(acc.cpu().numpy(), o.embed_shards(emb, toks.astype(np.int64), n))
    for rows in (2, 16):                                  # GEMV path, then the MFMA GEMM path
        h = torch.from_numpy(hidden_rows(52, rows, d)).cuda()
        lf, hn = full.readout(h)
        cat = torch.cat([st.readout(h)[0] for st in slices], dim=1)[:, :V]
        e = rel_l2(cat.cpu().numpy(), lf.cpu().numpy())
        want = o.readout_shards(o.rms_norm(h.cpu().numpy(), o.bf16_to_f32(g), s.rms_eps), ro, n)
        e_o = rel_l2(cat.cpu().numpy(), want)
        say(f"{name} vocab over {n} slices, {rows} rows: concat vs full {e:.2e}, vs oracle {e_o:.2e}")
        if rows <= 4:
            assert torch.equal(cat, lf)
        assert e <= 1e-6 and e_o <= 1e-3


@pytest.mark.parametrize("name,T,n,zigzag", [("tiny", 24, 2, False), ("tiny", 24, 4, True), ("8b", 64, 2, False),
                                             ("8b", 64, 4, True), ("8b", 96, 3, True)])
def test_ring_attention_matches_the_plain_sublayer(name, T, n, zigzag):
    # context parallelism ("41. Many GPUs", Ring attention): n ranks' query chunks attend the K/V
    # chunks passed round the ring, partials merged in hop order; chunks of 3..48 keys straddle the
    # kernel's 32-key tiles, exercising the key-range masking
    s = fx.TINY if name == "tiny" else fx.LLAMA8B
    w = attn_weights(s)
    x = hidden_rows(53, T, s.d_model)
    xt = torch.from_numpy(x).cuda()
    st = Stage(slice_shape(s, s.n_q_heads, s.n_kv_heads), 0, 1, False, False, max_slots=2, max_ctx=128,
               max_tokens=128)
    for r, t in w.items():
        st.load_weight(r, 0, t)
    plain = st.attn(0, xt, 0, 0).cpu().numpy()
    ring = st.attn_ring(0, xt, 1, n, zigzag).cpu().numpy()
    c = o.Dims.of(s)
    want = o.attn_sublayer_ring(x, w["attn_norm"], w["wq"], w["wk"], w["wv"], w["wo"], s.head_dim, c.rms_eps,
                                c.rope_theta, n, zigzag)
    e_gpu, e_o = rel_l2(ring, plain), rel_l2(ring, want)
    say(f"{name} ring attention T={T}, {n} ranks, zigzag={zigzag}: vs plain (gpu) {e_gpu:.2e}, vs oracle {e_o:.2e}")
    assert e_gpu <= 1e-5 and e_o <= 1e-3
    # the ring call wrote the same K/V into its slot
    assert torch.equal(st.kv_export(0, 0, 0, T)[0], st.kv_export(0, 1, 0, T)[0])
