"""The no-allocation entry point stage_attn_ring_noalloc against stage_attn_ring (GPU).

stage_attn_ring takes a caller-allocated workspace; stage_attn_ring_noalloc runs the same kernels
over the library's own device scratch.  Two calls in a row through the C ABI -- a sequence near
the scratch's limit, then a smaller one -- must give outputs bit-identical to the allocating entry
point's, both plain and accumulating, and a call past the limit must be refused on the host.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from pipeline_stage_decoder_amd import stage as S
from tests.gpu_util import hidden_rows

pytestmark = pytest.mark.gpu


def attn_stage(s, max_tokens):
    sh = fx.Shape(s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, 64, s.vocab, 1)
    st = S.Stage(sh, 0, 1, False, False, max_slots=2, max_ctx=max_tokens, max_tokens=max_tokens, kv="f16")
    for r in ("attn_norm", "wq", "wk", "wv", "wo"):
        st.load_weight(r, 0, fx.draw_weight(s, r, 0, gain_sigma=0.1))
    torch.cuda.synchronize()
    return st


def test_noalloc_ring_matches_the_allocating_entry_point():
    s = fx.LLAMA8B
    st = attn_stage(s, 1024)
    for T, n, zigzag in ((1008, 4, True), (64, 2, False)):        # near the 32 MiB limit, then smaller
        print(f"ring T={T}, {n} ranks, zigzag={zigzag}", flush=True)
        x = torch.from_numpy(hidden_rows(60, T, s.d_model)).cuda()
        want = st.attn_ring(0, x, 0, n, zigzag)
        got = torch.full_like(x, float("nan"))
        st.attn_ring_noalloc(0, x, 1, n, zigzag, out=got)
        torch.cuda.synchronize()
        assert torch.equal(got, want), T
        base = torch.from_numpy(hidden_rows(61, T, s.d_model)).cuda()
        want_acc = st.attn_ring(0, x, 0, n, zigzag, out=base.clone(), accumulate=True)
        got_acc = st.attn_ring_noalloc(0, x, 1, n, zigzag, out=base.clone(), accumulate=True)
        torch.cuda.synchronize()
        assert torch.equal(got_acc, want_acc), T
        assert torch.equal(st.kv_export(0, 0, 0, T)[0], st.kv_export(0, 1, 0, T)[0])
    assert st.device_errors() == 0


def test_noalloc_ring_refuses_a_call_past_its_scratch():
    s = fx.LLAMA8B
    st = attn_stage(s, 2048)
    x = torch.zeros((2048, s.d_model), dtype=torch.float32, device="cuda")
    out = torch.zeros_like(x)
    with pytest.raises(S.StageError) as e:
        st.attn_ring_noalloc(0, x, 0, 2, False, out=out)
    assert e.value.code == S.STAGE_E_DOES_NOT_FIT
    torch.cuda.synchronize()
    assert not out.any()                                          # nothing was enqueued
