"""GPU runtime properties: graph replay, device generator bits, arena/ABI behaviour on a GPU."""
import numpy as np
import pytest
import torch

import fixtures as fx
from tests.gpu_util import hidden_rows, make_stage

pytestmark = pytest.mark.gpu


def test_device_generator_matches_host_generator():
    dev = torch.device("cuda")
    for seed, stream, n, sigma in ((fx.SEED_WEIGHTS, 77, 100003, 0.02), (1, 2, 4096, 1.0)):
        t = fx.normal_bf16_gpu(torch.empty(n, dtype=torch.int16, device=dev), seed, stream, sigma)
        assert np.array_equal(t.cpu().numpy().view(np.uint16), fx.normal_bf16(seed, stream, n, sigma))
    g = fx.gain_bf16_gpu(torch.empty(4096, dtype=torch.int16, device=dev), 3, 4, 0.1)
    assert np.array_equal(g.cpu().numpy().view(np.uint16), fx.gain_bf16(3, 4, 4096, 0.1))
    h = fx.normal_f32_gpu(torch.empty(5000, dtype=torch.float32, device=dev), 5, 6, offset=17)
    assert np.array_equal(h.cpu().numpy(), fx.normal_f32(5, 6, 5000, offset=17))
    k = fx.tokens_gpu(torch.empty(999, dtype=torch.int32, device=dev), 7, 8, 128256)
    assert np.array_equal(k.cpu().numpy(), fx.tokens(7, 8, 999, 128256))


@pytest.mark.parametrize("B", [1, 8])
def test_decode_graph_replay_matches_eager(B):
    s = fx.TINY
    w = fx.draw_stage_weights(s, 0, 2, False, False, gain_sigma=0.1)
    dev = torch.device("cuda")

    def setup():
        st = make_stage(s, 0, 2, False, False, w, max_slots=B, max_ctx=64, max_tokens=16)
        for b in range(B):
            st.prefill(torch.from_numpy(hidden_rows(b, 5 + b, s.d_model)).to(dev), b, 0)
        return st

    xs = [torch.from_numpy(np.vstack([hidden_rows(50 + i, 1, s.d_model, b) for b in range(B)])).to(dev)
          for i in range(3)]
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    base = torch.tensor([5 + b for b in range(B)], dtype=torch.int32, device=dev)
    eager = setup()
    want = [eager.decode(xs[i], slots, base + i).cpu().numpy() for i in range(3)]
    st = setup()
    x_in = torch.empty_like(xs[0])
    pos = torch.empty_like(base)
    out = torch.empty_like(xs[0])
    x_in.copy_(xs[0])
    pos.copy_(base)
    st.decode(x_in, slots, pos, out=out)             # warm-up outside capture (position base)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cs):
        st.decode(x_in, slots, pos, out=out)
    for i in range(3):                                # replays with new inputs and positions
        x_in.copy_(xs[i])
        pos.copy_(base + i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert out.cpu().numpy().tobytes() == want[i].tobytes(), i


def test_stage_refuses_small_arena_and_foreign_roles():
    from pipeline_stage_decoder_amd import stage as S
    s = fx.TINY
    st = S.Stage(s, 0, 1, False, False, max_slots=1, max_ctx=64, max_tokens=4)
    with pytest.raises(S.StageError) as e:
        st.load_weight("embed", -1, np.zeros(s.vocab * s.d_model, np.uint16))
    assert e.value.code == S.STAGE_E_ROLE
    with pytest.raises(S.StageError) as e:
        st.load_weight("wq", 1, np.zeros(s.n_q_heads * s.head_dim * s.d_model, np.uint16))
    assert e.value.code == S.STAGE_E_ROLE
    with pytest.raises(S.StageError) as e:
        st.prefill(torch.zeros((2, s.d_model), device="cuda"), 0, 63)
    assert e.value.code == S.STAGE_E_RANGE
    with pytest.raises(S.StageError) as e:
        st.prefill(torch.zeros((5, s.d_model), device="cuda"), 0, 0)
    assert e.value.code == S.STAGE_E_INVALID
    import ctypes
    arena = torch.empty(1024, dtype=torch.uint8, device="cuda")
    h = ctypes.c_void_p()
    rc = S.lib().stage_create(ctypes.byref(st._m), ctypes.byref(st._s), arena.data_ptr(), arena.numel(), 0,
                              ctypes.byref(h))
    assert rc == S.STAGE_E_DOES_NOT_FIT


def test_kv_import_export_formats():
    # STAGE_KV_F32 keeps each value as a bf16 hi + lo pair: import splits F32 values (hi = bf16(x),
    # lo = bf16(x - hi), both rounded to nearest even), export returns hi + lo, so the round trip
    # is that sum bit for bit and within 2^-16 of x.  A bf16 cache returns the imported bits.
    from oracle import decoder as o
    s = fx.TINY
    dev = torch.device("cuda")
    n, shp = 40, (40, s.n_kv_heads, s.head_dim)
    per = int(np.prod(shp))
    st = make_stage(s, 0, 1, False, False, {}, max_slots=2, max_ctx=64, max_tokens=16, kv_f32=True)
    k = fx.normal_f32(9, 1, per).reshape(shp)
    v = fx.normal_f32(9, 2, per).reshape(shp)
    st.kv_import(0, 1, 3, torch.from_numpy(k).to(dev), torch.from_numpy(v).to(dev))
    ke, ve = st.kv_export(0, 1, 3, n)
    for x, got in ((k, ke.cpu().numpy()), (v, ve.cpu().numpy())):
        hi = o.bf16_to_f32(o.f32_to_bf16_bits(x))
        lo = o.bf16_to_f32(o.f32_to_bf16_bits((x - hi).astype(np.float32)))
        assert np.array_equal(got, (hi + lo).astype(np.float32))
        assert np.all(np.abs(got.astype(np.float64) - x) <= 2.0 ** -16 * np.abs(x))
    st2 = make_stage(s, 0, 1, False, False, {}, max_slots=2, max_ctx=64, max_tokens=16)
    kb = fx.normal_bf16(9, 3, per, 1.0).reshape(shp)
    vb = fx.normal_bf16(9, 4, per, 1.0).reshape(shp)
    st2.kv_import(0, 0, 0, torch.from_numpy(kb.view(np.int16)).to(dev), torch.from_numpy(vb.view(np.int16)).to(dev))
    ke2, ve2 = st2.kv_export(0, 0, 0, n)
    assert np.array_equal(ke2.cpu().numpy().view(np.uint16), kb)
    assert np.array_equal(ve2.cpu().numpy().view(np.uint16), vb)
