"""C ABI checks that need no GPU: the library loads, exports every declared entry point, and its
host-side validation refuses malformed and unsupported stages before any allocation."""
import ctypes
import os
import re

import pytest

import fixtures as fx
from pipeline_stage_decoder_amd import stage as S

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("stage.h", "pipeline.h", "placement.h")]


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(stage_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("stage_plan", "stage_create", "stage_load_weight", "stage_embed", "stage_prefill", "stage_decode",
              "stage_readout", "stage_mlp", "stage_kv_copy", "stage_kv_import", "stage_kv_export", "stage_destroy",
              "stage_status_str", "stage_last_error", "stage_greedy", "stage_describe", "stage_pipeline_workspace",
              "stage_pipeline_generate", "stage_place", "stage_attn", "stage_embed_range", "stage_attn_ring", "stage_attn_ring_workspace"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(S.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    # and the binding's table covers the same set
    assert set(declared_functions()) == set(S.EXPORTS)


def test_status_strings():
    L = S.lib()
    assert L.stage_status_str(0) == b"ok"
    assert b"fit" in L.stage_status_str(S.STAGE_E_DOES_NOT_FIT)
    assert L.stage_status_str(99) == b"unknown status"


def plan_rc(shape, **kw):
    base = dict(block_begin=0, block_end=shape.n_blocks_total, flags=S.STAGE_FIRST | S.STAGE_LAST, max_slots=2,
                max_ctx=64, max_tokens=16)
    base.update(kw)
    m = S.model_cfg(shape)
    s = S.StageCfg(base["block_begin"], base["block_end"], base["flags"], base["max_slots"], base["max_ctx"],
                   base["max_tokens"])
    p = S.Plan()
    return S.lib().stage_plan(ctypes.byref(m), ctypes.byref(s), ctypes.byref(p)), p


def test_plan_accepts_the_workloads_and_counts_bytes():
    rc, p = plan_rc(fx.TINY)
    assert rc == S.STAGE_OK
    assert p.total_bytes >= p.weight_bytes + p.kv_bytes + p.table_bytes + p.workspace_bytes
    rc, p8 = plan_rc(fx.LLAMA8B, block_end=16, flags=S.STAGE_FIRST, max_slots=1, max_ctx=2048, max_tokens=512)
    assert rc == S.STAGE_OK
    assert 8.0e9 < p8.weight_bytes < 8.1e9          # 16 blocks (6.98 GB) + embedding (1.05 GB)
    rc32, p32 = plan_rc(fx.LLAMA8B, block_end=16, flags=S.STAGE_FIRST | S.STAGE_KV_F32, max_slots=1,
                        max_ctx=2048, max_tokens=512)
    assert rc32 == S.STAGE_OK and p32.kv_bytes == 2 * p8.kv_bytes


@pytest.mark.parametrize("change,code", [
    (dict(head_dim=96), S.STAGE_E_UNSUPPORTED),
    (dict(n_kv_heads=3), S.STAGE_E_UNSUPPORTED),
    (dict(n_q_heads=64, n_kv_heads=2), S.STAGE_E_UNSUPPORTED),     # group of 32 > 16
    (dict(d_model=200), S.STAGE_E_UNSUPPORTED),
    (dict(d_ffn=680), S.STAGE_E_UNSUPPORTED),
    (dict(d_model=0), S.STAGE_E_INVALID),
])
def test_plan_refuses_unsupported_models(change, code):
    d = fx.TINY.__dict__.copy()
    d.update(change)
    rc, _ = plan_rc(fx.Shape(**d))
    assert rc == code


@pytest.mark.parametrize("kw,code", [
    (dict(block_begin=1, block_end=0), S.STAGE_E_INVALID),
    (dict(block_end=3), S.STAGE_E_INVALID),
    (dict(max_slots=0), S.STAGE_E_INVALID),
    (dict(max_tokens=0), S.STAGE_E_INVALID),
    (dict(flags=16), S.STAGE_E_INVALID),
    (dict(flags=S.STAGE_KV_F32 | S.STAGE_KV_F16), S.STAGE_E_INVALID),
    (dict(max_ctx=1 << 25), S.STAGE_E_UNSUPPORTED),
])
def test_plan_refuses_malformed_stages(kw, code):
    rc, _ = plan_rc(fx.TINY, **kw)
    assert rc == code


def test_create_refuses_before_touching_the_gpu():
    L = S.lib()
    m = S.model_cfg(fx.TINY)
    s = S.StageCfg(0, 2, 0, 1, 64, 16)
    h = ctypes.c_void_p()
    # null arena and an arena smaller than the plan are refused on the host
    assert L.stage_create(ctypes.byref(m), ctypes.byref(s), None, 1 << 30, 0, ctypes.byref(h)) == S.STAGE_E_INVALID
    assert L.stage_create(ctypes.byref(m), ctypes.byref(s), ctypes.c_void_p(1 << 20), 1024, 0,
                          ctypes.byref(h)) == S.STAGE_E_DOES_NOT_FIT
    bad = S.StageCfg(0, 2, 0, 1, 64, 0)
    assert L.stage_create(ctypes.byref(m), ctypes.byref(bad), ctypes.c_void_p(1 << 20), 1 << 30, 0,
                          ctypes.byref(h)) == S.STAGE_E_INVALID


def test_calls_on_a_null_handle_are_refused():
    L = S.lib()
    assert L.stage_prefill(None, 0, 0, 1, None, None, None) == S.STAGE_E_INVALID
    assert L.stage_decode(None, 1, None, None, None, None, None) == S.STAGE_E_INVALID
    assert L.stage_readout(None, 1, None, None, None, None) == S.STAGE_E_INVALID
    assert L.stage_embed(None, 1, None, None, None) == S.STAGE_E_INVALID
    assert L.stage_destroy(None) == S.STAGE_OK


def test_pipeline_and_greedy_refuse_bad_arguments_on_the_host():
    L = S.lib()
    cfg = S.GenCfg(2, 1, 16, 8)
    nbytes = ctypes.c_uint64(0)
    assert L.stage_pipeline_workspace(None, 2, ctypes.byref(cfg), ctypes.byref(nbytes)) == S.STAGE_E_INVALID
    handles = (ctypes.c_void_p * 2)(None, None)
    assert L.stage_pipeline_workspace(handles, 2, ctypes.byref(cfg), ctypes.byref(nbytes)) == S.STAGE_E_INVALID
    assert L.stage_pipeline_generate(handles, 0, ctypes.byref(cfg), None, None, None, 0, None) == S.STAGE_E_INVALID
    assert L.stage_greedy(-1, 10, None, None, None) == S.STAGE_E_INVALID
    assert L.stage_greedy(2, 0, None, None, None) == S.STAGE_E_INVALID
    assert L.stage_greedy(0, 10, None, None, None) == S.STAGE_OK          # nothing to do, no GPU call
    assert L.stage_describe(None, None, None, None) == S.STAGE_E_INVALID


def test_plan_kv_bytes_per_format():
    # bf16 and binary16 caches take 2 bytes per value, the F32-grade pair 4; nothing else changes
    def kv_bytes(flags):
        rc, p = plan_rc(fx.TINY, flags=flags)
        assert rc == S.STAGE_OK
        return p
    b16, f16, f32 = kv_bytes(0), kv_bytes(S.STAGE_KV_F16), kv_bytes(S.STAGE_KV_F32)
    assert f16.kv_bytes == b16.kv_bytes and f16.weight_bytes == b16.weight_bytes
    assert f32.kv_bytes >= 2 * b16.kv_bytes - 512
