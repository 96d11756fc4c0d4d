"""Byte/flop accounting pinned to the numbers the pages print (CPU only)."""
import json
import os

import fixtures as fx
from pipeline_stage_decoder_amd import accounting as acc

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_traffic.json")))


def test_pipeline_send_bytes_match_the_chapter():
    m, w, p = G["model"], G["workload"], G["printed"]
    b = acc.pp_send_bytes(w["prompts"], w["prompt_tokens"], w["new_tokens"], m["hidden"], m["dtype_bytes"])
    assert round(b / 1e6, 2) == p["pipeline_send_MB"]
    assert b == 8 * 64 * 512 * 4 + 15 * 8 * 512 * 4


def test_tensor_parallel_traffic_matches_the_chapter():
    m, w, p = G["model"], G["workload"], G["printed"]
    calls, b = acc.tp_all_reduce(m["layers"], w["prompts"], w["prompt_tokens"], w["new_tokens"], m["hidden"],
                                 m["dtype_bytes"])
    assert calls == p["tensor_all_reduce_calls"]
    assert round(b / 1e6, 2) == p["tensor_all_reduce_MB"]
    assert round(w["prompts"] * w["prompt_tokens"] * m["hidden"] * 4 / 2 ** 20, 2) == p["prefill_all_reduce_MB"]
    assert w["prompts"] * m["hidden"] * 4 // 1024 == p["decode_all_reduce_KB"]
    for ranks, key in ((2, "tensor_all_gather_MB_2_ranks"), (4, "tensor_all_gather_MB_4_ranks")):
        g = acc.tp_all_gather_bytes(w["new_tokens"], w["prompts"], m["vocab"], ranks, 4)
        assert round(g / 1e6, 2) == p[key]


def test_kv_bytes_and_prefill_flops_match_the_chapter():
    k = G["kv_example"]
    per_tok = acc.kv_bytes_per_token(k["layers"], k["kv_heads"], k["head_dim"], k["dtype_bytes"])
    assert per_tok // 1024 == k["kv_KB_per_token"]
    assert round(per_tok * k["prompt_tokens"] / 1e6) == k["prompt_MB"]
    assert round(2 * k["params_B"] * 1e9 * k["prompt_tokens"] / 1e12) == k["prefill_TFLOP"]


def test_stage_figures_of_the_workloads():
    s = fx.LLAMA8B
    assert acc.block_weight_bytes(s) == (6144 * 4096 + 4096 * 4096 + 3 * 14336 * 4096) * 2
    assert acc.kv_bytes_per_token_block(s) == 4096
    # config-1 decode: 16 blocks of weights plus KV; ~6.98 GB of weights per step
    b = acc.decode_step_bytes(s, 16, [1024], first=True)
    assert 6.97e9 < b < 7.1e9
    f = acc.prefill_flops(s, 16, 512)
    assert 3.55e12 < f < 3.65e12
    t = acc.prefill_flops(fx.LLAMA70B, 20, 4096)
    assert 1.45e14 < t < 1.47e14
