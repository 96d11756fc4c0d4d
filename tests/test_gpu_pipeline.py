"""GPU tests of greedy sampling and of the in-flight pipeline driver (include/pipeline.h).

* stage_greedy against numpy's argmax on seeded logits with planted ties and -inf rows: the
  index is integer work, so it must match exactly (lowest index on ties).
* stage_pipeline_generate on the tiny decoder split into two stages [0, 1) + [1, 2), with
  2 micro-batches of 2 sequences in flight ("41. Many GPUs", Pipeline parallelism: batches of
  disjoint requests, each a step behind the one ahead): every sequence's greedy tokens must equal
  the oracle's greedy generation of that sequence alone, with one stream per stage and on a single
  stream (one batch in flight in effect).
* the driver refuses chains that are out of order or too small before enqueuing anything.
"""
import numpy as np
import pytest
import torch

import fixtures as fx
from oracle import decoder as o
from pipeline_stage_decoder_amd import stage as S
from tests.gpu_util import make_stage, say

pytestmark = pytest.mark.gpu

TINY = fx.TINY


@pytest.mark.parametrize("n,V", [(7, 1024), (2, 128256), (3, 5)])
def test_greedy_matches_numpy_argmax(n, V):
    x = fx.normal_f32(fx.SEED_HIDDEN, 0x6000 + V, n * V).reshape(n, V)
    x[0, V // 3] = x[0].max() + 1.0          # a unique maximum
    x[0, V - 1] = x[0, V // 3]               # ... tied later in the row: the lower index wins
    if n > 1:
        x[1, :] = -np.inf                    # all -inf: index 0
    if n > 2:
        x[2, 1] = np.nan                     # NaN never wins
        x[2, 3] = 7.0
    got = S.greedy(torch.from_numpy(x).cuda()).cpu().numpy()
    want = np.argmax(np.where(np.isnan(x), -np.inf, x), axis=1)
    say(f"greedy n={n} V={V}: {got.tolist()} vs {want.tolist()}")
    assert np.array_equal(got, want.astype(np.int32))


@pytest.fixture(scope="module")
def weights():
    return fx.draw_stage_weights(TINY, 0, 2, True, True, gain_sigma=0.1)


def two_stages(w, max_slots=4, max_ctx=64, max_tokens=16):
    a = make_stage(TINY, 0, 1, True, False, w, max_slots=max_slots, max_ctx=max_ctx, max_tokens=max_tokens)
    b = make_stage(TINY, 1, 2, False, True, w, max_slots=max_slots, max_ctx=max_ctx, max_tokens=max_tokens)
    return a, b


@pytest.mark.parametrize("use_streams", [True, False])
def test_pipeline_generate_matches_oracle(weights, use_streams):
    n_micro, rows, plen, n_new = 2, 2, 16, 8
    prompts = np.stack([fx.tokens(fx.SEED_TOKENS, fx.token_stream(10 + i), plen, TINY.vocab)
                        for i in range(n_micro * rows)]).reshape(n_micro, rows, plen).astype(np.int32)
    a, b = two_stages(weights)
    streams = [torch.cuda.Stream(), torch.cuda.Stream()] if use_streams else None
    say(f"pipeline: {n_micro} micro-batches x {rows} rows, streams={use_streams}")
    got = S.pipeline_generate([a, b], torch.from_numpy(prompts).cuda(), n_new, streams=streams).cpu().numpy()
    assert a.device_errors() == 0 and b.device_errors() == 0
    for m in range(n_micro):
        for r in range(rows):
            oa = o.Stage(o.Dims.of(TINY), 0, 1, True, False, weights, 64)
            ob = o.Stage(o.Dims.of(TINY), 1, 2, False, True, weights, 64)
            want, trace = o.generate([oa, ob], prompts[m, r], n_new)
            margins = [float(o.top2_margin(lg[-1:])[0]) for lg in trace["logits"]]
            say(f"  seq ({m},{r}): gpu {got[m, :, r].tolist()} oracle {want.tolist()} "
                f"min top-2 margin {min(margins):.3g}")
            assert np.array_equal(got[m, :, r], want)


def test_pipeline_one_micro_batch_equals_two(weights):
    # the same sequences, run as one micro-batch of 4 rows and as 2 micro-batches of 2 on two
    # streams, give the same tokens bit for bit
    plen, n_new = 16, 6
    prompts = np.stack([fx.tokens(fx.SEED_TOKENS, fx.token_stream(20 + i), plen, TINY.vocab)
                        for i in range(4)]).astype(np.int32)
    a, b = two_stages(weights)
    one = S.pipeline_generate([a, b], torch.from_numpy(prompts.reshape(1, 4, plen)).cuda(), n_new).cpu().numpy()
    two = S.pipeline_generate([a, b], torch.from_numpy(prompts.reshape(2, 2, plen)).cuda(), n_new,
                              streams=[torch.cuda.Stream(), torch.cuda.Stream()]).cpu().numpy()
    assert np.array_equal(one[0].T, np.concatenate([two[0].T, two[1].T], axis=0))


def test_pipeline_refuses_bad_chains(weights):
    a, b = two_stages(weights, max_slots=2)
    p = torch.zeros((2, 2, 16), dtype=torch.int32, device="cuda")
    with pytest.raises(S.StageError) as e:
        S.pipeline_generate([b, a], p, 4)                       # last stage first
    assert e.value.code == S.STAGE_E_ROLE
    with pytest.raises(S.StageError) as e:
        S.pipeline_generate([a, b], p, 4)                       # 4 sequences, 2 slots
    assert e.value.code == S.STAGE_E_RANGE
    with pytest.raises(S.StageError) as e:
        S.pipeline_generate([a, b], torch.zeros((1, 1, 60), dtype=torch.int32, device="cuda"), 8)
    assert e.value.code in (S.STAGE_E_RANGE, S.STAGE_E_INVALID)   # 60 + 7 positions > max_ctx 64
