"""Host tests of the placement planner (include/placement.h): contiguous stages, >= 1 block per
device, each stage's stage_plan bytes within its own device's budget ("RFC: pipeline placement
...", Heterogeneous GPUs; TensorSharp, Supported stage executors), the highest requirement /
budget ratio minimised.  The dynamic program is pinned against exhaustive enumeration of every
cut on small models, using the same per-stage requirements."""
import itertools
from fractions import Fraction

import pytest

import fixtures as fx
from pipeline_stage_decoder_amd import stage as S

SMALL = fx.Shape(256, 4, 2, 64, 688, 1024, 8)     # the tiny decoder with 8 blocks
KW = dict(max_slots=2, max_ctx=64, max_tokens=16)


def requirement(shape, begin, end, n_total, **kw):
    first, last = begin == 0, end == n_total
    return S.plan(shape, begin, end, first, last, kw["max_slots"], kw["max_ctx"], kw["max_tokens"]).total_bytes


def brute_force(shape, budgets, **kw):
    """Smallest achievable max(required_i / budget_i) over every contiguous placement, or None."""
    L, n = shape.n_blocks_total, len(budgets)
    best = None
    for inner in itertools.combinations(range(1, L), n - 1):
        cuts = (0, *inner, L)
        worst = Fraction(0)
        for i in range(n):
            q = requirement(shape, cuts[i], cuts[i + 1], L, **kw)
            if q > budgets[i]:
                worst = None
                break
            worst = max(worst, Fraction(q, budgets[i]))
        if worst is not None and (best is None or worst < best):
            best = worst
    return best


def check(shape, budgets, cuts, req, **kw):
    L = shape.n_blocks_total
    assert cuts[0] == 0 and cuts[-1] == L
    assert all(cuts[i] < cuts[i + 1] for i in range(len(budgets)))
    for i, b in enumerate(budgets):
        q = requirement(shape, cuts[i], cuts[i + 1], L, **kw)
        assert q == req[i] and q <= b
    return max(Fraction(q, b) for q, b in zip(req, budgets))


@pytest.mark.parametrize("n", [1, 2, 3, 4])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_matches_exhaustive_search(n, seed):
    whole = requirement(SMALL, 0, 8, 8, **KW)
    # budgets between 30% and 110% of the whole model, deterministic per (n, seed)
    draws = fx.splitmix64_sequence(0x91AC + 97 * n + seed, n)
    budgets = [int(whole * (0.3 + 0.8 * (d % 1000) / 1000)) for d in draws]
    want = brute_force(SMALL, budgets, **KW)
    if want is None:
        with pytest.raises(S.StageError) as e:
            S.place(SMALL, budgets, **KW)
        assert e.value.code == S.STAGE_E_DOES_NOT_FIT
        return
    cuts, req = S.place(SMALL, budgets, **KW)
    assert check(SMALL, budgets, cuts, req, **KW) == want


def test_equal_budgets_split_the_8b_model_in_half():
    cuts, req = S.place(fx.LLAMA8B, [20 << 30, 20 << 30], max_slots=1, max_ctx=2048, max_tokens=512)
    assert cuts == [0, 16, 32]                 # embedding and readout are the same size
    assert 0 <= req[1] - req[0] <= 4 * fx.LLAMA8B.d_model   # the last stage adds the F32 final-norm gain


def test_unequal_budgets_give_an_asymmetric_split():
    big, small = 24 << 30, 12 << 30
    cuts, req = S.place(fx.LLAMA8B, [big, small], max_slots=1, max_ctx=2048, max_tokens=512)
    assert cuts[1] - cuts[0] > cuts[2] - cuts[1]
    assert req[0] <= big and req[1] <= small
    # the same pair the other way round
    cuts2, _ = S.place(fx.LLAMA8B, [small, big], max_slots=1, max_ctx=2048, max_tokens=512)
    assert cuts2[1] - cuts2[0] < cuts2[2] - cuts2[1]


def test_budgets_are_per_device_never_summed():
    whole = requirement(SMALL, 0, 8, 8, **KW)
    one_block_last = requirement(SMALL, 7, 8, 8, **KW)
    # device 1 cannot hold even its smallest possible stage, although the two budgets add up to
    # more than the whole model
    budgets = [whole, one_block_last - 1]
    assert sum(budgets) > whole
    with pytest.raises(S.StageError) as e:
        S.place(SMALL, budgets, **KW)
    assert e.value.code == S.STAGE_E_DOES_NOT_FIT


def test_one_device():
    whole = requirement(SMALL, 0, 8, 8, **KW)
    assert S.place(SMALL, [whole], **KW)[0] == [0, 8]
    with pytest.raises(S.StageError) as e:
        S.place(SMALL, [whole - 1], **KW)
    assert e.value.code == S.STAGE_E_DOES_NOT_FIT


def test_more_devices_than_blocks_is_refused():
    with pytest.raises(S.StageError) as e:
        S.place(SMALL, [1 << 40] * 9, **KW)
    assert e.value.code == S.STAGE_E_INVALID
