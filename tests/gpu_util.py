"""Helpers of the GPU parity tests: build stages from seeded weights, drive them like the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import fixtures as fx
from pipeline_stage_decoder_amd.stage import Stage


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2_whole(got, want) -> float:
    """||got - want|| / ||want|| over the whole tensor."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(w)
    return float(np.linalg.norm(g - w) / (den if den > 0 else 1.0))


def rel_l2_rows(got, want) -> float:
    """The worst per-row relative L2, a row being the last axis (a hidden row, a logits row); a row
    whose reference is zero counts its absolute error."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    if g.ndim == 0 or g.size == 0:
        return rel_l2_whole(g, w)
    g = g.reshape(-1, g.shape[-1])
    w = w.reshape(-1, w.shape[-1])
    num = np.linalg.norm(g - w, axis=1)
    den = np.linalg.norm(w, axis=1)
    return float(np.max(num / np.where(den > 0, den, 1.0)))


def rel_l2(got, want) -> float:
    """The error every parity assertion bounds: the larger of the whole-tensor relative L2 and
    the worst single row's, so an error confined to one row (one slot, one ragged tile row)
    cannot hide in a large tensor."""
    return max(rel_l2_whole(got, want), rel_l2_rows(got, want))


def rel_l2_kv(got, want) -> float:
    """Relative L2 of cached K or V [n, Hkv, Dh], the worst of the whole tensor and of each KV
    head's [n, Dh] block."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    heads = [rel_l2_whole(g[:, h], w[:, h]) for h in range(g.shape[1])]
    return max([rel_l2_whole(g, w)] + heads)


def make_stage(shape, begin, end, first, last, weights: dict, **kw) -> Stage:
    st = Stage(shape, begin, end, first, last, **kw)
    for (role, block), w in weights.items():
        if role == "embed" and not first:
            continue
        if role in ("final_norm", "readout") and not last:
            continue
        if block >= 0 and not (begin <= block < end):
            continue
        st.load_weight(role, block, w)
    torch.cuda.synchronize()
    return st


def gpu_generate(stages: list, prompt: np.ndarray, n_new: int, slot: int = 0):
    """Greedy generation through GPU stages with F32 handoff; same trace keys as oracle.generate."""
    dev = stages[0].arena.device
    trace = {"handoff": [], "final_hidden": [], "logits": [], "residual": []}
    toks_in = torch.tensor(np.asarray(prompt, np.int32), device=dev)
    x = stages[0].embed(toks_in)
    for st in stages:
        x = st.prefill(x, slot, 0)
        trace["handoff"].append(x.cpu().numpy())
    logits, hn = stages[-1].readout(x)
    trace["residual"].append(x.cpu().numpy())
    trace["final_hidden"].append(hn.cpu().numpy())
    trace["logits"].append(logits.cpu().numpy())
    toks = [int(torch.argmax(logits[-1]).item())]
    pos = len(prompt)
    slots = torch.tensor([slot], dtype=torch.int32, device=dev)
    for _ in range(n_new - 1):
        x = stages[0].embed(torch.tensor([toks[-1]], dtype=torch.int32, device=dev))
        positions = torch.tensor([pos], dtype=torch.int32, device=dev)
        for st in stages:
            x = st.decode(x, slots, positions)
            trace["handoff"].append(x.cpu().numpy())
        logits, hn = stages[-1].readout(x)
        trace["residual"].append(x.cpu().numpy())
        trace["final_hidden"].append(hn.cpu().numpy())
        trace["logits"].append(logits.cpu().numpy())
        toks.append(int(torch.argmax(logits[0]).item()))
        pos += 1
    return np.array(toks, dtype=np.int32), trace


def kv_bits(st: Stage, block: int, slot: int, n: int):
    """The cache's K and V of one block and slot as raw bits (uint16 for bf16 and binary16, uint32
    for F32)."""
    k, v = st.kv_export(block, slot, 0, n)
    torch.cuda.synchronize()
    view = np.uint32 if st.kv_f32 else np.uint16
    return k.cpu().numpy().view(view), v.cpu().numpy().view(view)


def kv_values(kv: str, bits: np.ndarray) -> np.ndarray:
    """float32 values of cache bits in format kv ("bf16", "f16" or "f32")."""
    if kv == "f32":
        return bits.view(np.float32)
    if kv == "f16":
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def kv_bits_of(kv: str, values: np.ndarray) -> np.ndarray:
    """Cache bits of float32 values already representable in format kv."""
    values = np.asarray(values, np.float32)
    if kv == "f32":
        return values.view(np.uint32)
    if kv == "f16":
        return values.astype(np.float16).view(np.uint16)
    return (values.view(np.uint32) >> 16).astype(np.uint16)


def hidden_rows(seed_slot: int, n: int, d: int, offset_pos: int = 0) -> np.ndarray:
    """Seeded F32 N(0,1) hidden rows of a slot at positions offset_pos .. offset_pos+n."""
    return fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(seed_slot), n * d, offset_pos * d).reshape(n, d)
