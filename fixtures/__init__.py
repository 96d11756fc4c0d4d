"""Seeded synthetic inputs for the stage decoder: weights, tokens and F32 hidden rows.

This module is the only code that both the CPU oracle's tests and the GPU path's tests/bench
use.  It draws numbers; it computes nothing of the decoder.  The generator (SplitMix64 draws,
Irwin-Hall(12) normals, round-to-nearest-even bf16) is defined in ``fx_core.h`` and compiled
twice from that one definition: ``libfx.so`` for the host and ``libfx_gpu.so`` for device fills.

The source pages draw their weights "N(0, 0.02) from seed" and their inputs as random tokens
(TensorSharp's measured runs use "random prefill" tokens); these generators stand in for the
checkpoints and prompts the pages used.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
HOST_SO = os.path.join(HERE, "libfx.so")
GPU_SO = os.path.join(HERE, "libfx_gpu.so")

SEED_WEIGHTS = 0x5EED0001
SEED_TOKENS = 0x5EED0002
SEED_HIDDEN = 0x5EED0003

# Stream ids of the weight tensors.  Per-block tensors are keyed by the GLOBAL block index, so
# every way of splitting the blocks into stages draws identical weights.
ROLE_CODES = {
    "embed": 1, "attn_norm": 2, "wq": 3, "wk": 4, "wv": 5, "wo": 6, "mlp_norm": 7,
    "wgate": 8, "wup": 9, "wdown": 10, "final_norm": 11, "readout": 12,
}
BLOCK_ROLES = ("attn_norm", "wq", "wk", "wv", "wo", "mlp_norm", "wgate", "wup", "wdown")
GAIN_ROLES = ("attn_norm", "mlp_norm", "final_norm")


def weight_stream(role: str, global_block: int = -1) -> int:
    return (global_block + 1) * 64 + ROLE_CODES[role]


def hidden_stream(slot: int) -> int:
    """Stream of the F32 hidden rows fed to a non-first stage: element (pos * d + i) of a slot."""
    return 0x40000000 + slot


def token_stream(slot: int) -> int:
    return 0x20000000 + slot


# --------------------------------------------------------------------------------------------
# build / load
# --------------------------------------------------------------------------------------------

def build_host(force: bool = True) -> str:
    if force or not os.path.exists(HOST_SO):
        subprocess.check_call(
            ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
             os.path.join(HERE, "fx_host.c"), "-o", HOST_SO + ".tmp"])
        os.replace(HOST_SO + ".tmp", HOST_SO)
    return HOST_SO


def build_gpu(force: bool = True) -> str:
    if force or not os.path.exists(GPU_SO):
        subprocess.check_call(
            ["hipcc", "--offload-arch=gfx950", "-O3", "-ffp-contract=off", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             os.path.join(HERE, "fx_gpu.hip"), "-o", GPU_SO + ".tmp"],
            stderr=subprocess.DEVNULL if os.environ.get("FX_QUIET") else None)
        os.replace(GPU_SO + ".tmp", GPU_SO)
    return GPU_SO


_host = None
_gpu = None

_u64, _f32, _vp, _u32 = ctypes.c_uint64, ctypes.c_float, ctypes.c_void_p, ctypes.c_uint32


def host_lib():
    global _host
    if _host is None:
        if not os.path.exists(HOST_SO):
            build_host()
        lib = ctypes.CDLL(HOST_SO)
        lib.fx_fill_normal_bf16.argtypes = [_u64, _u64, _u64, _u64, _f32, _vp]
        lib.fx_fill_gain_bf16.argtypes = [_u64, _u64, _u64, _f32, _vp]
        lib.fx_fill_normal_f32.argtypes = [_u64, _u64, _u64, _u64, _vp]
        lib.fx_fill_tokens.argtypes = [_u64, _u64, _u64, _u32, _vp]
        lib.fx_splitmix64_next.argtypes = [ctypes.POINTER(_u64)]
        lib.fx_splitmix64_next.restype = _u64
        lib.fx_fnv1a64.argtypes = [_vp, _u64]
        lib.fx_fnv1a64.restype = _u64
        for f in (lib.fx_fill_normal_bf16, lib.fx_fill_gain_bf16, lib.fx_fill_normal_f32,
                  lib.fx_fill_tokens):
            f.restype = None
        _host = lib
    return _host


def gpu_lib():
    global _gpu
    if _gpu is None:
        if not os.path.exists(GPU_SO):
            raise RuntimeError(f"{GPU_SO} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(GPU_SO)
        lib.fxg_fill_normal_bf16.argtypes = [_u64, _u64, _u64, _u64, _f32, _vp, _vp]
        lib.fxg_fill_gain_bf16.argtypes = [_u64, _u64, _u64, _f32, _vp, _vp]
        lib.fxg_fill_normal_f32.argtypes = [_u64, _u64, _u64, _u64, _vp, _vp]
        lib.fxg_fill_tokens.argtypes = [_u64, _u64, _u64, _u32, _vp, _vp]
        for f in (lib.fxg_fill_normal_bf16, lib.fxg_fill_gain_bf16, lib.fxg_fill_normal_f32,
                  lib.fxg_fill_tokens):
            f.restype = ctypes.c_int
        _gpu = lib
    return _gpu


# --------------------------------------------------------------------------------------------
# host draws (numpy arrays)
# --------------------------------------------------------------------------------------------

def normal_bf16(seed: int, stream: int, n: int, sigma: float, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().fx_fill_normal_bf16(seed, stream, offset, n, sigma, out.ctypes.data)
    return out


def gain_bf16(seed: int, stream: int, n: int, sigma: float) -> np.ndarray:
    out = np.empty(n, dtype=np.uint16)
    host_lib().fx_fill_gain_bf16(seed, stream, n, sigma, out.ctypes.data)
    return out


def normal_f32(seed: int, stream: int, n: int, offset: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    host_lib().fx_fill_normal_f32(seed, stream, offset, n, out.ctypes.data)
    return out


def tokens(seed: int, stream: int, n: int, vocab: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    host_lib().fx_fill_tokens(seed, stream, n, vocab, out.ctypes.data)
    return out


def splitmix64_sequence(seed: int, n: int) -> list[int]:
    st = _u64(seed)
    return [int(host_lib().fx_splitmix64_next(ctypes.byref(st))) for _ in range(n)]


def fnv1a64(a: np.ndarray) -> int:
    a = np.ascontiguousarray(a)
    return int(host_lib().fx_fnv1a64(a.ctypes.data, a.nbytes))


# --------------------------------------------------------------------------------------------
# device draws (torch tensors on cuda), same bits as the host draws
# --------------------------------------------------------------------------------------------

def _stream_handle(torch_stream) -> int:
    return int(torch_stream.cuda_stream) if torch_stream is not None else 0


def normal_bf16_gpu(t, seed: int, stream: int, sigma: float, offset: int = 0, torch_stream=None):
    """Fill the int16/uint16/bfloat16 cuda tensor ``t`` (contiguous) with bf16 N(0, sigma^2) bits."""
    rc = gpu_lib().fxg_fill_normal_bf16(seed, stream, offset, t.numel(), sigma, t.data_ptr(),
                                        _stream_handle(torch_stream))
    if rc:
        raise RuntimeError(f"fxg_fill_normal_bf16 failed: hip error {rc}")
    return t


def gain_bf16_gpu(t, seed: int, stream: int, sigma: float, torch_stream=None):
    rc = gpu_lib().fxg_fill_gain_bf16(seed, stream, t.numel(), sigma, t.data_ptr(),
                                      _stream_handle(torch_stream))
    if rc:
        raise RuntimeError(f"fxg_fill_gain_bf16 failed: hip error {rc}")
    return t


def normal_f32_gpu(t, seed: int, stream: int, offset: int = 0, torch_stream=None):
    rc = gpu_lib().fxg_fill_normal_f32(seed, stream, offset, t.numel(), t.data_ptr(),
                                       _stream_handle(torch_stream))
    if rc:
        raise RuntimeError(f"fxg_fill_normal_f32 failed: hip error {rc}")
    return t


def tokens_gpu(t, seed: int, stream: int, vocab: int, torch_stream=None):
    rc = gpu_lib().fxg_fill_tokens(seed, stream, t.numel(), vocab, t.data_ptr(),
                                   _stream_handle(torch_stream))
    if rc:
        raise RuntimeError(f"fxg_fill_tokens failed: hip error {rc}")
    return t


# --------------------------------------------------------------------------------------------
# decoder shapes and the workloads they are drawn for
# --------------------------------------------------------------------------------------------

@dataclass(frozen=True)
class Shape:
    """Decoder dimensions: hidden d, q/KV heads, head dim, SwiGLU width, vocabulary, blocks."""
    d_model: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    d_ffn: int
    vocab: int
    n_blocks_total: int
    rms_eps: float = 1e-5
    rope_theta: float = 1e4


def role_shape(s: Shape, role: str) -> tuple[int, ...]:
    d, dh = s.d_model, s.head_dim
    return {
        "embed": (s.vocab, d), "readout": (s.vocab, d),
        "attn_norm": (d,), "mlp_norm": (d,), "final_norm": (d,),
        "wq": (s.n_q_heads * dh, d), "wk": (s.n_kv_heads * dh, d), "wv": (s.n_kv_heads * dh, d),
        "wo": (d, s.n_q_heads * dh),
        "wgate": (s.d_ffn, d), "wup": (s.d_ffn, d), "wdown": (d, s.d_ffn),
    }[role]


def draw_weight(s: Shape, role: str, global_block: int = -1, seed: int = SEED_WEIGHTS,
                sigma: float = 0.02, gain_sigma: float = 0.0) -> np.ndarray:
    """bf16 bits of one weight tensor, shaped as the role's [out, in] (gains: [d])."""
    shape = role_shape(s, role)
    n = int(np.prod(shape))
    stream = weight_stream(role, global_block)
    if role in GAIN_ROLES:
        return gain_bf16(seed, stream, n, gain_sigma).reshape(shape)
    return normal_bf16(seed, stream, n, sigma).reshape(shape)


def stage_roles(block_begin: int, block_end: int, first: bool, last: bool):
    """(role, global_block) pairs a stage owns: its blocks' tensors plus the end tensors."""
    out = []
    if first:
        out.append(("embed", -1))
    for b in range(block_begin, block_end):
        out.extend((r, b) for r in BLOCK_ROLES)
    if last:
        out.extend([("final_norm", -1), ("readout", -1)])
    return out


def draw_stage_weights(s: Shape, block_begin: int, block_end: int, first: bool, last: bool,
                       seed: int = SEED_WEIGHTS, gain_sigma: float = 0.0) -> dict:
    return {(r, b): draw_weight(s, r, b, seed, gain_sigma=gain_sigma)
            for r, b in stage_roles(block_begin, block_end, first, last)}


@dataclass(frozen=True)
class Workload:
    name: str
    shape: Shape
    block_begin: int
    block_end: int
    first: bool
    last: bool
    prefill_tokens: int = 0
    decode_batch: int = 0
    decode_ctx: int = 0
    notes: str = ""
    extra: dict = field(default_factory=dict)


TINY = Shape(256, 4, 2, 64, 688, 1024, 2)
LLAMA8B = Shape(4096, 32, 8, 128, 14336, 128256, 32)
LLAMA70B = Shape(8192, 64, 8, 128, 28672, 128256, 80)

WORKLOADS = {
    "tiny_split": Workload(
        "tiny 2-block decoder split at block 1, 16-token prompt, greedy 8", TINY, 0, 2, True, True,
        prefill_tokens=16, decode_batch=1, extra={"split": 1, "greedy": 8}),
    "llama8b_first_stage": Workload(
        "8B-shaped first stage: embedding + blocks 0..15, prefill 512 then decode B=1 to ctx 2048",
        LLAMA8B, 0, 16, True, False, prefill_tokens=512, decode_batch=1, decode_ctx=2048),
    "llama8b_last_stage": Workload(
        "8B-shaped last stage: blocks 16..31 + final norm + readout, decode B=64 at ctx 4096",
        LLAMA8B, 16, 32, False, True, decode_batch=64, decode_ctx=4096),
    "llama70b_mid_stage": Workload(
        "70B-shaped middle stage: blocks 20..39, prefill chunk 4096, decode B=128 at ctx 8192",
        LLAMA70B, 20, 40, False, False, prefill_tokens=4096, decode_batch=128, decode_ctx=8192),
    "mlp_slices_8x3584": Workload(
        "sharded-MLP slice check: d 8192, 8 slices of 3584, T in {1, 64, 4096}",
        LLAMA70B, 0, 1, False, False, extra={"slices": 8, "slice_width": 3584,
                                             "tokens": (1, 64, 4096)}),
}
