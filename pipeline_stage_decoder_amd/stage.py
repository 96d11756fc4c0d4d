"""ctypes binding of the stage C ABI (include/stage.h): argument marshalling only.

Every step of the forward runs in the HIP kernels of ``libpsd_stage.so``; PyTorch supplies the
device arena, the in/out buffers and the stream.  There is no CPU fallback: without the built
library, or without a GPU, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

# PSD_STAGE_LIB selects another build of the same library (the host-sanitized one in the CPU tests)
LIB_PATH = os.environ.get("PSD_STAGE_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libpsd_stage.so")

STAGE_OK, STAGE_E_INVALID, STAGE_E_UNSUPPORTED, STAGE_E_DOES_NOT_FIT, STAGE_E_ROLE, STAGE_E_RANGE, \
    STAGE_E_HIP = range(7)
STAGE_FIRST, STAGE_LAST, STAGE_KV_F32, STAGE_KV_F16 = 1, 2, 4, 8
KV_FLAGS = {"bf16": 0, "f32": STAGE_KV_F32, "f16": STAGE_KV_F16}

KERNEL_KINDS = {"embed": 0, "norm": 1, "qkv": 2, "attn": 3, "o": 4, "gateup": 5, "down": 6, "readout": 7}

ROLES = {
    "embed": 0, "attn_norm": 1, "wq": 2, "wk": 3, "wv": 4, "wo": 5, "mlp_norm": 6, "wgate": 7,
    "wup": 8, "wdown": 9, "final_norm": 10, "readout": 11,
}


class ModelCfg(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("n_blocks_total", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class StageCfg(ctypes.Structure):
    _fields_ = [("block_begin", ctypes.c_int32), ("block_end", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("max_slots", ctypes.c_int32), ("max_ctx", ctypes.c_int32), ("max_tokens", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("weight_bytes", ctypes.c_uint64), ("kv_bytes", ctypes.c_uint64), ("table_bytes", ctypes.c_uint64),
                ("workspace_bytes", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64)]

    def as_dict(self):
        return {f: int(getattr(self, f)) for f, _ in self._fields_}


class GenCfg(ctypes.Structure):
    _fields_ = [("n_micro", ctypes.c_int32), ("rows", ctypes.c_int32), ("prompt_len", ctypes.c_int32),
                ("n_new", ctypes.c_int32)]


class StageError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(msg)
        self.code = code


_lib = None
_vp, _i32, _u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64

EXPORTS = {
    "stage_plan": [ctypes.POINTER(ModelCfg), ctypes.POINTER(StageCfg), ctypes.POINTER(Plan)],
    "stage_create": [ctypes.POINTER(ModelCfg), ctypes.POINTER(StageCfg), _vp, _u64, _i32, ctypes.POINTER(_vp)],
    "stage_load_weight": [_vp, _i32, _i32, _vp, _u64, _vp],
    "stage_embed": [_vp, _i32, _vp, _vp, _vp],
    "stage_prefill": [_vp, _i32, _i32, _i32, _vp, _vp, _vp],
    "stage_decode": [_vp, _i32, _vp, _vp, _vp, _vp, _vp],
    "stage_readout": [_vp, _i32, _vp, _vp, _vp, _vp],
    "stage_mlp": [_vp, _i32, _i32, _vp, _vp, _i32, _vp],
    "stage_kv_copy": [_vp, _i32, _i32, _i32, _vp],
    "stage_kv_import": [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp],
    "stage_kv_export": [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp],
    "stage_device_errors": [_vp, _i32, ctypes.POINTER(ctypes.c_uint32), _vp],
    "stage_timing": [_vp, ctypes.c_uint32],
    "stage_timing_read": [_vp, _i32, ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(ctypes.c_double)],
    "stage_attn": [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp],
    "stage_embed_range": [_vp, _i32, _vp, _i32, _vp, _i32, _vp],
    "stage_attn_ring_workspace": [_vp, _i32, ctypes.POINTER(ctypes.c_uint64)],
    "stage_attn_ring": [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp, _u64, _vp],
    "stage_attn_ring_noalloc": [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _i32, _vp],
    "stage_greedy": [_i32, _i32, _vp, _vp, _vp],
    "stage_describe": [_vp, ctypes.POINTER(ModelCfg), ctypes.POINTER(StageCfg), ctypes.POINTER(ctypes.c_int)],
    "stage_pipeline_workspace": [ctypes.POINTER(_vp), _i32, ctypes.POINTER(GenCfg), ctypes.POINTER(ctypes.c_uint64)],
    "stage_pipeline_generate": [ctypes.POINTER(_vp), _i32, ctypes.POINTER(GenCfg), _vp, _vp, _vp, _u64,
                                ctypes.POINTER(_vp)],
    "stage_place": [ctypes.POINTER(ModelCfg), ctypes.POINTER(StageCfg), _i32, ctypes.POINTER(ctypes.c_uint64),
                    ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_uint64)],
    "stage_destroy": [_vp],
    "stage_status_str": [_i32],
    "stage_last_error": [_vp],
}


def lib():
    """Load libpsd_stage.so (built by __graft_entry__.build()); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        for name, argtypes in EXPORTS.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_char_p if name in ("stage_status_str", "stage_last_error") else ctypes.c_int
        _lib = L
    return _lib


def model_cfg(shape) -> ModelCfg:
    """A stage_model_cfg from any object with the decoder's dimension attributes."""
    return ModelCfg(shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.d_ffn, shape.vocab,
                    shape.n_blocks_total, shape.rms_eps, shape.rope_theta)


def kv_format(kv, kv_f32: bool) -> str:
    """The cache format name: `kv` ("bf16", "f16" or "f32") if given, else "f32" when kv_f32."""
    fmt = kv if kv is not None else ("f32" if kv_f32 else "bf16")
    if fmt not in KV_FLAGS:
        raise ValueError(f"unknown KV cache format {fmt!r}")
    return fmt


def place(shape, budgets, *, max_slots: int = 1, max_ctx: int = 2048, max_tokens: int = 512,
          kv_f32: bool = False, kv: str | None = None):
    """Contiguous byte-balanced placement over len(budgets) devices (include/placement.h), host only.
    Returns (cuts, required): device i gets blocks [cuts[i], cuts[i+1])."""
    n = len(budgets)
    m = model_cfg(shape)
    s = StageCfg(0, 0, KV_FLAGS[kv_format(kv, kv_f32)], max_slots, max_ctx, max_tokens)
    b = (ctypes.c_uint64 * n)(*[int(x) for x in budgets])
    cuts = (ctypes.c_int32 * (n + 1))()
    req = (ctypes.c_uint64 * n)()
    rc = lib().stage_place(ctypes.byref(m), ctypes.byref(s), n, b, cuts, req)
    if rc != STAGE_OK:
        raise StageError(rc, f"stage_place: {lib().stage_status_str(rc).decode()}")
    return list(cuts), list(req)


def plan(shape, block_begin, block_end, first, last, max_slots, max_ctx, max_tokens, kv: str = "bf16") -> Plan:
    m = model_cfg(shape)
    s = StageCfg(block_begin, block_end, (STAGE_FIRST if first else 0) | (STAGE_LAST if last else 0)
                 | KV_FLAGS[kv_format(kv, False)], max_slots, max_ctx, max_tokens)
    p = Plan()
    rc = lib().stage_plan(ctypes.byref(m), ctypes.byref(s), ctypes.byref(p))
    if rc != STAGE_OK:
        raise StageError(rc, f"stage_plan: {lib().stage_status_str(rc).decode()}")
    return p


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


@dataclass
class StageSpec:
    block_begin: int
    block_end: int
    first: bool
    last: bool
    max_slots: int
    max_ctx: int
    max_tokens: int


class Stage:
    """One pipeline stage on one GPU: weights, KV cache and workspace in one torch-owned arena."""

    def __init__(self, shape, block_begin: int, block_end: int, first: bool, last: bool, *, max_slots: int = 1,
                 max_ctx: int = 2048, max_tokens: int = 512, device: int = 0, kv_f32: bool = False,
                 kv: str | None = None):
        if not torch.cuda.is_available():
            raise RuntimeError("Stage needs a ROCm GPU; none is visible")
        self.shape = shape
        self.spec = StageSpec(block_begin, block_end, first, last, max_slots, max_ctx, max_tokens)
        self.device = device
        self._m = model_cfg(shape)
        self.kv = kv_format(kv, kv_f32)          # KV cache format: "bf16", "f16" or "f32"
        self.kv_f32 = self.kv == "f32"
        self._s = StageCfg(block_begin, block_end, (STAGE_FIRST if first else 0) | (STAGE_LAST if last else 0)
                           | KV_FLAGS[self.kv], max_slots, max_ctx, max_tokens)
        self.plan = Plan()
        self._check(lib().stage_plan(ctypes.byref(self._m), ctypes.byref(self._s), ctypes.byref(self.plan)),
                    "stage_plan")
        self.arena = torch.empty(int(self.plan.total_bytes), dtype=torch.uint8, device=f"cuda:{device}")
        h = _vp()
        self._check(lib().stage_create(ctypes.byref(self._m), ctypes.byref(self._s), self.arena.data_ptr(),
                                       int(self.arena.numel()), device, ctypes.byref(h)), "stage_create")
        self._h = h

    # -- plumbing ---------------------------------------------------------------------------
    def _check(self, rc: int, what: str):
        if rc != STAGE_OK:
            detail = ""
            if getattr(self, "_h", None):
                detail = lib().stage_last_error(self._h).decode()
            raise StageError(rc, f"{what}: {lib().stage_status_str(rc).decode()} {detail}".strip())

    def close(self):
        if getattr(self, "_h", None):
            lib().stage_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def d(self) -> int:
        return self.shape.d_model

    # -- weights ------------------------------------------------------------------------------
    def load_weight(self, role: str, global_block: int, src, stream=None):
        """src: bf16 bits as a numpy uint16 array (host) or a torch int16/uint16/bfloat16 tensor (host or device)."""
        if isinstance(src, torch.Tensor):
            src = src.contiguous()
            ptr, n = src.data_ptr(), src.numel()
            keep = src
        else:
            import numpy as np
            keep = np.ascontiguousarray(src, dtype=np.uint16)
            ptr, n = keep.ctypes.data, keep.size
        self._check(lib().stage_load_weight(self._h, ROLES[role], global_block, ptr, n, _stream(stream)),
                    f"stage_load_weight({role}, {global_block})")
        del keep

    def load_weights(self, weights: dict, stream=None):
        for (role, block), w in weights.items():
            self.load_weight(role, block, w, stream)

    # -- forward ------------------------------------------------------------------------------
    def embed(self, tokens: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        n = tokens.numel()
        if out is None:
            out = torch.empty((n, self.d), dtype=torch.float32, device=tokens.device)
        self._check(lib().stage_embed(self._h, n, _ptr(tokens), _ptr(out), _stream(stream)), "stage_embed")
        return out

    def prefill(self, hidden_in: torch.Tensor, slot: int, pos0: int, out: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
        T = hidden_in.shape[0]
        if out is None:
            out = torch.empty_like(hidden_in)
        self._check(lib().stage_prefill(self._h, slot, pos0, T, _ptr(hidden_in), _ptr(out), _stream(stream)),
                    "stage_prefill")
        return out

    def decode(self, hidden_in: torch.Tensor, slots: torch.Tensor, positions: torch.Tensor,
               out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        B = hidden_in.shape[0]
        if out is None:
            out = torch.empty_like(hidden_in)
        self._check(lib().stage_decode(self._h, B, _ptr(slots), _ptr(positions), _ptr(hidden_in), _ptr(out),
                                       _stream(stream)), "stage_decode")
        return out

    def readout(self, hidden_in: torch.Tensor, logits: torch.Tensor | None = None,
                normed: torch.Tensor | None = None, want_normed: bool = True, stream=None):
        n = hidden_in.shape[0]
        if logits is None:
            logits = torch.empty((n, self.shape.vocab), dtype=torch.float32, device=hidden_in.device)
        if normed is None and want_normed:
            normed = torch.empty_like(hidden_in)
        self._check(lib().stage_readout(self._h, n, _ptr(hidden_in), _ptr(logits), _ptr(normed), _stream(stream)),
                    "stage_readout")
        return logits, normed

    def mlp(self, global_block: int, hidden_in: torch.Tensor, out: torch.Tensor | None = None,
            accumulate: bool = False, stream=None) -> torch.Tensor:
        n = hidden_in.shape[0]
        if out is None:
            out = torch.empty_like(hidden_in)
        self._check(lib().stage_mlp(self._h, global_block, n, _ptr(hidden_in), _ptr(out), int(accumulate),
                                    _stream(stream)), "stage_mlp")
        return out

    def attn(self, global_block: int, hidden_in: torch.Tensor, slot: int, pos0: int, out: torch.Tensor | None = None,
             accumulate: bool = False, stream=None) -> torch.Tensor:
        """Attention sublayer of one block without its residual (stage_attn)."""
        t = hidden_in.shape[0]
        if out is None:
            out = torch.empty_like(hidden_in)
        self._check(lib().stage_attn(self._h, global_block, slot, pos0, t, _ptr(hidden_in), _ptr(out), int(accumulate),
                                     _stream(stream)), "stage_attn")
        return out

    def attn_ring(self, global_block: int, hidden_in: torch.Tensor, slot: int, n_ranks: int, zigzag: bool,
                  out: torch.Tensor | None = None, accumulate: bool = False, stream=None) -> torch.Tensor:
        """stage_attn with the attention taken the ring way (stage_attn_ring), positions 0..T-1."""
        t = hidden_in.shape[0]
        if out is None:
            out = torch.empty_like(hidden_in)
        nbytes = ctypes.c_uint64(0)
        self._check(lib().stage_attn_ring_workspace(self._h, t, ctypes.byref(nbytes)), "stage_attn_ring_workspace")
        ws = torch.empty(int(nbytes.value), dtype=torch.uint8, device=hidden_in.device)
        self._check(lib().stage_attn_ring(self._h, global_block, slot, t, n_ranks, int(zigzag), _ptr(hidden_in),
                                          _ptr(out), int(accumulate), _ptr(ws), int(ws.numel()), _stream(stream)),
                    "stage_attn_ring")
        return out

    def attn_ring_noalloc(self, global_block: int, hidden_in: torch.Tensor, slot: int, n_ranks: int, zigzag: bool,
                          out: torch.Tensor, accumulate: bool = False, stream=None) -> torch.Tensor:
        """stage_attn_ring_noalloc: attn_ring with the library's own scratch (the caller passes `out`;
        nothing is allocated)."""
        t = hidden_in.shape[0]
        self._check(lib().stage_attn_ring_noalloc(self._h, global_block, slot, t, n_ranks, int(zigzag),
                                                  _ptr(hidden_in), _ptr(out), int(accumulate), _stream(stream)),
                    "stage_attn_ring_noalloc")
        return out

    def embed_range(self, tokens: torch.Tensor, vocab_lo: int, out: torch.Tensor | None = None,
                    accumulate: bool = False, stream=None) -> torch.Tensor:
        """Rows of a vocabulary slice holding ids [vocab_lo, vocab_lo + V) (stage_embed_range)."""
        n = tokens.shape[0]
        if out is None:
            out = torch.empty((n, self.shape.d_model), dtype=torch.float32, device=tokens.device)
        self._check(lib().stage_embed_range(self._h, n, _ptr(tokens), vocab_lo, _ptr(out), int(accumulate),
                                            _stream(stream)), "stage_embed_range")
        return out

    def kv_copy(self, src_slot: int, dst_slot: int, n_pos: int, stream=None):
        self._check(lib().stage_kv_copy(self._h, src_slot, dst_slot, n_pos, _stream(stream)), "stage_kv_copy")

    def kv_import(self, global_block: int, slot: int, pos0: int, k: torch.Tensor, v: torch.Tensor, stream=None):
        """k, v: [n, Hkv, Dh] device tensors in the cache's element type (bf16 or binary16 bits as int16,
        or float32 for the F32-grade cache)."""
        want = torch.float32 if self.kv_f32 else torch.int16
        if k.dtype != want or v.dtype != want:
            raise TypeError(f"kv_import expects {want} tensors for this stage")
        n = k.shape[0]
        self._check(lib().stage_kv_import(self._h, global_block, slot, pos0, n, _ptr(k.contiguous()),
                                          _ptr(v.contiguous()), _stream(stream)), "stage_kv_import")

    def kv_export(self, global_block: int, slot: int, pos0: int, n: int, stream=None):
        """K and V [n, Hkv, Dh] in the cache's element type (int16 bf16 or binary16 bits, or float32)."""
        shp = (n, self.shape.n_kv_heads, self.shape.head_dim)
        dev = self.arena.device
        dt = torch.float32 if self.kv_f32 else torch.int16
        k = torch.empty(shp, dtype=dt, device=dev)
        v = torch.empty(shp, dtype=dt, device=dev)
        self._check(lib().stage_kv_export(self._h, global_block, slot, pos0, n, _ptr(k), _ptr(v), _stream(stream)),
                    "stage_kv_export")
        return k, v

    def device_errors(self, reset: bool = False, stream=None) -> int:
        c = ctypes.c_uint32(0)
        self._check(lib().stage_device_errors(self._h, int(reset), ctypes.byref(c), _stream(stream)),
                    "stage_device_errors")
        return int(c.value)

    # -- kernel timing -----------------------------------------------------------------------------
    def timing(self, kinds=()):
        """Record HIP event pairs around the launches of the given kernel kinds (names of KERNEL_KINDS)."""
        mask = 0
        for k in kinds:
            mask |= 1 << KERNEL_KINDS[k]
        self._check(lib().stage_timing(self._h, mask), "stage_timing")

    def timing_read(self, kind: str):
        """(launches, total ms) of one kind since timing was enabled or last read."""
        n = ctypes.c_uint64(0)
        ms = ctypes.c_double(0.0)
        self._check(lib().stage_timing_read(self._h, KERNEL_KINDS[kind], ctypes.byref(n), ctypes.byref(ms)),
                    "stage_timing_read")
        return int(n.value), float(ms.value)


def _status(rc: int, what: str):
    if rc != STAGE_OK:
        raise StageError(rc, f"{what}: {lib().stage_status_str(rc).decode()}")


def greedy(logits: torch.Tensor, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """int32 [n] = argmax of each row of F32 logits [n, V] (lowest index on ties), on the GPU."""
    n, v = logits.shape
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device=logits.device)
    _status(lib().stage_greedy(n, v, _ptr(logits.contiguous()), _ptr(out), _stream(stream)), "stage_greedy")
    return out


def pipeline_generate(stages: list, prompts: torch.Tensor, n_new: int, streams=None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Greedy generation through the ordered stages with micro-batches in flight (include/pipeline.h).

    prompts: int32 [n_micro, rows, prompt_len] on the stages' device; returns int32
    [n_micro, n_new, rows].  streams: one torch.cuda.Stream per stage, or None for the default
    stream.  Returns after the run completes."""
    n_micro, rows, plen = prompts.shape
    cfg = GenCfg(n_micro, rows, plen, n_new)
    handles = (_vp * len(stages))(*[s._h.value for s in stages])
    nbytes = ctypes.c_uint64(0)
    _status(lib().stage_pipeline_workspace(handles, len(stages), ctypes.byref(cfg), ctypes.byref(nbytes)),
            "stage_pipeline_workspace")
    if workspace is None or workspace.numel() < nbytes.value:
        workspace = torch.empty(int(nbytes.value), dtype=torch.uint8, device=prompts.device)
    out = torch.empty((n_micro, n_new, rows), dtype=torch.int32, device=prompts.device)
    sarr = None
    if streams is not None:
        sarr = (_vp * len(stages))(*[_stream(s) for s in streams])
    _status(lib().stage_pipeline_generate(handles, len(stages), ctypes.byref(cfg), _ptr(prompts.contiguous()),
                                          _ptr(out), _ptr(workspace), int(workspace.numel()), sarr),
            "stage_pipeline_generate")
    return out
