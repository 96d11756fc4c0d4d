#!/usr/bin/env python3
"""Benchmark of one pipeline stage's decoder forward on one MI355X.

Workload (default): the 70B-shaped middle stage -- blocks 20..39 of an 80-block decoder (d 8192,
64 q / 8 KV heads, head dim 128, SwiGLU 28672), seeded synthetic bf16 weights N(0, 0.02), binary16
KV cache.  One step = one 4096-token prefill chunk (a fresh sequence) plus one batched decode step of
128 rows at context 8192 (slots filled by two 4096-token prefill chunks and copies).

Prints ONE JSON line.  `value` is the decode throughput (tokens/s, inputs resident in HBM); the
line also carries the prefill throughput, the dominant kernel's roofline (the prefill gate/up GEMM:
algorithmic flops per launch / its average duration, timed live with HIP events on the launch stream
over the timed region), the decode attention kernel's HBM roofline, the CPU oracle timed on this
host's cores over a bounded sample, and the 8B-shaped first stage's figures (prefill 512, decode to
2048, batch 1) under "first_8b".
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def fill_weights(st, shape, blocks, first, last, seed, gain_sigma=0.0):
    """Draw every weight tensor of the stage on the GPU and load it (device-to-device copies)."""
    import torch

    import fixtures as fx

    roles = fx.stage_roles(blocks[0], blocks[1], first, last)
    biggest = max(int(__import__("numpy").prod(fx.role_shape(shape, r))) for r, _ in roles)
    scratch = torch.empty(biggest, dtype=torch.int16, device="cuda")
    for role, b in roles:
        n = int(__import__("numpy").prod(fx.role_shape(shape, role)))
        t = scratch[:n]
        if role in fx.GAIN_ROLES:
            fx.gain_bf16_gpu(t, seed, fx.weight_stream(role, b), gain_sigma)
        else:
            fx.normal_bf16_gpu(t, seed, fx.weight_stream(role, b), 0.02)
        st.load_weight(role, b, t)
    torch.cuda.synchronize()
    del scratch


def cpu_threads() -> int:
    """Threads the oracle's numpy calls use on this host (the BLAS pool), else the core count."""
    try:
        from threadpoolctl import threadpool_info
        return max([int(i.get("num_threads", 1)) for i in threadpool_info()] or [os.cpu_count()])
    except Exception:  # pragma: no cover
        return os.cpu_count()


def cpu_model() -> str:
    """The host CPU's model name (first 'model name' line of /proc/cpuinfo), or 'unknown'."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


GEMV_SOURCES = ("pipeline_stage_decoder_amd/csrc/kernels_gemv.hip", "pipeline_stage_decoder_amd/csrc/common.h",
                "pipeline_stage_decoder_amd/csrc/norm.h")
GEMM_SOURCES = ("pipeline_stage_decoder_amd/csrc/kernels_gemm.hip", "pipeline_stage_decoder_amd/csrc/common.h",
                "pipeline_stage_decoder_amd/csrc/norm.h")
COUNTER_FILE = os.path.join(ROOT, "profiles", "decode_gemv_gateup_8b_counters.txt")
GEMM_COUNTER_FILE = os.path.join(ROOT, "profiles", "prefill_gemm_gateup_70b_traffic_counters.txt")


def source_hash(sources) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(path: str, kernel: str, sources):
    """HBM bytes per launch of a kernel from a committed counter summary: its FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch) scaled by what the same counters read for a plain 1 GiB copy.
    None when the summary is missing or was taken on another version of the kernel's sources."""
    try:
        kv = dict(line.split(":", 1) for line in open(path) if ":" in line and not line.startswith("#"))
        kv = {k.strip(): v.strip() for k, v in kv.items()}
        if kv.get("kernel_source_sha256_16") != source_hash(sources):
            return None
        fetch = float(kv[f"{kernel}_fetch_kib"]) * 1048576.0 / float(kv["copy_fetch_kib"])
        write = float(kv[f"{kernel}_write_kib"]) * 1048576.0 / float(kv["copy_write_kib"])
        return round((fetch + write) * 1024.0)
    except (OSError, KeyError, ValueError):
        return None


def summarize_rocprof(path: str, top: int = 12) -> None:
    """Print a short text summary of rocprofv3 CSV output under `path`: kernel statistics (calls,
    average and total duration) and, for counter runs, each counter's mean value per dispatch by
    kernel."""
    import csv
    import glob
    stats = glob.glob(os.path.join(path, "**", "*kernel_stats.csv"), recursive=True)
    for f in stats:
        rows = list(csv.DictReader(open(f)))
        rows.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
        print(f"# kernel statistics ({os.path.basename(f)}): name | calls | avg us | total ms | %")
        for r in rows[:top]:
            print(f"{r['Name'][:110]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['TotalDurationNs']) / 1e6:.2f} | {float(r.get('Percentage', 0)):.1f}")
    # one template can serve several launch shapes (the prefill and batched-decode projections share
    # their GEMM tile): the heaviest kernels again, per grid size, from the per-dispatch trace
    for f in glob.glob(os.path.join(path, "**", "*kernel_trace.csv"), recursive=True):
        agg = {}
        for r in csv.DictReader(open(f)):
            grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
            a = agg.setdefault((r["Kernel_Name"][:110], grid), [0, 0])
            a[0] += 1
            a[1] += int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        print(f"# per launch shape ({os.path.basename(f)}): name | grid (work-items x, y, z) | calls | avg us | "
              "total ms")
        for (k, grid), (n, ns) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:2 * top]:
            print(f"{k} | {grid} | {n} | {ns / n / 1e3:.2f} | {ns / 1e6:.2f}")
    for f in glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True):
        agg = {}
        for r in csv.DictReader(open(f)):
            key = (r["Kernel_Name"][:110], r["Counter_Name"])
            a = agg.setdefault(key, [0, 0.0])
            a[0] += 1
            a[1] += float(r["Counter_Value"])
        print(f"# counters ({os.path.basename(f)}): kernel | counter | dispatches | mean per dispatch")
        for (k, c), (n, v) in sorted(agg.items(), key=lambda kv: -kv[1][1])[:4 * top]:
            print(f"{k} | {c} | {n} | {v / n:.1f}")
        # MFMA utilisation (busy cycles over GPU-active cycles x SIMDs) and bf16 MFMA flops issued;
        # GRBM_GUI_ACTIVE arrives summed over the 8 XCDs (8x the dispatch's wall-clock cycles)
        kernels = sorted({k for k, _ in agg})
        simds = 256 * 4 / 8
        lines = []
        for k in kernels:
            busy, act = agg.get((k, "SQ_VALU_MFMA_BUSY_CYCLES")), agg.get((k, "GRBM_GUI_ACTIVE"))
            mops = agg.get((k, "SQ_INSTS_VALU_MFMA_MOPS_BF16"))
            if busy and act and act[1] > 0:
                lines.append((busy[1] / (act[1] * simds), k, act[0], (mops[1] * 512 / mops[0]) if mops else 0.0))
        if lines:
            print("# derived: kernel | dispatches | MFMA busy / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs) | "
                  "bf16 MFMA flops per dispatch")
            for u, k, n, fl in sorted(lines, key=lambda t: -t[3]):
                print(f"{k} | {n} | {100 * u:.1f}% | {fl:.4g}")


def time_handoff(rows_prefill, rows_decode, reps: int = 20, cold_bytes: int = 768 << 20) -> dict:
    """The stage boundary's cost: the F32 hidden rows a stage hands to the next, copied device to
    device (the one-GPU handoff) from sources rotated through more than `cold_bytes` of memory --
    past the 256 MB memory-side cache, so every copy reads HBM -- and as a pinned device->host->
    device round trip (the host-staged transfer of two stages on two PCIe-attached GPUs)."""
    import torch
    out = {}
    for name, src in (("prefill_rows", rows_prefill), ("decode_rows", rows_decode)):
        nbytes = src.numel() * 4
        srcs = [src.clone() for _ in range(max(2, -(-cold_bytes // nbytes)))]
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(srcs[0])
        torch.cuda.synchronize()
        e0.record()
        for i in range(reps):
            dst.copy_(srcs[i % len(srcs)])
        e1.record()
        torch.cuda.synchronize()
        out[f"d2d_{name}"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
        del srcs
        host = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
        host.copy_(src)
        dst.copy_(host)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            host.copy_(src)                 # synchronous D2H into pinned memory
            dst.copy_(host)
            torch.cuda.synchronize()
        out[f"pinned_round_trip_{name}"] = round((time.perf_counter() - t0) * 1e6 / reps, 2)
        out[f"bytes_{name}"] = nbytes
    return out


def counter_pass(shape, blocks, T, dev, n_dec: int = 32, kv: str = "f16"):
    """The workload's kernels for a hardware-counter run: one prefill of T tokens, then n_dec eager
    B = 1 decode steps, no timing events; progress every 8 steps."""
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd.stage import Stage

    st = Stage(shape, blocks[0], blocks[1], True, False, max_slots=1, max_ctx=T + n_dec, max_tokens=T, device=0,
               kv=kv)
    fill_weights(st, shape, blocks, True, False, fx.SEED_WEIGHTS)
    prompt = fx.tokens_gpu(torch.empty(T, dtype=torch.int32, device=dev), fx.SEED_TOKENS, fx.token_stream(0),
                           shape.vocab)
    toks = fx.tokens_gpu(torch.empty(n_dec, dtype=torch.int32, device=dev), fx.SEED_TOKENS, fx.token_stream(1),
                         shape.vocab)
    pos = torch.arange(T, T + n_dec, dtype=torch.int32, device=dev)
    slot0 = torch.zeros(1, dtype=torch.int32, device=dev)
    x = st.prefill(st.embed(prompt), 0, 0)
    torch.cuda.synchronize()
    log("[bench] counters: prefill done")
    x1 = torch.empty((1, shape.d_model), dtype=torch.float32, device=dev)
    for i in range(n_dec):
        st.embed(toks[i:i + 1], out=x1)
        st.decode(x1, slot0, pos[i:i + 1], out=x1)
        if i % 8 == 7:
            torch.cuda.synchronize()
            log(f"[bench] counters: decode step {i + 1}/{n_dec}")
    print(json.dumps({"phase": "counters", "prefill_tokens": T, "decode_steps": n_dec}), flush=True)


def prefill_only(args, shape, blocks, T, dev, stream, first=True):
    """Time the prefill alone: stage sized for one T-token prompt, W warmups then K timed prefills.
    A first stage embeds seeded tokens; any other stage takes seeded F32 N(0,1) hidden rows."""
    import numpy as np
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd import accounting as acc
    from pipeline_stage_decoder_amd.stage import Stage

    st = Stage(shape, blocks[0], blocks[1], first, False, max_slots=1, max_ctx=T, max_tokens=T, device=0,
               kv=args.kv)
    fill_weights(st, shape, blocks, first, False, fx.SEED_WEIGHTS)
    xin = torch.empty((T, shape.d_model), dtype=torch.float32, device=dev)
    hout = torch.empty_like(xin)
    if first:
        prompt = fx.tokens_gpu(torch.empty(T, dtype=torch.int32, device=dev), fx.SEED_TOKENS,
                               fx.token_stream(0), shape.vocab)
    else:
        fx.normal_f32_gpu(xin, fx.SEED_HIDDEN, fx.hidden_stream(0), 0)

    def run():
        if first:
            st.embed(prompt, out=xin)
        st.prefill(xin, 0, 0, out=hout)

    for _ in range(max(args.warmup, 1)):
        run()
    torch.cuda.synchronize()
    ms = []
    for k in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        log(f"[bench] prefill {k + 1}/{args.steps}: {ms[-1]:.3f} ms")
    pre_ms = float(np.median(ms))
    flops = acc.prefill_flops(shape, blocks[1] - blocks[0], T)
    print(json.dumps({"phase": "prefill", "prefill_tokens": T, "blocks": list(blocks),
                      "kv_cache": args.kv, "prefill_ms": round(pre_ms, 3),
                      "prefill_tok_s": round(T / (pre_ms / 1e3), 1),
                      "prefill_tflops": round(flops / (pre_ms / 1e3) / 1e12, 1),
                      "prefill_mfma_frac": round(flops / (pre_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}),
          flush=True)


def stage_kernel_ms(st, kinds):
    """(launches, total ms) per kind from the stage's HIP-event timing, then timing switched off."""
    out = {k: st.timing_read(k) for k in kinds}
    st.timing([])
    return out


def graph_of(fn, n: int):
    """Capture n calls of fn() into one HIP graph (fn is warmed once outside capture)."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    with torch.cuda.graph(g, stream=cs):
        for _ in range(n):
            fn()
    torch.cuda.synchronize()
    return g


def time_graph(g, reps: int) -> float:
    """Median ms of one replay of g over `reps` replays (events on the current stream)."""
    import numpy as np
    import torch
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
    return float(np.median(ms))


def fill_kv_by_prefill(st, slot0: int, n_pos: int, chunk: int, other_slots, d: int):
    """Fill slot0's cache with n_pos positions by chunked prefill of seeded F32 N(0,1) hidden rows,
    then copy it into the other slots (the decode rows then attend real, distinct-slot caches)."""
    import torch

    import fixtures as fx
    x = torch.empty((chunk, d), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for p0 in range(0, n_pos, chunk):
        t = min(chunk, n_pos - p0)
        fx.normal_f32_gpu(x[:t], fx.SEED_HIDDEN, fx.hidden_stream(slot0), p0 * d)
        st.prefill(x[:t], slot0, p0, out=y[:t])
    torch.cuda.synchronize()
    for i, s in enumerate(other_slots):
        st.kv_copy(slot0, s, n_pos)
        if i % 16 == 15:
            torch.cuda.synchronize()
            log(f"[bench] KV copied into {i + 1}/{len(other_slots)} slots")
    torch.cuda.synchronize()


def kernel_roofline(bytes_per_launch: int, launches: int, total_ms: float, name: str) -> dict:
    avg_s = total_ms / 1e3 / max(launches, 1)
    ach = bytes_per_launch / avg_s / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None, "kernel": name,
            "bytes_per_launch": bytes_per_launch, "avg_launch_us": round(avg_s * 1e6, 2), "launches": launches}


def batched_decode_line(args, workload: str, shape, blocks, first: bool, last: bool, B: int, ctx: int,
                        prefill_chunk: int, time_prefill: bool) -> dict:
    """B rows (distinct slots) decoding at context ctx (positions ctx), every step the same positions
    (each step rewrites position ctx): per-step bytes are constant, as in the workload's definition."""
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd import accounting as acc
    from pipeline_stage_decoder_amd.stage import Stage

    nb = blocks[1] - blocks[0]
    d = shape.d_model
    log(f"[bench] {workload}: creating stage {blocks}, {B} slots, ctx {ctx}")
    st = Stage(shape, blocks[0], blocks[1], first, last, max_slots=B, max_ctx=ctx + 1,
               max_tokens=max(B, prefill_chunk), device=0, kv=args.kv)
    kvb = 4 if args.kv == "f32" else 2
    fill_weights(st, shape, blocks, first, last, fx.SEED_WEIGHTS)
    pre = {}
    if time_prefill:
        # the fill itself is the prefill workload: chunks of prefill_chunk tokens at pos0 = 0, chunk, ..
        x = torch.empty((prefill_chunk, d), dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)
        ms = []
        for p0 in range(0, ctx, prefill_chunk):
            fx.normal_f32_gpu(x, fx.SEED_HIDDEN, fx.hidden_stream(0), p0 * d)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            st.prefill(x, 0, p0, out=y)
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
            fl = acc.prefill_flops(shape, nb, prefill_chunk, pos0=p0)
            log(f"[bench] prefill chunk at pos0 {p0}: {ms[-1]:.1f} ms, {fl / ms[-1] / 1e9:.1f} TFLOP/s")
        tot_fl = sum(acc.prefill_flops(shape, nb, prefill_chunk, pos0=p0) for p0 in range(0, ctx, prefill_chunk))
        pre = {"prefill_chunk": prefill_chunk, "prefill_chunk_ms": [round(m, 2) for m in ms],
               "prefill_tok_s": round(ctx / (sum(ms) / 1e3), 1),
               "prefill_tflops": round(tot_fl / (sum(ms) / 1e3) / 1e12, 1),
               "prefill_mfma_frac": round(tot_fl / (sum(ms) / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        for i, s in enumerate(range(1, B)):
            st.kv_copy(0, s, ctx)
            if i % 16 == 15:
                torch.cuda.synchronize()
                log(f"[bench] KV copied into {i + 1}/{B - 1} slots")
        torch.cuda.synchronize()
    else:
        fill_kv_by_prefill(st, 0, ctx, prefill_chunk, range(1, B), d)

    xin = fx.normal_f32_gpu(torch.empty((B, d), dtype=torch.float32, device="cuda"), fx.SEED_HIDDEN,
                            fx.hidden_stream(1000), 0)
    h = torch.empty_like(xin)
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    pos = torch.full((B,), ctx, dtype=torch.int32, device="cuda")
    logits = torch.empty((B, shape.vocab), dtype=torch.float32, device="cuda") if last else None

    def step():
        st.decode(xin, slots, pos, out=h)
        if last:
            st.readout(h, logits=logits)

    per_graph = 4
    g = graph_of(step, per_graph)
    for _ in range(args.warmup):
        g.replay()
    torch.cuda.synchronize()
    reps = max(args.steps, 1)
    ms = time_graph(g, reps) / per_graph
    kinds = ("qkv", "attn", "o", "gateup", "down") + (("readout",) if last else ())
    st.timing(list(kinds))
    step()
    torch.cuda.synchronize()
    kt = stage_kernel_ms(st, kinds)
    step_bytes = acc.decode_step_bytes(shape, nb, [ctx] * B, first=first, last=last, kv_elem_bytes=kvb)
    kv_launch = B * (ctx + 1) * acc.kv_bytes_per_token_block(shape, kvb)
    roof = kernel_roofline(kv_launch, kt["attn"][0], kt["attn"][1],
                           f"k_attn_decode + k_attn_merge (split-KV GQA decode over the slots' {args.kv} caches)")
    gbs = step_bytes / (ms / 1e3) / 1e9
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] {workload}: timing the CPU oracle on a bounded sample (one block)")
        cpu = cpu_baseline_block(shape, args.kv, blocks[0], nb, prefill_chunk, B, ctx, last=last)
    return {
        "metric": "stage decode tok/s & HBM GB/s %peak; prefill tok/s & MFMA util",
        "value": round(B / (ms / 1e3), 1), "unit": "tok/s", "n_gpus": 1, "steps": reps * per_graph,
        "warmup": args.warmup * per_graph, "ms_per_step": round(ms, 3), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights, F32 N(0,1) hidden rows",
        "config": {"workload": workload, "batch": B, "decode_ctx": ctx, "blocks": list(blocks),
                   "kv_cache": args.kv, "decode_graph": True},
        "decode_step_bytes": step_bytes, "decode_hbm_gbs": round(gbs, 1),
        "decode_hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
        "kernel_ms_per_step": {k: round(v[1], 3) for k, v in kt.items()},
        **pre, "roofline": roof, "cpu_baseline": cpu,
    }


def mlp_slices_line(args) -> dict:
    """8 column/row slices (width 3584) of a d 8192 / F 28672 SwiGLU MLP, one stage block each;
    stage_mlp per slice, accumulated in slice order, at T in {1, 64, 4096}."""
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd import accounting as acc
    from pipeline_stage_decoder_amd.stage import Stage

    s70 = fx.LLAMA70B
    n_sl, width = 8, s70.d_ffn // 8
    sh = fx.Shape(s70.d_model, s70.n_q_heads, s70.n_kv_heads, s70.head_dim, width, s70.vocab, n_sl)
    st = Stage(sh, 0, n_sl, False, False, max_slots=1, max_ctx=64, max_tokens=4096, device=0)
    roles = [r for r in fx.stage_roles(0, n_sl, False, False) if r[0] in ("mlp_norm", "wgate", "wup", "wdown")]
    big = max(int(__import__("numpy").prod(fx.role_shape(sh, r))) for r, _ in roles)
    scratch = torch.empty(big, dtype=torch.int16, device="cuda")
    for role, b in roles:
        n = int(__import__("numpy").prod(fx.role_shape(sh, role)))
        if role == "mlp_norm":
            fx.gain_bf16_gpu(scratch[:n], fx.SEED_WEIGHTS, fx.weight_stream(role, b), 0.0)
        else:
            fx.normal_bf16_gpu(scratch[:n], fx.SEED_WEIGHTS, fx.weight_stream(role, b), 0.02)
        st.load_weight(role, b, scratch[:n])
    torch.cuda.synchronize()
    del scratch
    per_T = {}
    for T in (1, 64, 4096):
        x = fx.normal_f32_gpu(torch.empty((T, sh.d_model), dtype=torch.float32, device="cuda"), fx.SEED_HIDDEN,
                              fx.hidden_stream(40), 0)
        acc_out = torch.empty_like(x)

        def run():
            for i in range(n_sl):
                st.mlp(i, x, out=acc_out, accumulate=i > 0)

        g = graph_of(run, 1)
        ms = time_graph(g, max(args.steps, 3)) / n_sl
        by = acc.mlp_slice_bytes(sh.d_model, width, T)
        fl = acc.mlp_slice_flops(sh.d_model, width, T)
        per_T[str(T)] = {"us_per_slice": round(ms * 1e3, 2), "hbm_gbs": round(by / (ms / 1e3) / 1e9, 1),
                         "hbm_frac": round(by / (ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                         "tflops": round(fl / (ms / 1e3) / 1e12, 1),
                         "mfma_frac": round(fl / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)}
        log(f"[bench] MLP slice T={T}: {per_T[str(T)]}")
    big_t = per_T["4096"]
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] MLP slices: timing the CPU oracle at T = 64")
        cpu = cpu_baseline_mlp_slices(sh, n_sl, 64)
    return {
        "metric": "stage decode tok/s & HBM GB/s %peak; prefill tok/s & MFMA util",
        "value": round(4096 / (big_t["us_per_slice"] * n_sl / 1e6), 1), "unit": "tok/s", "n_gpus": 1,
        "steps": max(args.steps, 3), "warmup": 1, "ms_per_step": round(big_t["us_per_slice"] * n_sl / 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights, F32 N(0,1) hidden rows",
        "config": {"workload": "sharded-MLP slices: d 8192, 8 slices of width 3584 (F 28672), "
                               "T in {1, 64, 4096}, F32 partials summed in slice order; value = "
                               "T=4096 rows/s through all 8 slices"},
        "per_T": per_T, "roofline": None, "cpu_baseline": cpu,
    }


def attn_parallel_line(args) -> dict:
    """The parallel attention and vocabulary layouts on one GPU, at the 8B shape ("41. Many GPUs":
    Tensor parallelism, Ring attention): one block's attention sublayer over a 4096-token sequence
    taken plainly and the ring way (n ranks' query chunks, the K/V chunks passed round the ring,
    partials merged by log-sum-exp; zigzag chunks for causal balance); the sublayer over 8 head
    slices summed in slice order against the full one (T = 512 and T = 1); the readout over 8
    vocabulary slices against the full one (64 rows)."""
    import numpy as np
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd.stage import Stage

    s, T, n = fx.LLAMA8B, 4096, 8
    d, hq, hkv, dh, V = s.d_model, s.n_q_heads, s.n_kv_heads, s.head_dim, s.vocab
    reps = max(args.steps, 3)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms))

    def gpu_weight(role, shape, sigma=0.02):
        t = torch.empty(int(np.prod(shape)), dtype=torch.int16, device="cuda")
        if role in fx.GAIN_ROLES:
            fx.gain_bf16_gpu(t, fx.SEED_WEIGHTS, fx.weight_stream(role, 0), 0.1)
        else:
            fx.normal_bf16_gpu(t, fx.SEED_WEIGHTS, fx.weight_stream(role, 0), sigma)
        return t.view(*shape)

    w = {r: gpu_weight(r, fx.role_shape(s, r)) for r in ("attn_norm", "wq", "wk", "wv", "wo")}
    st = Stage(s, 0, 1, False, False, max_slots=2, max_ctx=T, max_tokens=T, device=0, kv=args.kv)
    for r, t in w.items():
        st.load_weight(r, 0, t)
    x = fx.normal_f32_gpu(torch.empty((T, d), dtype=torch.float32, device="cuda"), fx.SEED_HIDDEN,
                          fx.hidden_stream(60), 0)
    proj = 2 * d * ((hq + 2 * hkv) * dh + hq * dh)

    def sub_flops(t):
        return proj * t + 4 * hq * dh * t * (t + 1) // 2

    log("[bench] attn-parallel: plain and ring attention over 4096 tokens")
    res = {"T": T, "plain_ms": timed(lambda: st.attn(0, x, 0, 0))}
    for ranks, zz in ((4, True), (8, False)):
        res[f"ring_{ranks}{'_zigzag' if zz else ''}_ms"] = timed(lambda: st.attn_ring(0, x, 1, ranks, zz))
    fl = sub_flops(T)
    for k in [k for k in res if k.endswith("_ms")]:
        res[k.replace("_ms", "_tflops")] = round(fl / (res[k] / 1e3) / 1e12, 1)
        res[k] = round(res[k], 3)

    log("[bench] attn-parallel: 8 head slices against the full sublayer")
    hq_s, hk_s = hq // n, max(hkv // n, 1)
    sh = fx.Shape(d, hq_s, hk_s, dh, 64, V, n)
    sl = Stage(sh, 0, n, False, False, max_slots=1, max_ctx=512, max_tokens=512, device=0, kv=args.kv)
    for i in range(n):
        qr = slice(i * hq_s * dh, (i + 1) * hq_s * dh)
        kr = slice((i * hkv // n) * dh, (i * hkv // n + hk_s) * dh)
        sl.load_weight("attn_norm", i, w["attn_norm"])
        sl.load_weight("wq", i, w["wq"][qr].contiguous())
        sl.load_weight("wk", i, w["wk"][kr].contiguous())
        sl.load_weight("wv", i, w["wv"][kr].contiguous())
        sl.load_weight("wo", i, w["wo"][:, qr].contiguous())
    heads = {}
    for t in (512, 1):
        xt = x[:t].contiguous()
        acc_out = torch.empty_like(xt)

        def slices():
            for i in range(n):
                sl.attn(i, xt, 0, 0, out=acc_out, accumulate=i > 0)

        heads[str(t)] = {"full_us": round(timed(lambda: st.attn(0, xt, 0, 0)) * 1e3, 1),
                         "slices_us": round(timed(slices) * 1e3, 1)}
    res["head_slices"] = heads

    log("[bench] attn-parallel: 8 vocabulary slices against the full readout")
    per = (V + n - 1) // n
    ro = gpu_weight("readout", (V, d))
    fn_ = gpu_weight("final_norm", (d,))
    full = Stage(s, 0, 0, False, True, max_slots=1, max_ctx=64, max_tokens=64, device=0)
    full.load_weight("final_norm", -1, fn_)
    full.load_weight("readout", -1, ro)
    vs = []
    for i in range(n):
        lo, hi = i * per, min(V, (i + 1) * per)
        part = torch.zeros((per, d), dtype=torch.int16, device="cuda")
        part[:hi - lo] = ro[lo:hi]
        stv = Stage(fx.Shape(d, hq, hkv, dh, 64, per, 0), 0, 0, False, True, max_slots=1, max_ctx=64,
                    max_tokens=64, device=0)
        stv.load_weight("final_norm", -1, fn_)
        stv.load_weight("readout", -1, part)
        vs.append(stv)
    h = x[:64].contiguous()
    full_ms = timed(lambda: full.readout(h, want_normed=False))
    slice_ms = timed(lambda: [v.readout(h, want_normed=False) for v in vs])
    by = V * d * 2
    res["vocab_slices_64_rows"] = {"full_us": round(full_ms * 1e3, 1), "slices_us": round(slice_ms * 1e3, 1),
                                   "full_hbm_gbs": round(by / (full_ms / 1e3) / 1e9, 1),
                                   "slices_hbm_gbs": round(by / (slice_ms / 1e3) / 1e9, 1)}
    log(f"[bench] attn-parallel: {res}")
    ring = res["ring_4_zigzag_ms"]
    return {
        "metric": "stage decode tok/s & HBM GB/s %peak; prefill tok/s & MFMA util",
        "value": round(T / (ring / 1e3), 1), "unit": "tok/s", "n_gpus": 1, "steps": reps, "warmup": 1,
        "ms_per_step": ring, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights, F32 N(0,1) hidden rows",
        "config": {"workload": "8B-shaped block 0, attention sublayer over 4096 tokens taken the ring way "
                               "(4 ranks' zigzag chunks on one GPU) against the plain sublayer and 8 ranks' "
                               "plain chunks; 8 head slices (T = 512, 1) and 8 vocabulary slices of the "
                               "readout (64 rows) against the full ones; value = tokens/s through the "
                               "4-rank zigzag ring"},
        "results": res, "roofline": None, "cpu_baseline": None,
    }


def placement_line(args) -> dict:
    """The placement planner (include/placement.h) on representative budgets, host only: the
    contiguous cuts, each device's requirement and the planner's time; a budget nothing fits in
    reports the typed does-not-fit status."""
    import fixtures as fx
    from pipeline_stage_decoder_amd.stage import StageError, place

    gib = 1 << 30
    cases = [("8B (32 blocks), 2 x 24 GiB", fx.LLAMA8B, [24 * gib] * 2),
             ("8B, 24 + 12 GiB", fx.LLAMA8B, [24 * gib, 12 * gib]),
             ("8B, 2 x 4 GiB", fx.LLAMA8B, [4 * gib] * 2),
             ("70B-shaped (80 blocks), 2 x 80 GiB", fx.LLAMA70B, [80 * gib] * 2),
             ("70B-shaped, 8 x 288 GiB", fx.LLAMA70B, [288 * gib] * 8)]
    out = []
    for name, shp, budgets in cases:
        t0 = time.perf_counter()
        try:
            cuts, req = place(shp, budgets, max_slots=1, max_ctx=4096, max_tokens=512)
            r = {"cuts": cuts, "required_gib": [round(x / gib, 2) for x in req]}
        except StageError as e:
            r = {"status": str(e)}
        r["plan_ms"] = round((time.perf_counter() - t0) * 1e3, 2)
        r["case"] = name
        out.append(r)
        log(f"[bench] placement {r}")
    return {"metric": "placement plan", "value": None, "unit": None, "n_gpus": 0, "steps": 1, "warmup": 0,
            "ms_per_step": round(sum(r["plan_ms"] for r in out), 2), "higher_is_better": False,
            "scaling": "weak", "vs_baseline": None, "dtype": "none", "data": "model shapes only",
            "config": {"workload": "placement planner: 1 slot, ctx 4096, 512 prefill tokens per stage"},
            "plans": out, "roofline": None, "cpu_baseline": None}


def pipeline_line(args) -> dict:
    """The whole 8B-shaped model as two stages on this GPU ([0, 16) + embedding, [16, 32) + final
    norm + readout), greedy generation through stage_pipeline_generate: two micro-batches of one
    sequence each, on two streams (in flight together) and on one stream (one batch in flight),
    plus the same two sequences as one batch of two rows for reference."""
    import numpy as np
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd import stage as S

    shape = fx.LLAMA8B
    plen, n_new = 128, 128
    stages = [S.Stage(shape, 0, 16, True, False, max_slots=2, max_ctx=plen + n_new, max_tokens=plen, device=0,
                      kv=args.kv),
              S.Stage(shape, 16, 32, False, True, max_slots=2, max_ctx=plen + n_new, max_tokens=plen, device=0,
                      kv=args.kv)]
    fill_weights(stages[0], shape, (0, 16), True, False, fx.SEED_WEIGHTS)
    fill_weights(stages[1], shape, (16, 32), False, True, fx.SEED_WEIGHTS)
    prompts = torch.stack([fx.tokens_gpu(torch.empty(plen, dtype=torch.int32, device="cuda"), fx.SEED_TOKENS,
                                         fx.token_stream(30 + i), shape.vocab) for i in range(2)])
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    modes = {"two_micro_batches_two_streams": (prompts.view(2, 1, plen), streams),
             "two_micro_batches_one_stream": (prompts.view(2, 1, plen), None),
             "one_batch_of_two_rows": (prompts.view(1, 2, plen), None)}
    res, toks = {}, {}
    for name, (p, st) in modes.items():
        S.pipeline_generate(stages, p, 4, streams=st)                # warm-up (short)
        torch.cuda.synchronize()
        times = []
        for _ in range(max(args.steps, 1)):
            t0 = time.perf_counter()
            out = S.pipeline_generate(stages, p, n_new, streams=st)
            times.append(time.perf_counter() - t0)
        t = float(np.median(times))
        toks[name] = out.cpu().numpy().transpose(0, 2, 1).reshape(-1, n_new)     # [sequence, token]
        res[name] = {"s": round(t, 4), "tok_s": round(2 * n_new / t, 1)}
        log(f"[bench] pipeline {name}: {res[name]}")
    seq = toks["two_micro_batches_one_stream"]
    same_pipe = bool(np.array_equal(toks["two_micro_batches_two_streams"], seq))
    # B = 2 decode takes other kernels (two-row GEMV, 256-key split-KV chunks instead of 128), so
    # its rounding differs and greedy choices may part after a near-tie
    same_batched = int((toks["one_batch_of_two_rows"] == seq).all(axis=0).sum())
    speedup = res["two_micro_batches_one_stream"]["s"] / res["two_micro_batches_two_streams"]["s"]
    return {
        "metric": "stage decode tok/s & HBM GB/s %peak; prefill tok/s & MFMA util",
        "value": res["two_micro_batches_two_streams"]["tok_s"], "unit": "tok/s", "n_gpus": 1,
        "steps": max(args.steps, 1), "warmup": 1, "ms_per_step": round(res["two_micro_batches_two_streams"]["s"] * 1e3, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights, uniform tokens",
        "config": {"workload": "8B-shaped model (32 blocks) as two pipeline stages on one GPU; greedy generation of "
                               f"2 sequences, {plen}-token prompts, {n_new} new tokens each (prefill + decode, "
                               "wall clock of the whole run)"},
        "modes": res, "bubble_speedup": round(speedup, 3), "tokens_pipelined_equal_sequential": same_pipe,
        "batched_tokens_agreeing_with_sequential": f"{same_batched} of {n_new} positions",
        "roofline": None, "cpu_baseline": None,
    }


def tiny_line(args) -> dict:
    """The tiny decoder (2 blocks, d 256, 4 q / 2 KV heads, Dh 64, F 688, vocab 1024) as two stages
    on this GPU ([0, 1) + embedding, [1, 2) + final norm + readout): greedy generation of 8 tokens
    from a 16-token prompt through stage_pipeline_generate, timed whole (median of --steps runs),
    and the time of one decode step through both stages from the difference between 8-token and
    1-token runs.  Its weights total under 4 MB, so it is bound by kernel launches, not by HBM or
    the matrix cores, and carries no roofline.  The oracle runs the same generation on the host,
    timed whole, and its tokens must equal the GPU's."""
    import numpy as np
    import torch

    import fixtures as fx
    from oracle import decoder as o
    from pipeline_stage_decoder_amd import stage as S

    shape = fx.TINY
    plen, n_new, ctx = 16, 8, 64
    w = fx.draw_stage_weights(shape, 0, 2, True, True, gain_sigma=0.1)
    parts = ((0, 1, True, False), (1, 2, False, True))
    stages = []
    for b0, b1, first, last in parts:
        st = S.Stage(shape, b0, b1, first, last, max_slots=1, max_ctx=ctx, max_tokens=plen, device=0, kv=args.kv)
        for (role, blk), t in w.items():
            if (role == "embed" and not first) or (role in ("final_norm", "readout") and not last):
                continue
            if blk >= 0 and not (b0 <= blk < b1):
                continue
            st.load_weight(role, blk, t)
        stages.append(st)
    prompt = np.asarray(fx.tokens(fx.SEED_TOKENS, fx.token_stream(0), plen, shape.vocab), np.int32)
    p = torch.tensor(prompt, device="cuda").view(1, 1, plen)

    def median_run(n):
        for _ in range(max(args.warmup, 1)):
            S.pipeline_generate(stages, p, n)
        times, out = [], None
        for _ in range(max(args.steps, 3)):
            t0 = time.perf_counter()
            out = S.pipeline_generate(stages, p, n)
            times.append(time.perf_counter() - t0)
        return float(np.median(times)), out

    t_all, out = median_run(n_new)
    t_one, _ = median_run(1)
    got = out.cpu().numpy().reshape(-1)
    step_us = (t_all - t_one) / (n_new - 1) * 1e6
    log(f"[bench] tiny: {t_all * 1e6:.0f} us for {n_new} tokens, {step_us:.0f} us per decode step")

    cpu = None
    if not args.no_cpu_baseline:
        ost = [o.Stage(o.Dims.of(shape), b0, b1, first, last, w, ctx, kv_dtype=args.kv)
               for b0, b1, first, last in parts]
        t0 = time.perf_counter()
        want, _ = o.generate(ost, prompt, n_new)
        t_cpu = time.perf_counter() - t0
        cpu = {"value": round(n_new / t_cpu, 2), "unit": "tok/s", "cores": cpu_threads(), "kind": "oracle",
               "sample": f"the whole generation ({plen}-token prompt, {n_new} tokens through both stages), "
                         f"timed once: {t_cpu:.3f} s",
               "tokens_equal_gpu": bool(np.array_equal(want, got)), "cpu_model": cpu_model()}
    return {
        "metric": "stage decode tok/s & HBM GB/s %peak; prefill tok/s & MFMA util",
        "value": round(n_new / t_all, 1), "unit": "tok/s", "n_gpus": 1, "steps": max(args.steps, 3),
        "warmup": max(args.warmup, 1), "ms_per_step": round(step_us / 1e3, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights (gains 1 + N(0,0.1)), uniform tokens",
        "config": {"workload": f"tiny decoder (2 blocks, d 256, 4q/2kv heads, head dim 64, SwiGLU 688, vocab 1024) "
                               f"as two stages on one GPU; greedy generation of {n_new} tokens from a {plen}-token "
                               "prompt through the on-device pipeline driver (value: tokens / s of the whole run)",
                   "kv_cache": args.kv},
        "us_per_generation": round(t_all * 1e6, 1), "us_per_decode_step": round(step_us, 1),
        "us_prefill_and_first_token": round(t_one * 1e6, 1), "tokens": got.tolist(),
        "roofline": None, "cpu_baseline": cpu,
    }


PREFILL_KINDS = ("norm", "qkv", "attn", "o", "gateup", "down")
DECODE_KINDS = ("qkv", "attn", "o", "gateup", "down")


def issued_mfma_flops(shape, n_blocks: int, T: int, kv: str, pos0: int = 0) -> int:
    """MFMA work a prefill issues: activation operands enter as bf16 planes, so each projection
    executes planes x its algorithmic flops.  Two planes, except the QKV rows whose outputs are
    rounded into a 2-byte cache: when the q rows alone make 256 or more 128 x 256 tiles only the
    K/V rows take three (the q rows are a separate two-plane GEMM), otherwise the fused projection
    takes three.  Attention takes 2 products per score / output term (3 over the F32-grade cache's
    pairs)."""
    from pipeline_stage_decoder_amd import accounting as acc
    lin = 0
    for kind, (n, k) in acc.projection_shapes(shape).items():
        if kind == "readout":
            continue
        if kind == "qkv" and kv != "f32":
            q_tiles = -(-T // 128) * -(-(shape.n_q_heads * shape.head_dim) // 256)
            n3 = 2 * shape.n_kv_heads * shape.head_dim if T >= 256 and q_tiles >= 256 else n
            lin += 2 * T * k * (2 * (n - n3) + 3 * n3)
        else:
            lin += 2 * T * n * k * 2
    attn = acc.prefill_flops(shape, 1, T, pos0=pos0) - acc.prefill_flops(shape, 1, T, pos0=pos0, attn=False)
    return n_blocks * (lin + attn * (3 if kv == "f32" else 2))


def _timed(fn, seconds: float):
    """Mean seconds of fn over about `seconds` (at least one call) after one untimed call."""
    fn()
    reps, t0 = 0, time.perf_counter()
    while reps < 1 or time.perf_counter() - t0 < seconds:
        fn()
        reps += 1
    return (time.perf_counter() - t0) / reps, reps


def cpu_baseline_block(shape, kv: str, blk: int, n_blocks: int, T: int, B: int, ctx: int, last: bool = False,
                       seconds: float = 4.0) -> dict:
    """The oracle, as it stands, on this host, on one real-shape block (global block blk) of the
    stage: a 64-row prefill (positions 0..63 of a fresh sequence) and a B = 2 decode step at
    position ctx over a seeded cache of ctx positions per slot, each repeated for about `seconds`;
    with `last`, also the final norm and readout of the 2 decode rows.  tok/s of the whole stage
    extrapolated linearly over blocks (and, for the prefill, over tokens: the timed chunk's rows
    attend up to T keys, the sample's up to 64, so attention -- a few % of a chunk's flops -- is
    under-counted)."""
    import numpy as np

    import fixtures as fx
    from oracle import decoder as o

    cores = cpu_threads()
    w = {(r, blk): fx.draw_weight(shape, r, blk) for r in fx.BLOCK_ROLES}
    if last:
        w[("final_norm", -1)] = fx.draw_weight(shape, "final_norm", -1)
        w[("readout", -1)] = fx.draw_weight(shape, "readout", -1)
    st = o.Stage(o.Dims.of(shape), blk, blk + 1, False, last, w, ctx + 1, kv_dtype=kv)
    n_s, b_s = 64, 2
    shp = (ctx, shape.n_kv_heads, shape.head_dim)
    for slot in range(b_s):
        k = o.KV_FORMATS[kv](fx.normal_f32(fx.SEED_HIDDEN, 0x7000 + 2 * slot, int(np.prod(shp))).reshape(shp))
        v = o.KV_FORMATS[kv](fx.normal_f32(fx.SEED_HIDDEN, 0x7001 + 2 * slot, int(np.prod(shp))).reshape(shp))
        st.import_kv(blk, slot, 0, k, v)
    xp = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(B), n_s * shape.d_model).reshape(n_s, shape.d_model)
    xd = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(1000), b_s * shape.d_model).reshape(b_s, shape.d_model)

    t_pre, r_pre = _timed(lambda: st.prefill(xp, b_s, 0), seconds)
    t_dec, r_dec = _timed(lambda: st.forward(xd, np.arange(b_s), np.full(b_s, ctx)), seconds)
    t_ro, r_ro = _timed(lambda: st.readout(xd), seconds) if last else (0.0, 0)
    ro = (f" + the final norm and readout of the {b_s} rows ({r_ro} reps, {t_ro:.2f} s each)" if last else "")
    return {"value": b_s / (t_dec * n_blocks + t_ro), "unit": "tok/s", "cores": cores, "kind": "oracle",
            "sample": f"decode: {r_dec} B={b_s} steps at position {ctx} of 1 of {n_blocks} blocks "
                      f"({t_dec:.2f} s per block-step){ro}; prefill: {r_pre} {n_s}-row prefills of 1 block "
                      f"({t_pre:.2f} s each); tok/s extrapolated linearly over the stage's {n_blocks} blocks "
                      f"(and the prefill over tokens, to a {T}-token chunk)",
            "prefill_value": n_s / (t_pre * n_blocks), "prefill_unit": "tok/s",
            "seconds_per_block_decode_step": t_dec, "seconds_per_block_prefill_64": t_pre,
            "seconds_readout": t_ro, "cpu_model": cpu_model()}


def cpu_baseline_mlp_slices(sh, n_sl: int, T: int = 64, seconds: float = 4.0) -> dict:
    """The oracle's sliced MLP on this host: T rows through all n_sl slices (each slice's SwiGLU
    MLP on its own weights, partials summed in slice order in F32), repeated for about `seconds`."""
    import numpy as np

    import fixtures as fx
    from oracle import decoder as o

    w = [{r: fx.draw_weight(sh, r, i) for r in ("mlp_norm", "wgate", "wup", "wdown")} for i in range(n_sl)]
    x = fx.normal_f32(fx.SEED_HIDDEN, fx.hidden_stream(40), T * sh.d_model).reshape(T, sh.d_model)
    eps = o.Dims.of(sh).rms_eps

    def run():
        acc_out = np.zeros((T, sh.d_model), np.float32)
        for wi in w:
            _, y = o.mlp_full(x, wi["mlp_norm"], wi["wgate"], wi["wup"], wi["wdown"], eps)
            acc_out = (acc_out + y).astype(np.float32)
        return acc_out

    t, reps = _timed(run, seconds)
    return {"value": T / t, "unit": "tok/s", "cores": cpu_threads(), "kind": "oracle",
            "sample": f"{reps} runs of {T} rows through all {n_sl} slices ({t:.2f} s each); rows/s at T = {T}, "
                      f"not extrapolated to the timed {4096}-row line", "cpu_model": cpu_model()}


def stage70b_line(args) -> dict:
    """The 70B-shaped middle stage (blocks 20..39 of 80): one step = a 4096-token prefill chunk (a
    fresh sequence, positions 0..4095) plus one batched decode step, B = 128 rows at position 8192
    of slots holding 8192 cached positions each."""
    import numpy as np
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd import accounting as acc
    from pipeline_stage_decoder_amd.stage import Stage

    shape, blocks, B, ctx, T = fx.LLAMA70B, (20, 40), 128, 8192, 4096
    nb, d, kv = blocks[1] - blocks[0], fx.LLAMA70B.d_model, args.kv
    kvb = 4 if kv == "f32" else 2
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    log(f"[bench] 70B-shaped stage {blocks}, {kv} cache: creating ({B + 1} slots, ctx {ctx + 1})")
    st = Stage(shape, blocks[0], blocks[1], False, False, max_slots=B + 1, max_ctx=ctx + 1, max_tokens=T,
               device=0, kv=kv)
    fill_weights(st, shape, blocks, False, False, fx.SEED_WEIGHTS)
    log("[bench] filling slot 0 with two 4096-token chunks, then copying it into the other decode slots")
    fill_kv_by_prefill(st, 0, ctx, T, range(1, B), d)
    xp = fx.normal_f32_gpu(torch.empty((T, d), dtype=torch.float32, device=dev), fx.SEED_HIDDEN,
                           fx.hidden_stream(B), 0)
    yp = torch.empty_like(xp)
    xd = fx.normal_f32_gpu(torch.empty((B, d), dtype=torch.float32, device=dev), fx.SEED_HIDDEN,
                           fx.hidden_stream(1000), 0)
    yd = torch.empty_like(xd)
    slots = torch.arange(B, dtype=torch.int32, device=dev)
    pos = torch.full((B,), ctx, dtype=torch.int32, device=dev)
    g = graph_of(lambda: st.decode(xd, slots, pos, out=yd), 1)
    log("[bench] decode step captured as a HIP graph")

    def run_step(ev):
        ev[0].record(stream)
        st.prefill(xp, B, 0, out=yp)              # slot B: a fresh sequence's first chunk
        ev[1].record(stream)
        g.replay()                                # B rows of slots 0..B-1 at position ctx
        ev[2].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]  # noqa: E731
    for w in range(args.warmup):
        run_step(mk())
        torch.cuda.synchronize()
        log(f"[bench] warmup step {w + 1}/{args.warmup}")
    # the roofline kernel (gate/up GEMM + SwiGLU of the prefill chunk) is timed live with HIP events
    # on the launch stream, over the timed region itself
    st.timing(["gateup"])
    evs = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        ev = mk()
        run_step(ev)
        evs.append(ev)
        if k % 5 == 4 or k == args.steps - 1:
            log(f"[bench] timed step {k + 1}/{args.steps} enqueued")
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n_gu, ms_gu = st.timing_read("gateup")
    st.timing([])
    pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    step_ms = float(np.median([e[0].elapsed_time(e[2]) for e in evs]))

    # per-kind kernel time of one step: one eager prefill and one eager decode step, every kind timed
    log("[bench] per-kind kernel times over one eager step")
    st.timing(list(PREFILL_KINDS))
    st.prefill(xp, B, 0, out=yp)
    torch.cuda.synchronize()
    pre_kinds = {k: st.timing_read(k) for k in PREFILL_KINDS}
    st.timing(list(DECODE_KINDS))
    st.decode(xd, slots, pos, out=yd)
    torch.cuda.synchronize()
    dec_kinds = {k: st.timing_read(k) for k in DECODE_KINDS}
    st.timing([])

    pre_flops = acc.prefill_flops(shape, nb, T)
    dec_bytes = acc.decode_step_bytes(shape, nb, [ctx] * B, kv_elem_bytes=kvb)
    gu_flops = acc.projection_flops(shape, "gateup", T)
    gu_avg_s = ms_gu / 1e3 / max(n_gu, 1)
    gu_tf = gu_flops / gu_avg_s / 1e12
    roofline = {"bound": "mfma", "achieved": round(gu_tf, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": counter_traffic(GEMM_COUNTER_FILE, "gateup", GEMM_SOURCES),
                "kernel": "k_gemm_dma (gate/up projection + SwiGLU of the 4096-token chunk: 128 x 256 tiles, "
                          "64-deep stages, two activation-plane and three weight LDS buffers)",
                "flops_per_launch": gu_flops, "algorithmic_bytes_per_launch": acc.projection_gemm_bytes(shape, "gateup", T),
                "avg_launch_us": round(gu_avg_s * 1e6, 2), "launches": n_gu,
                "issued_frac": round(2 * gu_tf / MFMA_BF16_PEAK_TFLOPS, 4),
                "share_of_step": round(pre_kinds["gateup"][1] / step_ms, 4)}
    n_at, ms_at = dec_kinds["attn"]
    at_bytes = B * (ctx + 1) * acc.kv_bytes_per_token_block(shape, kvb)
    roof_dec = kernel_roofline(at_bytes, n_at, ms_at,
                               f"k_attn_decode + k_attn_merge (split-KV GQA decode, B={B} at ctx {ctx}, {kv} cache)")
    dec_gbs = dec_bytes / (dec_ms / 1e3) / 1e9
    pre_tf = pre_flops / (pre_ms / 1e3) / 1e12
    return {
        "metric": "stage decode tok/s & HBM GB/s %peak; prefill tok/s & MFMA util",
        "value": round(B / (dec_ms / 1e3), 1), "unit": "tok/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(step_ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,0.02) bf16 weights, F32 N(0,1) hidden rows (random-init weights, no dataset)",
        "config": {"workload": "70B-shaped middle stage: blocks 20..39 of 80, d 8192, 64 q / 8 KV heads, head dim 128, "
                               "SwiGLU 28672, bf16 weights; step = one 4096-token prefill chunk + one batched decode "
                               "step B=128 at ctx 8192, F32 hidden in and out",
                   "prefill_chunk": T, "decode_batch": B, "decode_ctx": ctx, "blocks": list(blocks), "kv_cache": kv,
                   "decode_graph": True},
        "decode_ms": round(dec_ms, 3), "decode_step_bytes": dec_bytes, "decode_hbm_gbs": round(dec_gbs, 1),
        "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
        "prefill_tok_s": round(T / (pre_ms / 1e3), 1), "prefill_ms": round(pre_ms, 3),
        "prefill_tflops": round(pre_tf, 1), "prefill_mfma_frac": round(pre_tf / MFMA_BF16_PEAK_TFLOPS, 4),
        "prefill_mfma_issued_frac": round(issued_mfma_flops(shape, nb, T, kv) / (pre_ms / 1e3) / 1e12
                                          / MFMA_BF16_PEAK_TFLOPS, 4),
        "prefill_kernel_ms": {k: round(v[1], 3) for k, v in pre_kinds.items()},
        "decode_kernel_ms": {k: round(v[1], 3) for k, v in dec_kinds.items()},
        "wall_s_timed": round(wall, 3), "roofline": roofline, "roofline_decode": roof_dec,
        "handoff_us": time_handoff(yp, yd),
    }


def first8b_figures(args, reps: int = 3) -> dict:
    """The 8B-shaped first stage (embedding + blocks 0..15 of 32), batch 1: a 512-token prefill, then
    teacher-forced decode to ctx 2048 replayed from HIP graphs of 128 steps; `reps` timed requests."""
    import numpy as np
    import torch

    import fixtures as fx
    from pipeline_stage_decoder_amd import accounting as acc
    from pipeline_stage_decoder_amd.stage import Stage

    shape, blocks, T, ctx, kv = fx.LLAMA8B, (0, 16), 512, 2048, args.kv
    n_dec = ctx - T
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    log(f"[bench] 8B-shaped first stage, {kv} cache")
    st = Stage(shape, blocks[0], blocks[1], True, False, max_slots=1, max_ctx=ctx, max_tokens=T, device=0, kv=kv)
    fill_weights(st, shape, blocks, True, False, fx.SEED_WEIGHTS)
    prompt = fx.tokens_gpu(torch.empty(T, dtype=torch.int32, device=dev), fx.SEED_TOKENS, fx.token_stream(0),
                           shape.vocab)
    dec_tok = fx.tokens_gpu(torch.empty(n_dec, dtype=torch.int32, device=dev), fx.SEED_TOKENS,
                            fx.token_stream(1), shape.vocab)
    positions = torch.arange(T, ctx, dtype=torch.int32, device=dev)
    slot0 = torch.zeros(1, dtype=torch.int32, device=dev)
    xin = torch.empty((T, shape.d_model), dtype=torch.float32, device=dev)
    hout = torch.empty_like(xin)
    x1 = torch.empty((1, shape.d_model), dtype=torch.float32, device=dev)
    h1 = torch.empty_like(x1)
    st.embed(dec_tok[:1], out=x1)
    st.decode(x1, slot0, positions[:1], out=h1)
    torch.cuda.synchronize()
    graph_steps, graphs = 128, []
    cs = torch.cuda.Stream()
    for g0 in range(0, n_dec, graph_steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            for i in range(g0, g0 + graph_steps):
                st.embed(dec_tok[i:i + 1], out=x1)
                st.decode(x1, slot0, positions[i:i + 1], out=h1)
        graphs.append(g)
    torch.cuda.synchronize()

    def run(ev):
        ev[0].record(stream)
        st.embed(prompt, out=xin)
        st.prefill(xin, 0, 0, out=hout)
        ev[1].record(stream)
        for g in graphs:
            g.replay()
        ev[2].record(stream)

    mk = lambda: [torch.cuda.Event(enable_timing=True) for _ in range(3)]  # noqa: E731
    run(mk())
    torch.cuda.synchronize()
    evs = []
    for r in range(reps):
        ev = mk()
        run(ev)
        torch.cuda.synchronize()
        evs.append(ev)
        log(f"[bench] 8B request {r + 1}/{reps}")
    pre_ms = float(np.median([e[0].elapsed_time(e[1]) for e in evs]))
    dec_ms = float(np.median([e[1].elapsed_time(e[2]) for e in evs]))
    # the dominant decode kernel (gate/up GEMV + SwiGLU), timed live with HIP events over one eager
    # decode pass of the request
    st.embed(prompt, out=xin)
    st.prefill(xin, 0, 0, out=hout)
    st.timing(list(DECODE_KINDS))
    kern = {k: [0, 0.0] for k in DECODE_KINDS}
    for i in range(n_dec):
        st.embed(dec_tok[i:i + 1], out=x1)
        st.decode(x1, slot0, positions[i:i + 1], out=h1)
        if i % 256 == 255 or i == n_dec - 1:
            for k in DECODE_KINDS:
                n, ms = st.timing_read(k)
                kern[k][0] += n
                kern[k][1] += ms
    st.timing([])
    kvb = 4 if kv == "f32" else 2
    dec_bytes = sum(acc.decode_step_bytes(shape, 16, [c], first=True, kv_elem_bytes=kvb) for c in range(T, ctx))
    dec_gbs = dec_bytes / (dec_ms / 1e3) / 1e9
    pre_tf = acc.prefill_flops(shape, 16, T) / (pre_ms / 1e3) / 1e12
    gu = kern["gateup"]
    gu_bytes = acc.projection_bytes(shape, "gateup", 1)
    out = {"workload": "8B-shaped first stage: embedding + blocks 0..15 of 32, d 4096, 32q/8kv heads, head dim 128, "
                       "SwiGLU 14336, vocab 128256; batch 1, prefill 512 then decode to ctx 2048",
           "kv_cache": kv, "requests_timed": reps,
           "decode_tok_s": round(n_dec / (dec_ms / 1e3), 2), "decode_ms_per_token": round(dec_ms / n_dec, 4),
           "decode_hbm_gbs": round(dec_gbs, 1), "decode_hbm_frac": round(dec_gbs / HBM_PEAK_GBS, 4),
           "prefill_tok_s": round(T / (pre_ms / 1e3), 1), "prefill_ms": round(pre_ms, 3),
           "prefill_tflops": round(pre_tf, 1), "prefill_mfma_frac": round(pre_tf / MFMA_BF16_PEAK_TFLOPS, 4),
           "prefill_mfma_issued_frac": round(issued_mfma_flops(shape, 16, T, kv) / (pre_ms / 1e3) / 1e12
                                             / MFMA_BF16_PEAK_TFLOPS, 4),
           "decode_kernel_avg_us": {k: round(v[1] * 1e3 / max(v[0], 1), 2) for k, v in kern.items()},
           "roofline_decode_gateup": kernel_roofline(gu_bytes, gu[0], gu[1],
                                                     "k_gemv1 (gate/up projection + SwiGLU, B=1)")}
    out["roofline_decode_gateup"]["traffic"] = counter_traffic(COUNTER_FILE, "gateup", GEMV_SOURCES)
    del graphs
    st.close()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--kv", choices=("f16", "f32", "bf16"), default="f16",
                    help="KV cache format (f16 and f32 are validated against the oracle at full stage depth)")
    ap.add_argument("--workload", choices=("mid-70b", "first-8b", "last-8b", "mlp-slices", "pipeline-8b",
                                           "attn-parallel", "placement", "tiny"),
                    default="mid-70b",
                    help="mid-70b: the benchmark line (70B-shaped stage; also reports the 8B first stage); "
                         "the others report the remaining workloads")
    ap.add_argument("--phase", choices=("both", "prefill", "counters"), default="both",
                    help="prefill: only time the prefill; counters: prefill + 32 plain decode steps and nothing "
                         "else (short runs for hardware-counter passes)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-first-8b", action="store_true", help="skip the 8B first-stage figures of the default line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="only summarise the rocprofv3 CSV output under DIR")
    ap.add_argument("--source-hash", choices=("gemv", "gemm"),
                    help="only print the hash of the kernel sources a counter summary was taken on")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof)
        return
    if args.source_hash:
        print(source_hash(GEMV_SOURCES if args.source_hash == "gemv" else GEMM_SOURCES))
        return
    if args.workload == "placement":             # host only
        print(json.dumps(placement_line(args)), flush=True)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs one pipeline stage on one GPU; "
                                   "--gpus above 1 is not supported (the stage has no cross-GPU path)"}))
        sys.exit(2)

    import torch

    if args.copy_calibration:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")       # 1 GiB
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": a.numel() * 4, "bytes_written": b.numel() * 4,
                          "dispatches": 5}))
        return

    import fixtures as fx

    torch.cuda.set_device(0)
    if args.phase == "prefill":
        if args.workload == "mid-70b":     # one 4096-token chunk at position 0
            prefill_only(args, fx.LLAMA70B, (20, 40), 4096, torch.device("cuda:0"), torch.cuda.current_stream(),
                         first=False)
        else:
            prefill_only(args, fx.LLAMA8B, (0, 16), 512, torch.device("cuda:0"), torch.cuda.current_stream())
        return
    if args.phase == "counters":
        counter_pass(fx.LLAMA8B, (0, 16), 512, torch.device("cuda:0"), kv=args.kv)
        return
    if args.workload == "last-8b":
        print(json.dumps(batched_decode_line(
            args, "8B-shaped last stage: blocks 16..31 of 32 + final norm + readout (vocab 128256); "
                  "batched decode B=64 at context 4096, F32 hidden in, F32 logits out",
            fx.LLAMA8B, (16, 32), False, True, 64, 4096, 1024, False)), flush=True)
        return
    if args.workload == "pipeline-8b":
        print(json.dumps(pipeline_line(args)), flush=True)
        return
    if args.workload == "tiny":
        print(json.dumps(tiny_line(args)), flush=True)
        return
    if args.workload == "mlp-slices":
        print(json.dumps(mlp_slices_line(args)), flush=True)
        return
    if args.workload == "attn-parallel":
        print(json.dumps(attn_parallel_line(args)), flush=True)
        return
    if args.workload == "first-8b":
        print(json.dumps(first8b_figures(args, reps=max(args.steps, 1))), flush=True)
        return

    out = stage70b_line(args)
    torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample (one 70B-shaped block)")
        cpu = cpu_baseline_block(fx.LLAMA70B, args.kv, 20, 20, 4096, 128, 8192)
    out["cpu_baseline"] = cpu
    if not args.no_first_8b:
        out["first_8b"] = first8b_figures(args)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
