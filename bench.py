#!/usr/bin/env python3
"""Benchmark: per-rank attention of a context-parallel video diffusion transformer on one MI355X.

One step = one denoising step's worth of attention on the full single-GPU
video workload: 36 layers x (bf16 self-attention S=44160, H=24, D=128, plus
cross-attention of the 44160 video queries to 2992 text keys), on seeded
synthetic N(0,1) inputs resident in HBM before timing starts.  The workload
models the Cosmos 3 setting described in "Simplifying model serving across
multiple GPUs with NVIDIA TensorRT multi-device integration in NVIDIA
Dynamo-Triton" (44160 video tokens, a 2992-token text path, 36 transformer
layers); heads and head dim are assumed.

Printed: one JSON line with the step throughput in TFLOP/s (4*B*H*Sq*Skv*D per
attention call), the roofline of the dominant kernel (the self-attention
launch, timed with HIP events on its own stream inside the timed region),
the fp64 CPU oracle timed on a bounded row sample, and secondary
measurements of the other kernels on the path (LSE merge, ring driver,
Ulysses pack/unpack) at their per-rank shapes.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 matrix-core peak (256 CUs at 2.4 GHz)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_CLOCK_MHZ = 2400.0     # engine clock the matrix-core peak is quoted at
LAYERS = 36
KERNEL_SRC = [os.path.join(ROOT, "long_sequence_bidirectional_amd", "csrc", f)
              for f in ("attn_fwd_kernel.h", "attn_fwd_bf16.hip", "unit_sched.h", "kernels.h", "common.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_bf16_video_layer_traffic.json")
# calibration copy for the HBM counters: Ulysses pack of a [44160, 24, 128] bf16 shard
CALIB_SHAPE = (1, 44160, 24, 128)


def _code_only(text: str) -> str:
    """C++ source without its comments and blank lines (the compiled code does not depend on them).
    The kernel sources hold no string literal with "//" or "/*" in it."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash() -> str:
    """SHA-256 over the code of the bf16 attention kernel's sources (template, instantiation, unit
    schedule and the shared headers), comments left out."""
    import hashlib
    h = hashlib.sha256()
    for path in KERNEL_SRC:
        with open(path, encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
        h.update(b"\0")
    return h.hexdigest()


def measured_counters(path):
    """(HBM bytes per self-attention launch, derived counter figures) from the committed
    counter summary, or (None, None) when the kernel source changed after the counters
    were taken."""
    if not path or not os.path.exists(path):
        return None, None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None, None
    c = t.get("counters") or {}
    derived = {k: c[k] for k in ("gfx_clock_ghz", "mfma_busy_frac_at_clock", "busy_cycles_per_mfma") if k in c}
    return t.get("traffic_bytes_per_launch"), (derived or None)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--layers", type=int, default=LAYERS, help="attention layers per step (36 in the workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the CPU oracle sample")
    ap.add_argument("--no-secondary", action="store_true", help="skip merge/ring/relayout measurements")
    ap.add_argument("--traffic", type=str, default=TRAFFIC_FILE,
                    help="JSON with the measured HBM bytes per launch of the dominant kernel")
    ap.add_argument("--profile-pass", nargs="?", const="all", choices=["all", "short"], default=None,
                    help="the program profiled by the rocprofv3 --pmc passes, instead of the bench: 'all' runs "
                         "one self-attention launch, one calibration copy and the other kernels once; 'short' "
                         "runs one launch of each short-key-range shape (cross-attention, AllGather-KV rank, "
                         "ring chunks) and the calibration copy")
    return ap.parse_args()


def elapsed_ms(pairs):
    return [a.elapsed_time(b) for a, b in pairs]


def smi_sample():
    """(socket power W, mean gfx clock MHz) from one amd-smi reading, or None.  The kernel runs at
    the board's power limit, so the clock it ran at is part of the measurement."""
    import subprocess
    try:
        r = subprocess.run(["amd-smi", "metric", "-p", "-c", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        g = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clks = [float(g["clock"][f"gfx_{i}"]["clk"]["value"]) for i in range(8) if f"gfx_{i}" in g["clock"]]
        return float(g["power"]["socket_power"]["value"]), sum(clks) / len(clks)
    except Exception:
        return None


def cpu_baseline(budget_s: float):
    """Time the fp64 oracle on a bounded sample of the self-attention workload.

    Sample: blocks of 64 query rows of the S=44160 self-attention, head after
    head, until the time budget is used; throughput = the sample's flops
    (4 * rows * Skv * D) / seconds.
    """
    import numpy as np
    import oracle
    from long_sequence_bidirectional_amd import inputs

    g = inputs.video_set()
    D, S, H = inputs.HEAD_DIM, inputs.S_VIDEO, inputs.N_HEADS
    scale = 1.0 / math.sqrt(D)
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        blas_threads = cores
    rows_done, t_total, heads_used = 0, 0.0, 0
    rng = np.random.Generator(np.random.PCG64(inputs.SEED))
    for h in range(H):
        if t_total >= budget_s:
            break
        k = inputs.bf16_bits_to_f32(g["k"][:, h:h + 1]).astype(np.float64)
        v = inputs.bf16_bits_to_f32(g["v"][:, h:h + 1]).astype(np.float64)
        heads_used += 1
        while t_total < budget_s * (h + 1) / H:     # an equal share of the budget per head
            r0 = int(rng.integers(0, S - 64))
            q = inputs.bf16_bits_to_f32(g["q"][:, h:h + 1, r0:r0 + 64]).astype(np.float64)
            t0 = time.perf_counter()
            oracle.attention(q, k, v, scale)
            t_total += time.perf_counter() - t0
            rows_done += 64
    flops = 4.0 * rows_done * S * D
    cpu = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": int(min(cores, blas_threads)),
            "kind": "oracle",
            "sample": f"{rows_done} query rows (blocks of 64) of the S=44160 H=24 D=128 self-attention "
                      f"over {heads_used} heads, fp64 numpy, {t_total:.1f} s; host has {cores} cores ({cpu})"}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(no collectives); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import long_sequence_bidirectional_amd as cp
    from long_sequence_bidirectional_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    cp.lib()   # fail loudly now if the library is missing

    D, S, H, S_TXT = inputs.HEAD_DIM, inputs.S_VIDEO, inputs.N_HEADS, inputs.S_TEXT
    scale = 1.0 / math.sqrt(D)
    g = inputs.video_set()

    def dev(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v, kt, vt = (dev(g[n]) for n in ("q", "k", "v", "k_text", "v_text"))
    if args.profile_pass == "short":
        profile_pass_short(cp, torch, q, k, v, kt, vt)
        return
    if args.profile_pass:
        profile_pass(cp, torch, q, k, v)
        return
    o_self = torch.empty_like(q)
    l_self = torch.empty((1, H, S), dtype=torch.float32, device="cuda")
    o_x = torch.empty_like(q)
    l_x = torch.empty_like(l_self)
    stream = torch.cuda.current_stream()
    # workspaces of the key-range split of each call's last, partial wave of tiles
    ws_self = workspace(cp, torch, 1, H, S, S, D)
    ws_x = workspace(cp, torch, 1, H, S, S_TXT, D)

    flops_self = 4.0 * H * S * S * D
    flops_cross = 4.0 * H * S * S_TXT * D
    flops_step = args.layers * (flops_self + flops_cross)

    def step(ev_self=None):
        for _ in range(args.layers):
            if ev_self is not None:
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
            cp.attn_fwd_ex(q, k, v, o=o_self, lse=l_self, scale=scale, workspace=ws_self, stream=stream)
            if ev_self is not None:
                b.record(stream)
                ev_self.append((a, b))
            cp.attn_fwd_ex(q, kt, vt, o=o_x, lse=l_x, scale=scale, workspace=ws_x, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev_self = []
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # one power / clock reading taken while the timed steps run (host thread, no GPU work)
    smi = []
    sampler = threading.Thread(target=lambda: (time.sleep(0.8), smi.append(smi_sample())), daemon=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    sampler.start()
    for _ in range(args.steps):
        step(ev_self)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    sampler.join(timeout=30)
    power_clock = smi[0] if smi else None
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps
    value = flops_step / (ms_step * 1e-3) / 1e12
    self_ms = elapsed_ms(ev_self)
    self_avg = sum(self_ms) / len(self_ms)
    self_sorted = sorted(self_ms)
    achieved = flops_self / (self_avg * 1e-3) / 1e12

    traffic, counters = measured_counters(args.traffic)

    secondary = None if args.no_secondary else secondary_rows(cp, torch, q, k, v, stream, kt, vt)

    result = {
        "metric": "attention TFLOP/s (bf16) and % of MFMA peak at S=44160, H=24, D=128",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1), bf16)",
        "config": {"workload": "video_layer: 36 x (self-attention S=44160 + cross-attention to 2992 text "
                               "tokens), H=24, D=128, B=1, non-causal",
                   "B": 1, "H": H, "S": S, "S_text": S_TXT, "D": D, "layers": args.layers},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
                     "kernel": "attn_fwd_mfma_kernel<128,bf16,o bf16,head-major> + merge_pieces_kernel<bf16> "
                               "(self-attention S=44160; the events bracket both)",
                     "avg_launch_ms": round(self_avg, 4), "launches": len(self_ms),
                     "median_launch_ms": round(self_sorted[len(self_sorted) // 2], 4),
                     "min_launch_ms": round(self_sorted[0], 4), "max_launch_ms": round(self_sorted[-1], 4),
                     "socket_power_w": power_clock[0] if power_clock else None,
                     "gfx_clock_mhz": round(power_clock[1]) if power_clock else None,
                     # the same fraction against the peak scaled to the clock measured during the run
                     "frac_at_clock": (round(achieved / (PEAK_BF16_TFLOPS * power_clock[1] / PEAK_CLOCK_MHZ), 4)
                                       if power_clock and power_clock[1] else None),
                     "split": split_of(cp, H, S, S, D, ws_self),
                     "counters": counters},
        "wall_s_timed": round(wall, 3),
        "secondary": secondary,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


def workspace(cp, torch, B, H, Sq, Skv, D, f32_out=False):
    n = cp.attn_fwd_workspace_size(B, H, Sq, Skv, D, o_dtype=cp.F32 if f32_out else cp.BF16)
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def split_of(cp, H, Sq, Skv, D, ws):
    """The split plan attn_fwd_ex follows on this device for this workspace."""
    import torch
    props = torch.cuda.get_device_properties(0)
    slots = props.multi_processor_count   # one 160 KB-LDS workgroup per CU
    tiles, pieces, nbytes = cp.attn_fwd_split_plan(1, H, Sq, Skv, D, slots, ws.numel())
    return {"slots": slots, "tiles": H * -(-Sq // 256), "split_tiles": tiles, "pieces": pieces,
            "workspace_bytes": nbytes}


def profile_pass(cp, torch, q, k, v):
    """One self-attention launch and one copy of known size (counter calibration)."""
    o = torch.empty_like(q)
    l = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    B, H, S, D = q.shape
    cp.attn_fwd_ex(q, k, v, o=o, lse=l, workspace=workspace(cp, torch, B, H, S, k.shape[2], D))
    shard = torch.empty(CALIB_SHAPE, dtype=torch.bfloat16, device="cuda").view(torch.int16).random_().view(
        torch.bfloat16)
    send = torch.empty((1, 8, CALIB_SHAPE[1], CALIB_SHAPE[2] // 8, CALIB_SHAPE[3]), dtype=torch.bfloat16,
                       device="cuda")
    torch.cuda.synchronize()
    cp.ulysses_pack(shard, 8, cp.SEQ_TO_HEAD, dst=send)
    torch.cuda.synchronize()
    del shard, send
    # merge and relayout at their per-rank shapes, each over 12 rotating buffer sets (> the 256 MB
    # MALL), so the counters see HBM traffic: f32 merge of [1,24,5520,128] partials in place, then
    # pack and unpack of [5520,24,128] bf16 shards
    from long_sequence_bidirectional_amd import inputs
    S_L, P, H, D = inputs.S_LOCAL, inputs.CP_DEGREE, inputs.N_HEADS, inputs.HEAD_DIM
    sets = [(torch.randn((1, H, S_L, D), device="cuda"), torch.randn((1, H, S_L), device="cuda"),
             torch.randn((1, H, S_L, D), device="cuda"), torch.randn((1, H, S_L), device="cuda")) for _ in range(12)]
    torch.cuda.synchronize()
    for oa, la, ob, lb in sets:
        cp.attn_merge(oa, la, ob, lb, o_out=oa, lse_out=la)
    torch.cuda.synchronize()
    del sets
    shards = [torch.randn((1, S_L, H, D), device="cuda").to(torch.bfloat16) for _ in range(12)]
    sends = [torch.empty((1, P, S_L, H // P, D), dtype=torch.bfloat16, device="cuda") for _ in range(12)]
    torch.cuda.synchronize()
    for a, b in zip(shards, sends):
        cp.ulysses_pack(a, P, cp.SEQ_TO_HEAD, dst=b)
    torch.cuda.synchronize()
    for a, b in zip(shards, sends):
        cp.ulysses_unpack(b, P, cp.SEQ_TO_HEAD, dst=a.view(1, H // P, S_L * P, D))
    torch.cuda.synchronize()
    # the same shards as 4 batched packs of three (one rank's Q, K, V per launch)
    for i in range(0, 12, 3):
        cp.ulysses_pack_n(shards[i:i + 3], P, cp.SEQ_TO_HEAD, dsts=sends[i:i + 3])
    torch.cuda.synchronize()
    del shards, sends
    # the fp8 self-attention (E4M3 of N(0,1) draws, made on the device) and the QK-RMSNorm
    # prologue over the attention sample's K [56320, 32, 128] fp16 (461 MB each way)
    q8, k8, v8 = (torch.randn((1, H, inputs.S_VIDEO, D), device="cuda").to(torch.float8_e4m3fn)
                  for _ in range(3))
    o8 = torch.empty((1, H, inputs.S_VIDEO, D), dtype=torch.bfloat16, device="cuda")
    l8 = torch.empty((1, H, inputs.S_VIDEO), dtype=torch.float32, device="cuda")
    ws8 = torch.empty(cp.attn_fwd_workspace_size(1, H, inputs.S_VIDEO, inputs.S_VIDEO, D, cp.E4M3, cp.BF16),
                      dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    cp.attn_fwd_fp8(q8, k8, v8, o=o8, lse=l8, workspace=ws8)
    torch.cuda.synchronize()
    del q8, k8, v8, o8, l8
    x = torch.randn((1, inputs.P4_SEQ, inputs.P4_HEADS, D), device="cuda").to(torch.float16)
    w = torch.randn((D,), device="cuda").to(torch.float16)
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    cp.qk_rmsnorm(x, w, 1e-6, D ** -0.25, out=y)
    torch.cuda.synchronize()
    norm_bytes = x.numel() * 2
    del x, w, y
    # the bf16 self-attention again with K stored sequence-last [1,24,128,44160]
    kt = k.transpose(2, 3).contiguous()
    cp.attn_fwd_ex(q, kt, v, o=o, lse=l, workspace=workspace(cp, torch, B, H, S, k.shape[2], D), k_seq_last=True)
    torch.cuda.synchronize()
    print(f"profile pass done; calibration copy {CALIB_SHAPE[1] * CALIB_SHAPE[2] * CALIB_SHAPE[3] * 2} bytes "
          "read and written; 12 cold merges, packs and unpacks; 4 batched packs of 3 shards; fp8 "
          f"self-attention; QK-RMSNorm of {norm_bytes} bytes; self-attention with K sequence-last", flush=True)


def timed_leg(torch, stream, fn, flops=None, nbytes=None, iters=50, warmup=3, clock=True):
    """`warmup` untimed calls, then `iters` calls each bracketed by its own HIP event pair on the
    launch stream: mean / median / min / max per call, the throughput of the median call, and one
    amd-smi power and clock reading taken while the same call keeps running (the kernels run at
    the board's power limit, so the clock belongs to the result)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    pairs = []
    for _ in range(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        pairs.append((a, b))
    torch.cuda.synchronize()
    ms = sorted(elapsed_ms(pairs))
    med = ms[len(ms) // 2]
    out = {"iters": iters, "warmup": warmup, "ms_mean": round(sum(ms) / len(ms), 4), "ms_median": round(med, 4),
           "ms_min": round(ms[0], 4), "ms_max": round(ms[-1], 4)}
    if flops is not None:
        out["tflops_median"] = round(flops / med / 1e9, 1)
        out["frac_of_bf16_peak"] = round(flops / med / 1e9 / PEAK_BF16_TFLOPS, 4)
    if nbytes is not None:
        out["GBps_median"] = round(nbytes / med / 1e6, 1)
    if clock:
        # two readings in a row, the second kept: the first can still reflect the idle time
        # before the leg (the board averages its power readings over a short window)
        sample = []
        th = threading.Thread(target=lambda: (smi_sample(), sample.append(smi_sample())), daemon=True)
        th.start()
        while th.is_alive():      # keep this leg's kernel running until the reading is back
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
        th.join()
        pc = sample[0] if sample else None
        out["socket_power_w"] = pc[0] if pc else None
        out["gfx_clock_mhz"] = round(pc[1]) if pc else None
    return out


def calibration_copy(cp, torch):
    """The copy of known size the HBM counters are scaled by: a Ulysses pack of a [44160,24,128]
    bf16 shard, 271,319,040 bytes read and the same written."""
    shard = torch.empty(CALIB_SHAPE, dtype=torch.bfloat16, device="cuda").view(torch.int16).random_().view(
        torch.bfloat16)
    send = torch.empty((1, 8, CALIB_SHAPE[1], CALIB_SHAPE[2] // 8, CALIB_SHAPE[3]), dtype=torch.bfloat16,
                       device="cuda")
    torch.cuda.synchronize()
    cp.ulysses_pack(shard, 8, cp.SEQ_TO_HEAD, dst=send)
    torch.cuda.synchronize()


def profile_pass_short(cp, torch, q, k, v, kt, vt):
    """One launch of each short-key-range shape, in this order (each attention launch followed
    by its piece merge): cross-attention 44160 x 2992 (bf16 O), the AllGather-KV rank 5520 x 44160
    (bf16 O), ring chunk 0 then ring chunk 1 folded in by the accumulate epilogue (5520 x 5520,
    f32 O); then the calibration copy."""
    from long_sequence_bidirectional_amd import inputs
    S_L, H, D = inputs.S_LOCAL, inputs.N_HEADS, inputs.HEAD_DIM
    legend = []
    o = torch.empty_like(q)
    l = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    cp.attn_fwd_ex(q, kt, vt, o=o, lse=l, workspace=workspace(cp, torch, 1, H, q.shape[2], kt.shape[2], D))
    torch.cuda.synchronize()
    legend.append("cross 44160x2992")
    del o, l
    q_l = q[:, :, :S_L].contiguous()
    o_b = torch.empty((1, H, S_L, D), dtype=torch.bfloat16, device="cuda")
    l = torch.empty((1, H, S_L), dtype=torch.float32, device="cuda")
    ws = workspace(cp, torch, 1, H, S_L, inputs.S_VIDEO, D)
    torch.cuda.synchronize()
    cp.attn_fwd_ex(q_l, k, v, o=o_b, lse=l, workspace=ws)
    torch.cuda.synchronize()
    legend.append("allgather_kv_rank 5520x44160")
    kc = [k[:, :, c * S_L:(c + 1) * S_L].contiguous() for c in range(2)]
    vc = [v[:, :, c * S_L:(c + 1) * S_L].contiguous() for c in range(2)]
    o_f = torch.empty((1, H, S_L, D), dtype=torch.float32, device="cuda")
    ws_c = workspace(cp, torch, 1, H, S_L, S_L, D, f32_out=True)
    torch.cuda.synchronize()
    for c in range(2):
        cp.attn_fwd_ex(q_l, kc[c], vc[c], o=o_f, lse=l, workspace=ws_c, accumulate=c > 0)
        torch.cuda.synchronize()
        legend.append(f"ring chunk {c} 5520x5520{' (accumulate)' if c else ''}")
    calibration_copy(cp, torch)
    print("profile pass (short key ranges) done: " + "; ".join(legend) + "; calibration copy "
          f"{CALIB_SHAPE[1] * CALIB_SHAPE[2] * CALIB_SHAPE[3] * 2} bytes read and written", flush=True)


def secondary_rows(cp, torch, q, k, v, stream, kt=None, vt=None):
    """Timings of the other kernels on the path, at their per-rank shapes."""
    from long_sequence_bidirectional_amd import inputs
    S_L, P, H, D = inputs.S_LOCAL, inputs.CP_DEGREE, inputs.N_HEADS, inputs.HEAD_DIM
    out = {}

    def timeit(fn, iters=20):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(iters):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / iters

    # The per-rank legs: 3 warm-ups, then 50 calls each timed on its own, median reported.
    # ring_rank: Q 5520 rows vs 8 chunks of 5520 keys (chunk attention folded into the f32
    # accumulator in its epilogue; the work buffers hold the split pieces)
    q_l = q[:, :, :S_L].contiguous()
    kc = torch.stack([k[:, :, c * S_L:(c + 1) * S_L] for c in range(P)]).contiguous()
    vc = torch.stack([v[:, :, c * S_L:(c + 1) * S_L] for c in range(P)]).contiguous()
    o = torch.empty((1, H, S_L, D), dtype=torch.float32, device="cuda")
    l = torch.empty((1, H, S_L), dtype=torch.float32, device="cuda")
    ow, lw = torch.empty_like(o), torch.empty_like(l)
    ring_flops = 4.0 * H * S_L * S_L * P * D
    out["ring_rank"] = timed_leg(torch, stream, lambda: cp.ring_attn_fwd(q_l, kc, vc, o=o, lse=l, o_work=ow,
                                                                          lse_work=lw, stream=stream), ring_flops)
    out["ring_rank_unsplit"] = timed_leg(
        torch, stream, lambda: cp.ring_attn_fwd(q_l, kc, vc, o=o, lse=l, use_work=False, stream=stream), ring_flops,
        clock=False)
    # one chunk's attention alone (the ring step's kernel), accumulating into the f32 result
    ws_c = workspace(cp, torch, 1, H, S_L, S_L, D, f32_out=True)
    out["ring_chunk"] = timed_leg(torch, stream, lambda: cp.attn_fwd_ex(q_l, kc[3], vc[3], o=o, lse=l, workspace=ws_c,
                                                                        accumulate=True, stream=stream),
                                  ring_flops / P, clock=False)
    # allgather_kv_rank: Q 5520 vs K/V 44160
    o_b = torch.empty((1, H, S_L, D), dtype=torch.bfloat16, device="cuda")
    ws = workspace(cp, torch, 1, H, S_L, inputs.S_VIDEO, D)
    agkv_flops = 4.0 * H * S_L * inputs.S_VIDEO * D
    out["allgather_kv_rank"] = timed_leg(
        torch, stream, lambda: cp.attn_fwd_ex(q_l, k, v, o=o_b, lse=l, workspace=ws, stream=stream), agkv_flops)
    out["allgather_kv_rank_unsplit"] = timed_leg(
        torch, stream, lambda: cp.attn_fwd(q_l, k, v, o=o_b, lse=l, stream=stream), agkv_flops, clock=False)
    # ulysses_rank attention: H=3, S=44160
    q3, k3, v3 = (x[:, :3].contiguous() for x in (q, k, v))
    o3 = torch.empty_like(q3)
    l3 = torch.empty((1, 3, inputs.S_VIDEO), dtype=torch.float32, device="cuda")
    ws3 = workspace(cp, torch, 1, 3, inputs.S_VIDEO, inputs.S_VIDEO, D)
    uly_flops = 4.0 * 3 * inputs.S_VIDEO ** 2 * D
    out["ulysses_rank"] = timed_leg(
        torch, stream, lambda: cp.attn_fwd_ex(q3, k3, v3, o=o3, lse=l3, workspace=ws3, stream=stream), uly_flops)
    out["ulysses_rank_unsplit"] = timed_leg(
        torch, stream, lambda: cp.attn_fwd(q3, k3, v3, o=o3, lse=l3, stream=stream), uly_flops, clock=False)
    # the rank's local work between the two all-to-alls, from the receive buffers of Q, K, V
    # ([P, S_l, Hp, D] each) to the send buffer of O: unpack x3 + head-major attention + pack,
    # against sequence-major attention reading and writing those buffers in place
    recv = [x.transpose(1, 2).contiguous() for x in (q3, k3, v3)]          # [1, S, 3, D] = [1, P, S_l, 3, D]
    o_send = torch.empty_like(recv[0])
    ws3s = workspace(cp, torch, 1, 3, inputs.S_VIDEO, inputs.S_VIDEO, D)
    r5 = [x.view(1, P, S_L, H // P, D) for x in recv]
    unpacked = [torch.empty_like(q3) for _ in range(3)]

    def unfused():
        cp.ulysses_unpack_n(r5, P, cp.SEQ_TO_HEAD, dsts=unpacked, stream=stream)
        cp.attn_fwd_ex(unpacked[0], unpacked[1], unpacked[2], o=o3, lse=l3, workspace=ws3, stream=stream)
        cp.ulysses_pack(o3, P, cp.HEAD_TO_SEQ, dst=o_send.view(1, P, S_L, H // P, D), stream=stream)

    out["ulysses_rank_local_unfused"] = timed_leg(torch, stream, unfused, uly_flops, clock=False)
    out["ulysses_rank_local_fused"] = timed_leg(
        torch, stream, lambda: cp.attn_fwd_ex(recv[0], recv[1], recv[2], o=o_send, lse=l3, workspace=ws3s,
                                              seq_major=True, stream=stream), uly_flops, clock=False)
    # cross-attention of the video layer on its own: 44160 queries against the 2992 text keys
    if kt is not None:
        o_x = torch.empty_like(q)
        l_x = torch.empty((1, H, inputs.S_VIDEO), dtype=torch.float32, device="cuda")
        ws_x = workspace(cp, torch, 1, H, inputs.S_VIDEO, kt.shape[2], D)
        out["cross_attention"] = timed_leg(
            torch, stream, lambda: cp.attn_fwd_ex(q, kt, vt, o=o_x, lse=l_x, workspace=ws_x, stream=stream),
            4.0 * H * inputs.S_VIDEO * kt.shape[2] * D)
        del o_x, l_x, ws_x
    # merge (f32 O, the ring partial format): reads 2 O + 2 LSE, writes 1 O + 1 LSE
    ms = timeit(lambda: cp.attn_merge(o, l, ow, lw, o_out=o, lse_out=l, stream=stream))
    merge_bytes = 3 * o.numel() * 4 + 3 * l.numel() * 4
    out["merge_f32_us"] = round(ms * 1e3, 2)
    out["merge_f32_GBps"] = round(merge_bytes / ms / 1e6, 1)
    # Ulysses relayout of a [5520, 24, 128] bf16 shard (33.9 MB read + written), hot in the 256 MB MALL
    shard = q[0, :, :S_L].transpose(0, 1).contiguous().unsqueeze(0)
    send = torch.empty((1, P, S_L, H // P, D), dtype=torch.bfloat16, device="cuda")
    heads = torch.empty((1, H // P, S_L * P, D), dtype=torch.bfloat16, device="cuda")
    nbytes = 2 * shard.numel() * 2
    ms = timeit(lambda: cp.ulysses_pack(shard, P, cp.SEQ_TO_HEAD, dst=send, stream=stream))
    out["pack_s2h_us"] = round(ms * 1e3, 2)
    out["pack_s2h_GBps"] = round(nbytes / ms / 1e6, 1)
    ms = timeit(lambda: cp.ulysses_unpack(send, P, cp.SEQ_TO_HEAD, dst=heads, stream=stream))
    out["unpack_s2h_us"] = round(ms * 1e3, 2)
    out["unpack_s2h_GBps"] = round(nbytes / ms / 1e6, 1)
    out.update(cold_rows(cp, torch, stream))
    out.update(p4_rows(cp, torch, stream))
    out.update(fp8_rows(cp, torch, stream))
    # self-attention S=44160 with K stored sequence-last ([1,24,128,44160], the attention sample's
    # hint-file layout for K), Q, V, O head-major, its planned workspace
    kt_ = k.transpose(2, 3).contiguous()
    o_kt = torch.empty_like(q)
    l_kt = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
    ws_kt = workspace(cp, torch, 1, H, inputs.S_VIDEO, inputs.S_VIDEO, D)
    out["self_k_seq_last"] = timed_leg(
        torch, stream, lambda: cp.attn_fwd_ex(q, kt_, v, o=o_kt, lse=l_kt, workspace=ws_kt, k_seq_last=True,
                                              stream=stream), 4.0 * H * inputs.S_VIDEO ** 2 * D, iters=20)
    del kt_, o_kt, l_kt, ws_kt
    return out


PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 matrix-core peak (twice bf16)


def fp8_rows(cp, torch, stream):
    """Self-attention S=44160, H=24, D=128 with E4M3 inputs (N(0,1) draws rounded to E4M3,
    scales 1) on the fp8 matrix cores with its planned workspace; O in bf16.  3 warm-ups, 50 calls timed one by one."""
    from long_sequence_bidirectional_amd import inputs
    S, H, D = inputs.S_VIDEO, inputs.N_HEADS, inputs.HEAD_DIM
    q8, k8, v8 = (torch.from_numpy(inputs.random_e4m3((1, H, S, D), 7300 + i)).cuda() for i in range(3))
    o = torch.empty((1, H, S, D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, H, S), dtype=torch.float32, device="cuda")
    flops = 4.0 * H * S * S * D
    ws = torch.empty(cp.attn_fwd_workspace_size(1, H, S, S, D, cp.E4M3, cp.BF16), dtype=torch.uint8, device="cuda")
    leg = timed_leg(torch, stream, lambda: cp.attn_fwd_fp8(q8, k8, v8, o=o, lse=lse, workspace=ws, stream=stream),
                    flops)
    tf = flops / leg["ms_median"] / 1e9
    leg.pop("frac_of_bf16_peak", None)
    leg["frac_of_fp8_peak"] = round(tf / PEAK_FP8_TFLOPS, 4)
    return {"fp8_self": leg, "fp8_self_ms": leg["ms_median"], "fp8_self_tflops": round(tf, 1),
            "fp8_self_frac_of_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}


def p4_rows(cp, torch, stream, iters=50):
    """The attention sample of "TensorRT multi-device attention inference in practice":
    fp16 (seq, batch=1, 32, 128) tensors, QK-RMSNorm prologue (eps 1e-6, weights, cast to
    fp16, (1/128)^(1/4) on each of Q and K), then attention; timed as the sample times it,
    1 warm-up and 50 iterations.  Single-device run: S = 56320; one rank of two under
    AllGather-KV: its 28160 query rows against the gathered 56320 keys (the K prologue runs
    on the gathered keys, the Q prologue on the local rows)."""
    import numpy as np
    from long_sequence_bidirectional_amd import inputs
    S, H, D = inputs.P4_SEQ, inputs.P4_HEADS, inputs.HEAD_DIM
    S_r = S // inputs.P4_RANKS
    g = inputs.p4_set()
    q, k, v, wq, wk = (torch.from_numpy(np.ascontiguousarray(g[n])).cuda() for n in ("q", "k", "v", "w_q", "w_k"))
    s4 = D ** -0.25
    qn, kn = torch.empty_like(q), torch.empty_like(k)
    out = {}
    for name, Sq in (("p4_single", S), ("p4_rank", S_r)):
        qs, qns = q[:, :Sq], qn[:, :Sq]
        o = torch.empty((1, Sq, H, D), dtype=torch.float16, device="cuda")
        lse = torch.empty((1, H, Sq), dtype=torch.float32, device="cuda")
        ws = torch.empty(cp.attn_fwd_workspace_size(1, H, Sq, S, D, cp.F16, cp.F16), dtype=torch.uint8,
                         device="cuda")

        def prologue():
            cp.qk_rmsnorm(qs, wq, 1e-6, s4, out=qns, stream=stream)
            cp.qk_rmsnorm(k, wk, 1e-6, s4, out=kn, stream=stream)

        def attn():
            cp.attn_fwd_ex(qns, kn, v, o=o, lse=lse, scale=1.0, workspace=ws, seq_major=True, stream=stream)

        def layer():
            prologue()
            attn()

        def timed(fn):
            fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(iters):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / iters

        ms_layer, ms_attn, ms_pro = timed(layer), timed(attn), timed(prologue)
        flops = 4.0 * H * Sq * S * D
        out[f"{name}_ms"] = round(ms_layer, 3)
        out[f"{name}_attn_tflops"] = round(flops / ms_attn / 1e9, 1)
        out[f"{name}_prologue_ms"] = round(ms_pro, 3)
        out[f"{name}_prologue_GBps"] = round(2 * 2 * (Sq + S) * H * D / ms_pro / 1e6, 1)
    return out


def cold_rows(cp, torch, stream, n_sets=12):
    """Merge and relayout on rotating buffer sets larger than the 256 MB MALL, so every
    call reads its inputs from HBM (reported beside the hot figures)."""
    from long_sequence_bidirectional_amd import inputs
    S_L, P, H, D = inputs.S_LOCAL, inputs.CP_DEGREE, inputs.N_HEADS, inputs.HEAD_DIM
    out = {}

    def rotate(fns):
        for f in fns:
            f()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for f in fns:
            f()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / len(fns)

    # merge: n_sets x (o_a, o_b f32 [1,24,5520,128] + LSEs), in place into o_a: 814 MB of inputs
    sets = []
    for _ in range(n_sets):
        oa = torch.randn((1, H, S_L, D), device="cuda")
        la = torch.randn((1, H, S_L), device="cuda")
        ob = torch.randn((1, H, S_L, D), device="cuda")
        lb = torch.randn((1, H, S_L), device="cuda")
        sets.append((oa, la, ob, lb))
    fns = [lambda t=t: cp.attn_merge(t[0], t[1], t[2], t[3], o_out=t[0], lse_out=t[1], stream=stream) for t in sets]
    ms = rotate(fns)
    nbytes = 3 * sets[0][0].numel() * 4 + 3 * sets[0][1].numel() * 4
    out["merge_f32_cold_us"] = round(ms * 1e3, 2)
    out["merge_f32_cold_GBps"] = round(nbytes / ms / 1e6, 1)
    del sets, fns
    # relayout: n_sets x (shard [1,5520,24,128] bf16 -> send buffer): 814 MB touched
    shards = [torch.randn((1, S_L, H, D), device="cuda").to(torch.bfloat16) for _ in range(n_sets)]
    sends = [torch.empty((1, P, S_L, H // P, D), dtype=torch.bfloat16, device="cuda") for _ in range(n_sets)]
    fns = [lambda a=a, b=b: cp.ulysses_pack(a, P, cp.SEQ_TO_HEAD, dst=b, stream=stream) for a, b in zip(shards, sends)]
    ms = rotate(fns)
    nbytes = 2 * shards[0].numel() * 2
    out["pack_s2h_cold_us"] = round(ms * 1e3, 2)
    out["pack_s2h_cold_GBps"] = round(nbytes / ms / 1e6, 1)
    fns = [lambda a=a, b=b: cp.ulysses_unpack(b, P, cp.SEQ_TO_HEAD, dst=a.view(1, H // P, S_L * P, D), stream=stream)
           for a, b in zip(shards, sends)]
    ms = rotate(fns)
    out["unpack_s2h_cold_us"] = round(ms * 1e3, 2)
    out["unpack_s2h_cold_GBps"] = round(nbytes / ms / 1e6, 1)
    # the same shards as n_sets / 3 batched calls of three (one rank's Q, K, V in one launch)
    groups = [list(range(i, i + 3)) for i in range(0, n_sets - n_sets % 3, 3)]
    fns = [lambda g=g: cp.ulysses_pack_n([shards[i] for i in g], P, cp.SEQ_TO_HEAD, dsts=[sends[i] for i in g],
                                         stream=stream) for g in groups]
    ms = rotate(fns)
    out["pack_qkv_s2h_cold_us"] = round(ms * 1e3, 2)
    out["pack_qkv_s2h_cold_GBps"] = round(3 * nbytes / ms / 1e6, 1)
    fns = [lambda g=g: cp.ulysses_unpack_n([sends[i] for i in g], P, cp.SEQ_TO_HEAD,
                                           dsts=[shards[i].view(1, H // P, S_L * P, D) for i in g], stream=stream)
           for g in groups]
    ms = rotate(fns)
    out["unpack_qkv_s2h_cold_us"] = round(ms * 1e3, 2)
    out["unpack_qkv_s2h_cold_GBps"] = round(3 * nbytes / ms / 1e6, 1)
    return out


if __name__ == "__main__":
    main()
