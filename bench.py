"""Benchmark: paged-FP8 MLA decode on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload uniform]

A step is one decode call (one launch: the decode workgroups, and the split
merge workgroups when the plan splits) over one layer of a resident multi-layer paged FP8 cache.  Consecutive steps
decode consecutive layers, as a model's per-layer calls do; the cache holds
enough layers (>= 512 MiB) that no step finds its layer in the 256 MB
Infinity Cache, and 512 MiB are streamed through that cache before each
timed workload's warm-up.  Inputs are drawn once (synthetic, seeded) and stay
in HBM.  By default the ragged, long-context and speculative workloads are
timed first, back to back, and the headline (uniform) workload last, so that
it runs at the clocks of a busy GPU.

Prints one JSON line: KV tokens/s over the whole step (value), the main
kernel's achieved rate against its roofline (timed inside the timed region
with HIP events that carry the main kernel's own start and end, on every
--event-every-th step: each event-carrying launch adds several microseconds
to the steps around it, ~1.3 us per step on the uniform workload at every
5th step, ~0.8 at every 10th), and the FP64 oracle timed on the host cores over the
same workload (one layer) as a reported baseline.
"""

import argparse
import ctypes
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_MFMA16_TFLOPS = 2500.0      # MI355X dense FP16/BF16 MFMA
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
MALL_BYTES = 256 << 20
WORKLOADS = ("uniform", "ragged", "long1", "long4", "spec", "chunk", "tiny")
KERNEL_SRC = os.path.join(ROOT, "mla_decode_attention_paged_amd", "csrc", "mla_decode.hip")
KERNEL_SRC_BF16 = os.path.join(ROOT, "mla_decode_attention_paged_amd", "csrc", "mla_decode_bf16.hip")
UNIT_ORDER_SRC = os.path.join(ROOT, "mla_decode_attention_paged_amd", "csrc", "unit_order.h")
SPLIT_MERGE_SRC = os.path.join(ROOT, "mla_decode_attention_paged_amd", "csrc", "split_merge.h")

# HBM traffic of one decode launch, from two rocprofv3 --pmc runs of
# `bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-configs` (FETCH_SIZE,
# then WRITE_SIZE, KiB per dispatch, averaged over the dispatches), each
# scaled by what the same counter reads for a plain 1 GiB device copy
# (`bench.py --calibrate-copy`: FETCH_SIZE 524,302.5 KiB and WRITE_SIZE
# 1,048,576 KiB for 1,048,576 KiB moved).  Beyond the algorithmic bytes the
# launch writes the split partials (workspace) and its merge workgroups read
# them back.  Keyed by the SHA-256 of the device code the counters were taken
# on (kernel_digest): any later edit of a kernel makes the figure stale and
# bench reports traffic as null.
_COPY_KIB = 1048576.0
_FETCH_PER_KIB = 524302.5 / _COPY_KIB
_WRITE_PER_KIB = 1048576.0 / _COPY_KIB
MEASURED_TRAFFIC = {
    "329ebabe2b27f1484e335737f2bd2331e4ead10d31b1b0ea8282cb8545381893": {
        "uniform_b16_l4096": {"fetch_kib": 36451.3, "write_kib": 34922.0},
        "ragged_b64": {"fetch_kib": 95204.7, "write_kib": 40045.9},
        "long_b1": {"fetch_kib": 54476.7, "write_kib": 32997.1},
        "long_b4": {"fetch_kib": 170616.7, "write_kib": 33385.2},
        "spec_b128": {"fetch_kib": 697664.3, "write_kib": 65536.0},
    },
    # unquantized (bf16) cache kernel, the same runs with `--op bf16`
    "641ccc1eae71d3df27dbb8e43e4d7c38f65a6cc532418ac8f90c6233ea21a5b5": {
        "uniform_bf16_b16_l4096": {"fetch_kib": 54762.9, "write_kib": 34922.0},
    },
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def make(name, device, unquantized=False):
    from mla_decode_attention_paged_amd import synth
    if unquantized:
        # the same shapes over an unquantized (bf16) cache
        if name == "uniform":
            return synth.uniform_bf16(device=device)
        if name in ("long1", "long4"):
            B = 1 if name == "long1" else 4
            return synth.make_workload(B, 128, [131072] * B, 128, 576, seed=3000, device=device, poison=False,
                                       kv_dtype="bf16", name=f"long_bf16_b{B}")
        if name == "tiny":
            return synth.make_workload(2, 16, [37, 100], 16, 576, spare_blocks=6, seed=0, device=device,
                                       poison=False, kv_dtype="bf16", name="tiny_bf16")
        raise ValueError(f"workload {name} has no unquantized form here")
    if name == "uniform":
        return synth.uniform(device=device)
    if name == "ragged":
        return synth.ragged(device=device)
    if name == "long1":
        return synth.long_context(device=device, batch=1)
    if name == "long4":
        return synth.long_context(device=device, batch=4)
    if name == "spec":
        return synth.speculative(device=device)
    if name == "chunk":
        return synth.query_chunk(device=device)
    if name == "tiny":
        return synth.tiny(device=device, poison=False)
    raise ValueError(name)


def replicate_layers(w, min_bytes):
    """Give the cache enough layers that consecutive steps never share a cached layer."""
    import torch
    NB, KVD, NL, P, HK, D = w.blocks.shape
    layer_bytes = NB * P * D * w.blocks.element_size()
    if w.scales is not None:
        layer_bytes += w.scales.shape[0] * P * w.scales.shape[-1] * 4
    n = max(NL, int(math.ceil(min_bytes / layer_bytes)))
    if n == NL:
        return w, list(range(NL)) if NL > 1 else [w.layer_idx]
    src_b = w.blocks[:, :, w.layer_idx:w.layer_idx + 1]
    blocks = src_b.expand(NB, KVD, n, P, HK, D).contiguous()
    scales = None
    if w.scales is not None:
        src_s = w.scales[:, :, w.layer_idx:w.layer_idx + 1]
        scales = src_s.expand(w.scales.shape[0], KVD, n, P, HK, w.scales.shape[-1]).contiguous()
    torch.cuda.synchronize()
    w2 = type(w)(**{**w.__dict__, "blocks": blocks, "scales": scales, "layer_idx": 0})
    return w2, list(range(n))


_FLUSH = []


def flush_infinity_cache(dev):
    """Stream twice the Infinity Cache's capacity through it (a 512 MiB copy:
    reads and writes), so that no data laid out before, such as the freshly
    replicated layers, is still cached when a timed run starts."""
    import torch
    if not _FLUSH:
        n = 2 * MALL_BYTES
        _FLUSH.extend([torch.empty(n, dtype=torch.uint8, device=dev), torch.ones(n, dtype=torch.uint8, device=dev)])
    _FLUSH[0].copy_(_FLUSH[1])
    torch.cuda.synchronize()


def algorithmic(w):
    """Algorithmic bytes and flops of one decode call on workload w."""
    lens = w.lengths()
    B, Q, H, D = w.q.shape
    P = w.page_size
    tables = 1 if w.scales_lookup_table is None else 2
    if w.scales is None:                      # unquantized: bf16 rows, no scales
        kv_bytes = sum(lens) * D * 2
    else:
        kv_bytes = sum(lens) * (D + 4 * w.scales.shape[-1])
    table_bytes = sum((L + P - 1) // P for L in lens) * 4 * tables
    io_bytes = B * Q * H * D * 2 + B * Q * H * 512 * 2 + 4 * B
    visible = sum(max(0, min(L, L - Q + i + 1)) for L in lens for i in range(Q))
    flops = visible * H * 2 * (D + 512)
    return kv_bytes + table_bytes + io_bytes, flops, sum(lens)


class HipEvents:
    """Raw HIP events (hipEvent_t) for timing the main kernel on the launch stream."""

    def __init__(self, n):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            self.ev.append(e.value)

    def pair(self, i):
        return self.ev[2 * i], self.ev[2 * i + 1]

    def elapsed_ms(self, i):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), *[ctypes.c_void_p(x) for x in self.pair(i)]) == 0
        return ms.value

    def elapsed_to_torch_event_ms(self, i, tev):
        """From the end event of pair i to a later torch.cuda.Event on the same stream."""
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.pair(i)[1]),
                                            ctypes.c_void_p(tev.cuda_event)) == 0
        return ms.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def kernel_digest(unquantized=False):
    """SHA-256 of the device code in the kernel source (everything between the
    first device helper and the host launchers) and of the shared unit
    mapping (unit_order.h) and split merge (split_merge.h)."""
    import hashlib
    path = KERNEL_SRC_BF16 if unquantized else KERNEL_SRC
    with open(path, "r") as f:
        src = f.read()
    if unquantized:
        a = src.index("namespace bf16_path {")
        b = src.index("// ---------------------------------------------------------------- host launcher")
    else:
        a = src.index("// ---------------------------------------------------------------- page resolution")
        b = src.index("// ---------------------------------------------------------------- host launchers")
    with open(UNIT_ORDER_SRC, "r") as f:       # the workgroup -> unit mapping both kernels use
        order = f.read()
    with open(SPLIT_MERGE_SRC, "r") as f:
        merge = f.read()
    return hashlib.sha256((src[a:b] + order + merge).encode()).hexdigest()


def measured_traffic(workload, unquantized=False):
    """HBM bytes per main-kernel launch (read, written, total), or None."""
    m = MEASURED_TRAFFIC.get(kernel_digest(unquantized), {}).get(workload)
    if m is None:
        return None
    rd = m["fetch_kib"] * 1024 / _FETCH_PER_KIB
    wr = m["write_kib"] * 1024 / _WRITE_PER_KIB
    return {"read_bytes": rd, "write_bytes": wr, "total_bytes": rd + wr}


def calibrate_copy(n_bytes=1 << 30, reps=3):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"calibrate-copy: {reps} copies of {n_bytes} bytes (read {n_bytes}, write {n_bytes} each)")


def cpu_baseline(w):
    """The FP64 oracle, as it stands, timed on the host over one layer of w."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from tests.oracle_inputs import to_numpy
    from oracle import decode, decode_unquantized
    wc = w.to("cpu")
    q, blocks, scales, lt, slt, cl = to_numpy(wc)
    blocks = np.ascontiguousarray(blocks[:, :, w.layer_idx:w.layer_idx + 1])
    if scales is None:
        def decode(q, blocks, scales, lt, slt, cl, layer, q_len, sm, batches):  # noqa: F811
            return decode_unquantized(q, blocks, lt, cl, layer, q_len, sm, batches=batches)
    else:
        scales = np.ascontiguousarray(scales[:, :, w.layer_idx:w.layer_idx + 1])
    # run requests in order, cycling, until about 10 s of CPU work is done
    budget_s = 10.0
    t0 = time.perf_counter()
    done_tokens, calls = 0, 0
    B = q.shape[0]
    while True:
        b = calls % B
        decode(q, blocks, scales, lt, slt, cl, 0, w.q_len, w.softmax_scale, batches=[b])
        done_tokens += int(cl[b])
        calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    pools = threadpool_info()
    blas = [i for i in pools if i.get("user_api") == "blas"]
    threads = max([i.get("num_threads", 1) for i in blas] or [1])
    return {"value": done_tokens / dt, "unit": "KV tokens/s", "cores": int(threads), "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas": ", ".join(f"{i.get('internal_api')} {i.get('version')} ({i.get('num_threads')} threads)"
                              for i in blas) or "none",
            "sample": f"{calls} single-request oracle calls cycling over the {B} requests of one layer of the "
                      f"same workload ({done_tokens} cached tokens, all {w.num_heads} heads, q_len {w.q_len}), "
                      f"{dt:.1f} s wall; cores = the BLAS threads the oracle's matrix products used"}


def bench_append(args, w):
    """Time the append-and-quantize kernel on the workload's shape (B requests x q_len new rows)."""
    import torch
    from mla_decode_attention_paged_amd import mla_append_kv_fp8
    dev = w.q.device
    B, Q = w.batch, w.q_len
    g = torch.Generator(device=dev)
    g.manual_seed(4242)
    kv = (torch.randn((B, Q, 576), generator=g, device=dev) *
          torch.exp(0.5 * torch.randn((B, Q, 1), generator=g, device=dev))).to(torch.bfloat16)
    NG = w.scales.shape[-1]
    tables = 1 if w.scales_lookup_table is None else 2
    alg_bytes = B * Q * (576 * 2 + 576 + 4 * NG + 4 * tables) + 4 * B

    def call():
        mla_append_kv_fp8(kv, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table, w.cache_lengths,
                          w.layer_idx, Q)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = sum(a.elapsed_time(b) for a, b in ev) / len(ev)
    gbs = alg_bytes / (kern_ms * 1e-3) / 1e9
    log(f"bench append: {kern_ms * 1e3:.2f} us/launch, {gbs:.1f} GB/s algorithmic ({alg_bytes} B)")
    print(json.dumps({
        "metric": "KV append + quantize (paged FP8), 1 MI355X", "value": B * Q / (kern_ms * 1e-3),
        "unit": "rows/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": (t1 - t0) * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16-in/fp8e4m3+fp32-scales-out", "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "q_len": Q, "granularity": w.granularity,
                   "page_size": w.page_size},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None, "kernel": "mla_append_kernel",
                     "kernel_avg_us": kern_ms * 1e3, "alg_bytes_per_launch": alg_bytes},
    }), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="uniform", choices=WORKLOADS)
    ap.add_argument("--splits", type=int, default=None, help="explicit split count (default: library plan)")
    ap.add_argument("--fp8-mfma", choices=["v", "kv"], default=None,
                    help="contractions on the FP8 MFMA: v = P'V (mla_decode_paged_fp8_mfma8), kv = QK^T and P'V "
                         "(mla_decode_paged_fp8_mfma8_kv); per-token scales")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="time only the selected workload (by default the uniform headline line also carries "
                         "the ragged, long-context and speculative workloads in its 'configs' object)")
    ap.add_argument("--op", default="decode", choices=("decode", "append", "bf16"),
                    help="decode (default, the headline line); append: the KV append-and-quantize "
                         "kernel for the workload's q_len new tokens per request; bf16: decode over "
                         "an unquantized bf16 cache of the workload's shape")
    ap.add_argument("--event-every", type=int, default=10,
                    help="time the main kernel with HIP events on every k-th timed step (events on "
                         "every launch add several microseconds of launch overhead per step)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not part "
              "of this build", file=sys.stderr)
        sys.exit(2)

    if args.calibrate_copy:
        calibrate_copy()
        return
    import torch
    from mla_decode_attention_paged_amd import lib_path

    dev = torch.device("cuda:0")
    log(f"bench: workload {args.workload}, op {args.op}, library {lib_path()}")
    unq = args.op == "bf16"
    w = make(args.workload, dev, unquantized=unq)
    if args.op == "append":
        bench_append(args, w)
        return
    configs = None
    if not args.no_configs and not unq and args.workload == "uniform" and args.splits is None:
        # the other workloads of the same path, each timed the same way, before
        # the headline, all generated and laid out first and then timed back to
        # back, longest first: the GPU raises its clocks only after ~10-20 ms of
        # sustained work and drops them again after ~50 ms idle, so the
        # generation of one workload between the timings of others would
        # leave each timed region to start on a GPU that has cooled down
        names = ("spec", "ragged", "long1", "long4")
        preps = {name: prepare_decode(make(name, dev), None) for name in names}
        configs = {}
        for name in names:
            steps, warm = (20, 3) if name == "spec" else (50, 5)
            rc = time_decode(preps.pop(name), steps, warm, args.event_every, False)
            rf = rc["roofline"]
            configs[rc["name"]] = {
                "kv_tokens_per_s": rc["kv_tokens"] / (rc["ms_per_step"] * 1e-3), "steps": steps,
                "step_us": rc["ms_per_step"] * 1e3, "main_kernel_us": rf["kernel_avg_us"],
                "after_main_us": rc["after_main_us"], "frac": rf["frac"], "step_frac": rf["step_frac"],
                "bound": rf["bound"], "alg_flops": rf["alg_flops_per_launch"], "alg_bytes": rf["alg_bytes_per_launch"],
                "traffic": rf["traffic"], "plan": rc["plan"]}
    # the headline's layers are replicated right before it is timed (measured
    # 1-2 us per step faster than replicating them before the other workloads)
    prep = prepare_decode(w, args.splits)
    r = time_decode(prep, args.steps, args.warmup, args.event_every, unq, args.fp8_mfma)
    del prep
    result = {
        "metric": "MLA decode KV tokens/s + achieved GB/s & MFMA util vs roofline, 1 MI355X",
        "value": r["kv_tokens"] / (r["ms_per_step"] * 1e-3),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16-kv/bf16-mfma/fp32-acc" if unq else "fp8e4m3-kv/bf16+f16-mfma/fp32-acc",
        "data": ("synthetic (seeded; N(0,1) x LogNormal(0,0.5) latent rows stored as bf16)" if unq else
                 "synthetic (seeded; N(0,1) x LogNormal(0,0.5) latent rows quantised to E4M3FN)"),
        "config": {"workload": w.name, "batch": w.batch, "q_len": w.q_len, "num_heads": w.num_heads,
                   "page_size": w.page_size, "granularity": None if unq else w.granularity,
                   "kv_tokens_per_step": r["kv_tokens"], "layers_rotated": r["layers"], "plan": r["plan"]},
        "roofline": r["roofline"],
    }
    if unq:
        result["metric"] = "MLA decode over an unquantized bf16 paged cache, KV tokens/s, 1 MI355X"
    if configs is not None:
        result["configs"] = configs
        result["config"]["timed_after"] = "the configs' workloads (sustained clocks)"
    if not args.no_cpu_baseline:
        log("bench: timing the FP64 oracle on the host (bounded sample)")
        result["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(result), flush=True)


def prepare_decode(w, splits):
    """Everything a timed decode run needs, allocated up front: the workload
    replicated over enough layers to defeat the Infinity Cache, the plan, the
    output and the workspace."""
    import torch
    from mla_decode_attention_paged_amd import mla_decode_paged_fp8_plan, new_workspace
    dev = w.q.device
    w, layers = replicate_layers(w, 2 * MALL_BYTES)
    scales_shape = tuple(w.scales.shape) if w.scales is not None else (1,) + tuple(w.blocks.shape[1:5]) + (1,)
    plan = mla_decode_paged_fp8_plan(tuple(w.q.shape), tuple(w.blocks.shape), scales_shape,
                                     tuple(w.lookup_table.shape), w.q_len, splits or 0)
    out = torch.empty((w.batch, w.q_len, w.num_heads, 512), dtype=torch.bfloat16, device=dev)
    ws = new_workspace(plan["workspace_bytes"], dev)   # allocated and its counters zeroed once
    return {"w": w, "layers": layers, "plan": plan, "out": out, "ws": ws, "splits": splits}


def time_decode(prep, steps, warmup, event_every, unq, fp8_mfma=None):
    """Time `steps` decode calls on a prepared workload (after `warmup` untimed
    ones); returns the step rate, the main kernel's own time and the roofline
    record."""
    import torch
    from mla_decode_attention_paged_amd import mla_decode_paged_bf16, mla_decode_paged_fp8
    w, layers, plan, out, ws, splits = (prep[k] for k in ("w", "layers", "plan", "out", "ws", "splits"))
    alg_bytes, alg_flops, kv_tokens = algorithmic(w)
    log(f"bench: {w.name}: layers {len(layers)}, plan {plan}, kv tokens/step {kv_tokens}")
    every = max(1, event_every)
    timed = [i for i in range(steps) if i % every == 0]
    ev = HipEvents(len(timed))
    after = torch.cuda.Event(enable_timing=True)   # (after the first timed launch only)

    def step(i, events=None):
        if unq:
            mla_decode_paged_bf16(w.q, w.blocks, w.lookup_table, w.cache_lengths, layers[i % len(layers)],
                                  w.q_len, w.softmax_scale, out=out, workspace=ws, num_splits=splits,
                                  main_events=events)
        else:
            mla_decode_paged_fp8(w.q, w.blocks, w.scales, w.lookup_table, w.scales_lookup_table,
                                 w.cache_lengths, layers[i % len(layers)], w.q_len, w.softmax_scale,
                                 out=out, workspace=ws, num_splits=splits, main_events=events,
                                 fp8_mfma=fp8_mfma)

    flush_infinity_cache(w.q.device)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if i % every == 0:
            step(warmup + i, ev.pair(i // every))
            if i == 0:
                after.record()
        else:
            step(warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    kern_ms = [ev.elapsed_ms(k) for k in range(len(timed))]
    # decode launch end -> the call's last work on the stream (nothing else is
    # launched since the split merge joined the decode launch: the gap only),
    # on the first timed launch
    after_ms = [ev.elapsed_to_torch_event_ms(0, after)]
    ev.close()
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    tflops = alg_flops / (kern_avg_ms * 1e-3) / 1e12
    gbs = alg_bytes / (kern_avg_ms * 1e-3) / 1e9
    step_tflops = alg_flops / (ms_per_step * 1e-3) / 1e12
    log(f"bench: {w.name}: {ms_per_step * 1e3:.1f} us/step, main kernel {kern_avg_ms * 1e3:.1f} us "
        f"(min {min(kern_ms) * 1e3:.1f}), {tflops:.0f} TFLOP/s, {gbs:.0f} GB/s algorithmic")
    traffic = measured_traffic(w.name, unq)
    if unq:
        # arithmetic intensity below the 16-bit ridge (flop per byte < 312.5): HBM binds
        roof = {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                "step_frac": alg_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBS,
                "traffic": (traffic or {}).get("total_bytes"), "traffic_detail": traffic,
                "kernel": "mla_decode_bf16_kernel", "kernel_avg_us": kern_avg_ms * 1e3,
                "kernel_timed_launches": len(timed), "alg_flops_per_launch": alg_flops,
                "alg_bytes_per_launch": alg_bytes, "alg_TFLOPs": tflops, "mfma_frac": tflops / PEAK_MFMA16_TFLOPS}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": PEAK_MFMA16_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_MFMA16_TFLOPS,
                "step_frac": step_tflops / PEAK_MFMA16_TFLOPS,
                "frac_note": "frac: the decode launch (its split merge included); step_frac: the whole "
                             "call per step, launch gaps included",
                "traffic": (traffic or {}).get("total_bytes"),
                "traffic_detail": traffic,
                "kernel": "mla_decode_kernel", "kernel_avg_us": kern_avg_ms * 1e3,
                "kernel_timed_launches": len(timed),
                "alg_flops_per_launch": alg_flops, "alg_bytes_per_launch": alg_bytes,
                "alg_GBps": gbs, "hbm_frac": gbs / PEAK_HBM_GBS}
    return {"name": w.name, "ms_per_step": ms_per_step, "kv_tokens": kv_tokens, "layers": len(layers), "plan": plan,
            "roofline": roof, "after_main_us": 1e3 * sum(after_ms) / len(after_ms)}


if __name__ == "__main__":
    main()
