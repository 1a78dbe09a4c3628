"""Benchmark of the weight-only quantized linear on one MI355X.

One step = one decode pass of the W8A16 per-channel projection set at M = 1
token: wq_linear (-> split-K GEMV) on the four weight shapes (K, N) =
(5120, 27648) fused gate+up, (13824, 5120) down, (5120, 7168) fused QKV,
(6144, 5120) out-proj.  Weights are int8 codes with bf16 per-channel scales, x is
bf16 ~ N(0, 1), y bf16.  Every call reads a different copy of its weight from a
rotation pool of >= 1.28 GB per shape (five times the 256 MB Infinity Cache), so
the weights come from HBM, as in the Marlin benchmark page's fixed-input
projection check (weights rotating over more than five times the cache, each
captured graph running whole rotations).  The timed steps run as one HIP graph
replay; split_k is tuned per shape first, as the awq heuristic page describes
(grid {1..32}, 1000 warm-up + 1000 timed calls).

The headline value is whole-step weight-stream throughput in GB/s of
algorithmic bytes (packed codes + scales + x + y, each counted once).  The JSON
line also carries the roofline of the GEMV kernel, the CPU oracle timed on the
host cores, and (unless --quick) per-shape detail for the other workloads: the
W8A16 M sweep, W4A16 group-128 GEMV, the split-K stress shapes and the prefill
GEMM (TFLOP/s against the bf16 MFMA peak).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
ROTATE_BYTES = 1.28e9           # >= 5 x 256 MB Infinity Cache
METRIC = "W8A16/W4A16 GEMV weight GB/s & % HBM peak at M=1; prefill GEMM TFLOP/s"
DECODE_SHAPES = [(5120, 27648), (13824, 5120), (5120, 7168), (6144, 5120)]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_w8pc_decode_traffic.json")


def algorithmic_bytes(fmt: str, K: int, N: int, M: int) -> int:
    """Packed codes + scales (+ zeros) + x + y, each counted once."""
    G = K // (int(fmt[3:]) if fmt[2] == "g" else 128)  # groups per row of a grouped format
    if fmt == "w8pc":
        w = K * N + 2 * N
    elif fmt.startswith("w8g"):
        w = K * N + 2 * N * G
    elif fmt == "w4pc":  # one scale and zero-point per row (the gfx950 layout repeats them per group)
        w = K * N // 2 + 2 * N + (N // 8) * 4
    else:
        w = K * N // 2 + 2 * N * G + G * (N // 8) * 4
    return w + 2 * M * K + 2 * M * N


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class Pool:
    """Rotation pool of identical packed copies of one seeded weight on the GPU."""

    def __init__(self, wq, torch, cfg: int, fmt: str, K: int, N: int, M: int, min_copies: int = 2,
                 act: str = "bf16"):
        import synth
        self.fmt, self.K, self.N, self.M, self.cfg, self.act = fmt, K, N, M, cfg, act
        W = synth.weight(cfg, K, N, synth.uses_outliers(fmt))
        Wd = torch.from_numpy(W).to("cuda")
        base = wq.quantize(Wd, fmt)
        del Wd
        self.W = W
        n = max(min_copies, int(np.ceil(ROTATE_BYTES / base.nbytes())))
        self.copies = [base] + [base.clone() for _ in range(n - 1)]
        xb = synth.activation_f16(cfg, K, M) if act == "f16" else synth.activation(cfg, K, M)
        dt = torch.float16 if act == "f16" else torch.bfloat16
        self.x_bits = xb
        self.x = torch.from_numpy(xb.view(np.int16)).to("cuda").view(dt)
        self.y = torch.empty((M, N), dtype=dt, device="cuda")
        self.ws = wq.workspace(wq.wq_workspace_size(base, M))
        self.i = 0

    def call(self, wq):
        w = self.copies[self.i]
        self.i = (self.i + 1) % len(self.copies)
        if self.act == "f16":
            wq.wq_linear_act(w, self.x, self.y, ws=self.ws)
        else:
            wq.wq_linear(w, self.x, self.y, ws=self.ws)

    def bytes_per_call(self) -> int:
        return algorithmic_bytes(self.fmt, self.K, self.N, self.M)

    def check(self, wq, torch, cols: int = 128, full_elems: int = 1 << 28) -> dict:
        """Parity of copy 0 against the oracle -- on every output channel for the GEMV
        (M < 8) when K * N <= full_elems, else on sampled channels -- and every copy's
        y bit-identical to copy 0's (a determinism check)."""
        import oracle
        ys = []
        for _ in range(len(self.copies)):
            self.call(wq)
            ys.append(self.y.clone())
        torch.cuda.synchronize()
        same = all(torch.equal(ys[0], t) for t in ys[1:])
        del ys
        self.i = 0
        self.call(wq)
        torch.cuda.synchronize()
        if self.M < 8 and self.K * self.N <= full_elems:
            rows = np.arange(self.N)
        else:
            blocks = np.unique(np.linspace(0, self.N // 8 - 1, cols // 8).astype(int))
            rows = (blocks[:, None] * 8 + np.arange(8)[None, :]).ravel()
        P = oracle.pack(self.fmt, self.W[rows])
        y = self.y.view(torch.int16).cpu().numpy().view(np.uint16)[:, rows]
        st = oracle.compare(y, oracle.ref_linear(self.x_bits, P, act=self.act), act=self.act)
        st["channels_checked"] = int(len(rows))
        st["copies_bit_identical"] = bool(same)
        self.i = 0
        return st

    def free(self):
        self.copies = []
        self.W = None


SETTLE_S = 1.0   # untimed replays before a timed measurement (see time_graph)


def time_graph(torch, fn, n_calls: int, reps: int = 9, stats: dict | None = None, settle_s: float | None = None):
    """Capture n_calls of fn() in one HIP graph; after 2 warm-up replays and `settle_s`
    seconds of untimed replays return the median of `reps` timed replays (ms), measured
    with HIP events on the capturing stream (min and max go into `stats` when given).

    The settle phase is there because MI355X's memory-side clocks rise under sustained
    memory-bound load: the W8 (5120, 27648) M = 1 GEMV measured 26.9 us from cold, 23.6 us
    after 45 s of GEMV load and 27.9 us again after 20 s idle (45 s of compute-bound
    matmuls left it at 26.4 us), so a short timing right after setup sees the idle clocks,
    not the steady state of a serving loop."""
    settle_s = SETTLE_S if settle_s is None else settle_s
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(n_calls):
                fn()
        torch.cuda.synchronize()
        g.replay()
        g.replay()
        torch.cuda.synchronize()
        t_end = time.perf_counter() + settle_s
        while time.perf_counter() < t_end:
            for _ in range(4):
                g.replay()
            torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
    del g
    if stats is not None:
        stats.update(min_ms=float(min(times)), max_ms=float(max(times)), reps=reps)
    return float(np.median(times))


def device_warmup(torch):
    """100 bf16 8192 x 8192 products (the awq heuristic page's device warm-up)."""
    a = torch.randn((8192, 8192), device="cuda", dtype=torch.bfloat16)
    for _ in range(100):
        torch.mm(a, a)
    torch.cuda.synchronize()


def tune(wq, pool: Pool, warmup: int, iters: int):
    x, y = pool.x, pool.y
    if pool.act == "f16":  # the tuner times bf16 calls; the fp16 layer takes its choice
        import synth
        import torch
        xb = synth.activation(pool.cfg, pool.K, pool.M)
        x = torch.from_numpy(xb.view(np.int16)).to("cuda").view(torch.bfloat16)
        y = torch.empty((pool.M, pool.N), dtype=torch.bfloat16, device="cuda")
    chosen, lat = wq.wq_tune(pool.copies, x, y, pool.ws, warmup=warmup, iters=iters)
    return chosen, lat


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas_build() -> str:
    try:
        b = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        return f"{b.get('name', '?')} {b.get('version', '?')}"
    except Exception:  # pragma: no cover
        return "unknown"


def cpu_baseline(budget_s: float = 12.0) -> dict:
    """The oracle (dequantise to fp32 + fp64 matmul) on the host cores, over the
    same four weights at M = 1, repeated until budget_s of CPU work.  BLAS threads
    are pinned to the usable cores (capped by OMP_NUM_THREADS where the host sets
    it); the quantise + pack of the four weights is timed separately."""
    import oracle
    import synth
    usable = len(os.sched_getaffinity(0))
    want = min(usable, int(os.environ.get("OMP_NUM_THREADS", "0") or usable))
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(limits=want)
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        limiter, threads = None, 1
    packed, pack_s = [], 0.0
    for K, N in DECODE_SHAPES:
        W = synth.weight(2, K, N)
        t = time.perf_counter()
        P = oracle.pack("w8pc", W)
        pack_s += time.perf_counter() - t
        packed.append((P, synth.activation(2, K, 1), K, N))
        del W
    done_bytes, t0, passes = 0, time.perf_counter(), 0
    while True:
        for P, x, K, N in packed:
            oracle.ref_linear(x, P)
            done_bytes += algorithmic_bytes("w8pc", K, N, 1)
        passes += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    return {"value": round(done_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu": _cpu_model(), "blas": _blas_build(), "usable_cores": usable,
            "seconds": round(dt, 2), "pack_seconds": round(pack_s, 2),
            "sample": f"{passes} passes of the oracle's dequantise + fp64 matmul over the 4 decode weights "
                      f"at M=1 (the headline step's work); elementwise dequant on 1 thread, BLAS on {threads}"}


def traffic_entry(kernel_src_sha: str):
    """Measured HBM bytes per launch of the dominant kernel (rocprofv3 FETCH_SIZE +
    WRITE_SIZE, scaled by a plain copy kernel), only while the GEMV source is the
    one the counters were taken with."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        d = json.load(open(TRAFFIC_FILE))
    except Exception:
        return None
    if d.get("kernel_src_sha256") != kernel_src_sha:
        return None
    return d.get("bytes_per_step_avg_launch")


# Launch configuration of the headline GEMV per shape (split_k, waves, rows) used by
# the counter pass, so the profiled kernels are the ones the tuner picks on MI355X.
PROFILE_CONFIG = {(5120, 27648): (1, 3, 4 | 0x100), (13824, 5120): (1, 6, 4), (5120, 7168): (1, 1, 4 | 0x100),
                  (6144, 5120): (1, 6, 4)}
COPY_BYTES = 1 << 30


def streaming_settle(torch, seconds: float = 5.0):
    """Untimed memory-bound work (a 1 GiB elementwise kernel, a few dispatches a
    millisecond) so that the memory-side clocks reach their steady state before a
    profiled workload, without adding thousands of the profiled kernel's dispatches to
    the trace (see time_graph)."""
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(8):
            torch.bitwise_not(a, out=b)
        torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def profile_pass(steps: int = 10, replays: int = 2):
    """Kernels for a rocprofv3 run: the elementwise reference (COPY_BYTES in and out,
    the scale for FETCH_SIZE / WRITE_SIZE), then the headline step exactly as the
    timed region runs it -- one HIP graph of `steps` steps (4 GEMV launches each, in
    DECODE_SHAPES order, rotating weight copies), replayed `replays` times -- with
    each shape's tuned launch configuration fixed to PROFILE_CONFIG."""
    import torch
    import gemm_decode_amd.wq as wq
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.bitwise_not(a, out=b)  # one elementwise dispatch: COPY_BYTES read, COPY_BYTES written
    torch.cuda.synchronize()
    del a, b
    pools = []
    for K, N in DECODE_SHAPES:
        pools.append(Pool(wq, torch, 2, "w8pc", K, N, 1))
        split, waves, rows = PROFILE_CONFIG[(K, N)]
        wq.wq_tune_cache_set("w8pc", K, N, 1, wq.KIND_GEMV, wq.gemv_cache_value(split, waves, rows))

    def step():
        for p in pools:
            p.call(wq)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                step()
        torch.cuda.synchronize()
        streaming_settle(torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(replays):
            g.replay()
        e1.record(s)
        torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (replays * steps)
    log(f"profile pass: {replays} replays x {steps} steps x {len(pools)} GEMV launches: {us:.2f} us per step "
        f"(HIP events), {sum(p.bytes_per_call() for p in pools) / us / 1e3:.0f} GB/s")


PREFILL_PROFILE = [("w8pc", 5120, 27648, 2048, 13), ("w4g128", 5120, 27648, 2048, 13)]


def profile_prefill(calls: int = 10):
    """Kernels for a rocprofv3 run of the prefill GEMM: the elementwise reference (the
    FETCH_SIZE / WRITE_SIZE scale, as in profile_pass), then for each (fmt, K, N, M,
    tile) of PREFILL_PROFILE `calls` wq_linear calls on rotating weight copies with the
    GEMM tile fixed, as one HIP graph replayed once."""
    import torch
    import gemm_decode_amd.wq as wq
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.bitwise_not(a, out=b)
    torch.cuda.synchronize()
    del a, b
    for fmt, K, N, M, tile in PREFILL_PROFILE:
        p = Pool(wq, torch, 5, fmt, K, N, M)
        wq.wq_tune_cache_set(fmt, K, N, M, wq.KIND_GEMM, tile)
        streaming_settle(torch, 3.0)
        ms = time_graph(torch, lambda: p.call(wq), calls, reps=1, settle_s=0.0)
        us = ms * 1e3 / calls
        log(f"profile prefill {fmt} K={K} N={N} M={M} tile={tile}: {us:.1f} us per call "
            f"(HIP events), {2.0 * M * K * N / us / 1e6:.1f} TFLOP/s")
        p.free()
        del p
        torch.cuda.empty_cache()


# Few-token GEMM rows for rocprofv3 (fmt, K, N, M, tile): the tiles the tuner picks on
# MI355X at 8 and 64 tokens on the widest decode shape.
FEWTOKEN_PROFILE = [("w4g128", 5120, 27648, 8, 22), ("w4g128", 5120, 27648, 64, 15),
                    ("w8pc", 5120, 27648, 8, 5), ("w8pc", 5120, 27648, 64, 15),
                    ("w4g128", 13824, 5120, 64, 25), ("w8pc", 13824, 5120, 64, 25)]


def profile_fewtoken(calls: int = 10):
    """Kernels for a rocprofv3 run of the few-token GEMM: the elementwise reference (the
    FETCH_SIZE / WRITE_SIZE scale), then for each row of FEWTOKEN_PROFILE `calls`
    wq_linear calls on rotating weight copies with the tile fixed, as one HIP graph
    replayed once (after its 2 eager warm-up calls), between a small torch.neg and a
    small torch.abs dispatch (the row's bounds for summarize_fewtoken)."""
    import torch
    import gemm_decode_amd.wq as wq
    a = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        torch.bitwise_not(a, out=b)
    torch.cuda.synchronize()
    del a, b
    mark = torch.zeros(64, device="cuda")
    for fmt, K, N, M, tile in FEWTOKEN_PROFILE:
        p = Pool(wq, torch, 5, fmt, K, N, M)
        wq.wq_tune_cache_set(fmt, K, N, M, wq.KIND_GEMM, tile)
        streaming_settle(torch, 2.0)
        torch.neg(mark, out=mark)
        torch.cuda.synchronize()
        ms = time_graph(torch, lambda: p.call(wq), calls, reps=1, settle_s=0.0)
        torch.abs(mark, out=mark)
        torch.cuda.synchronize()
        log(f"profile few-token {fmt} K={K} N={N} M={M} tile={tile}: {ms * 1e3 / calls:.1f} us per call (HIP events)")
        p.free()
        del p
        torch.cuda.empty_cache()


def summarize_fewtoken(trace_dir: str, fetch_dir: str, write_dir: str, out_txt: str):
    """Per row of FEWTOKEN_PROFILE (the dispatches between torch.neg separators): each
    kernel's dispatch count, mean duration (kernel trace), and median FETCH_SIZE /
    WRITE_SIZE per dispatch scaled by the elementwise reference; the call's bytes against
    the algorithmic bytes."""
    import glob

    def stream(d, pattern):
        rows = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            rows += _read_csv_rows(f)
        return sorted(rows, key=lambda r: int(r.get("Dispatch_Id", 0)))

    def short(name):
        return name.replace("void ", "").replace("wq::(anonymous namespace)::", "").split("(")[0]

    def by_row(rows):
        out, cur = [], None
        for r in rows:
            name = r["Kernel_Name"]
            if "neg_kernel" in name:
                cur = {}
                out.append(cur)
            elif "AbsFunctor" in name or "abs_kernel" in name:
                cur = None
            elif cur is not None:
                cur.setdefault(short(name), []).append(r)
        return out

    trace = by_row(stream(trace_dir, "*kernel_trace.csv"))
    if len(trace) != len(FEWTOKEN_PROFILE):
        raise SystemExit(f"found {len(trace)} row separators in the trace (full kernel names needed: no -T)")
    scale = {}
    counters = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = [r for r in stream(d, "*counter_collection.csv") if r["Counter_Name"] == counter]
        ref = [float(r["Counter_Value"]) for r in rows if "bitwise_not" in r["Kernel_Name"]]
        if not ref:
            raise SystemExit("reference kernel counters missing")
        scale[counter] = COPY_BYTES / float(np.median(ref))  # bytes per counter unit
        counters[counter] = by_row(rows)
    lines = []
    for i, (fmt, K, N, M, tile) in enumerate(FEWTOKEN_PROFILE):
        alg = algorithmic_bytes(fmt, K, N, M)
        parts, tot_b, tot_t = [], 0.0, 0.0
        for name, rs in trace[i].items():
            if len(rs) < 10:  # not one of the call's kernels (the graph holds 10 calls)
                continue
            us = float(np.mean([(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rs]))
            fb = float(np.median([float(r["Counter_Value"]) for r in counters["FETCH_SIZE"][i].get(name, [])] or [0])) * scale["FETCH_SIZE"]
            wb = float(np.median([float(r["Counter_Value"]) for r in counters["WRITE_SIZE"][i].get(name, [])] or [0])) * scale["WRITE_SIZE"]
            parts.append(f"{name}: {len(rs)} dispatches, {us:.2f} us mean, FETCH {fb/1e6:.2f} MB + WRITE {wb/1e6:.2f} MB")
            tot_b += fb + wb
            tot_t += us
        lines.append(f"{fmt} K={K} N={N} M={M} tile={tile}: " + "; ".join(parts) +
                     f"; per call {tot_t:.2f} us of kernel time, {tot_b/1e6:.1f} MB = {tot_b/alg:.3f} x algorithmic "
                     f"{alg/1e6:.1f} MB -> {alg/tot_t/1e3:.0f} GB/s ({alg/tot_t/1e3/HBM_PEAK_GBS*100:.1f} % of 8 TB/s)")
    for f in ("wq_gemm.hip", "wq_gemv.hip"):
        src = open(os.path.join(ROOT, "gemm_decode_amd", "csrc", f), "rb").read()
        lines.append(f"kernel source: gemm_decode_amd/csrc/{f} sha256 {hashlib.sha256(src).hexdigest()}")
    with open(out_txt, "a") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# (K, N) -> (split_k, waves, rows): the launches the tuner picks for the W4 decode shapes
PROFILE_W4 = {(5120, 27648): (1, 4, 16 | 0x200), (13824, 5120): (1, 4, 4)}


def profile_w4(calls: int = 10):
    """Kernels for a rocprofv3 run of the W4 group-128 decode GEMV at M = 1: for each
    (K, N) of PROFILE_W4 that launch (set in the tuning cache, so no tuner dispatches
    enter the profile), `calls` wq_linear calls on rotating weight copies as one HIP
    graph replayed once."""
    import torch
    import gemm_decode_amd.wq as wq
    for (K, N), (sk, wv, rw) in PROFILE_W4.items():
        p = Pool(wq, torch, 3, "w4g128", K, N, 1)
        wq.wq_tune_cache_set("w4g128", K, N, 1, wq.KIND_GEMV, sk | (wv << 8) | (rw << 16))
        v = wq.wq_tune_cache_get("w4g128", K, N, 1, wq.KIND_GEMV)
        streaming_settle(torch, 3.0)
        ms = time_graph(torch, lambda: p.call(wq), calls, reps=1, settle_s=0.0)
        log(f"profile w4 K={K} N={N} M=1 (split, waves, rows) = ({v & 0xFF}, {(v >> 8) & 0xFF}, "
            f"{v >> 16:#x}): {ms * 1e3 / calls:.2f} us per call (HIP events)")
        p.free()
        del p
        torch.cuda.empty_cache()


def summarize_valu(pmc_dir: str, out_txt: str):
    """Turn one rocprofv3 --pmc pass (SQ_WAVES SQ_INSTS_VALU SQ_INSTS_VMEM_RD
    SQ_WAVE_CYCLES SQ_WAIT_INST_ANY) of --profile-w4 into per-wave instruction counts and
    the VALU issue time per SIMD (4 cycles per wave64 instruction, 1024 SIMDs)."""
    import glob
    from collections import defaultdict
    rows = []
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        rows += _read_csv_rows(f)
    d = defaultdict(dict)
    for r in rows:
        if "gemv" in r["Kernel_Name"]:
            name = r["Kernel_Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
            key = (name, int(r["Grid_Size"]), int(r["Dispatch_Id"]))
            d[key][r["Counter_Name"]] = float(r["Counter_Value"])
    groups = defaultdict(list)
    for (name, grid, _), c in d.items():
        groups[(name, grid)].append(c)
    lines = []
    for (name, grid), cs in groups.items():
        avg = {k: float(np.mean([c[k] for c in cs])) for k in cs[0]}
        w = avg["SQ_WAVES"]
        valu_us = avg["SQ_INSTS_VALU"] * 4 / 1024 / 2.4e3
        lines.append(f"{name} grid={grid}: {len(cs)} dispatches, {w:.0f} waves; per wave {avg['SQ_INSTS_VALU'] / w:.0f} "
                     f"VALU, {avg['SQ_INSTS_VMEM_RD'] / w:.1f} vector-memory reads, waiting to issue "
                     f"{100 * avg['SQ_WAIT_INST_ANY'] / avg['SQ_WAVE_CYCLES']:.0f} % of wave cycles; VALU issue "
                     f"per SIMD {valu_us:.2f} us at 2.4 GHz")
    with open(out_txt, "a") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def profile_topk(calls: int = 10):
    """Kernels for a rocprofv3 run of the LM head + top-k call: W8 and W4 group-128 LM
    heads (5120, 151936) at M = 1, k = 50, tuned, `calls` calls on rotating weight
    copies as one HIP graph replayed once."""
    import torch
    import gemm_decode_amd.wq as wq
    for fmt in ("w8g128", "w4g128"):
        rec = measure_lm_head_topk(wq, torch, 4, fmt, 5120, 151936, 1)
        log(f"profile lm head + top-k {fmt}: {rec}")


def _read_csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_counters(fetch_dir: str, write_dir: str, trace_dir: str | None, out_txt: str):
    """Turn rocprofv3 runs of the profile pass (two --pmc runs: FETCH_SIZE, WRITE_SIZE
    in KiB per dispatch; optionally a --kernel-trace run) into HBM bytes and kernel
    time per GEMV launch.  Counters are scaled by what they read for the elementwise
    reference of COPY_BYTES in / COPY_BYTES out."""
    import glob

    def dispatches(d, pattern):
        rows = []
        for f in glob.glob(os.path.join(d, "**", pattern), recursive=True):
            rows += _read_csv_rows(f)
        return sorted(rows, key=lambda r: int(r.get("Dispatch_Id", 0)))

    def split(rows, value):
        # the graph issues the shapes round-robin: launch j is shape j % 4
        ref = [value(r) for r in rows if "bitwise_not" in r["Kernel_Name"]]
        gemv = [value(r) for r in rows if "gemv_kernel" in r["Kernel_Name"]]
        n = len(DECODE_SHAPES)
        return ref, [gemv[i::n] for i in range(n)]

    cval = lambda r: float(r["Counter_Value"])
    f_ref, f_sh = split([r for r in dispatches(fetch_dir, "*counter_collection.csv") if r["Counter_Name"] == "FETCH_SIZE"], cval)
    w_ref, w_sh = split([r for r in dispatches(write_dir, "*counter_collection.csv") if r["Counter_Name"] == "WRITE_SIZE"], cval)
    if not f_ref or not w_ref:
        raise SystemExit("reference kernel counters missing")
    f_scale = COPY_BYTES / 1024.0 / float(np.median(f_ref))
    w_scale = COPY_BYTES / 1024.0 / float(np.median(w_ref))
    t_sh = None
    if trace_dir:
        dur = lambda r: (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        _, t_sh = split(dispatches(trace_dir, "*kernel_trace.csv"), dur)
    lines = [f"reference: elementwise kernel over {COPY_BYTES} B in + {COPY_BYTES} B out; "
             f"FETCH_SIZE reads {np.median(f_ref):.0f} KiB (scale {f_scale:.4f}), "
             f"WRITE_SIZE reads {np.median(w_ref):.0f} KiB (scale {w_scale:.4f})"]
    shapes = {}
    for i, (K, N) in enumerate(DECODE_SHAPES):
        fb = float(np.median(f_sh[i])) * 1024 * f_scale
        wb = float(np.median(w_sh[i])) * 1024 * w_scale
        alg = algorithmic_bytes("w8pc", K, N, 1)
        rec = {"fetch_bytes": fb, "write_bytes": wb, "algorithmic_bytes": alg,
               "traffic_over_algorithmic": (fb + wb) / alg}
        line = (f"{K}x{N} M=1 config (split,waves,rows)={PROFILE_CONFIG[(K, N)]}: FETCH {fb/1e6:.2f} MB + "
                f"WRITE {wb/1e6:.3f} MB = {(fb + wb)/alg:.4f} x algorithmic {alg/1e6:.2f} MB")
        if t_sh:
            us = float(np.mean(t_sh[i]))
            rec["kernel_us_mean"] = us
            line += f"; kernel {us:.2f} us mean of {len(t_sh[i])} -> {alg/us/1e3:.0f} GB/s ({alg/us/1e3/HBM_PEAK_GBS*100:.1f}% of 8 TB/s)"
        shapes[f"{K}x{N}"] = rec
        lines.append(line)
    avg = float(np.mean([v["fetch_bytes"] + v["write_bytes"] for v in shapes.values()]))
    if t_sh:
        tot_b = sum(v["algorithmic_bytes"] for v in shapes.values())
        tot_t = sum(v["kernel_us_mean"] for v in shapes.values())
        lines.append(f"4-shape step, kernel time only: {tot_t:.2f} us -> {tot_b/tot_t/1e3:.0f} GB/s "
                     f"({tot_b/tot_t/1e3/HBM_PEAK_GBS*100:.1f}% of 8 TB/s)")
    src = open(os.path.join(ROOT, "gemm_decode_amd", "csrc", "wq_gemv.hip"), "rb").read()
    rec = {"kernel_src_sha256": hashlib.sha256(src).hexdigest(), "per_shape": shapes,
           "bytes_per_step_avg_launch": avg, "copy_scale": {"fetch": f_scale, "write": w_scale}}
    json.dump(rec, open(TRAFFIC_FILE, "w"), indent=1)
    with open(out_txt, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_prefill_traffic(fetch_dir: str, write_dir: str, out_txt: str):
    """Turn two rocprofv3 --pmc runs of --profile-prefill (FETCH_SIZE, then WRITE_SIZE,
    KiB per dispatch) into HBM bytes per GEMM call against the algorithmic bytes
    (weights + metadata + x + y once): the GEMM kernel, and with it the kernels the
    call adds (the tail reduction, and x to fp16 for group-128).  Scaled by what the
    counters read for the elementwise reference."""
    import glob

    def rows_of(d, counter):
        out = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            out += [r for r in _read_csv_rows(f) if r["Counter_Name"] == counter]
        return sorted(out, key=lambda r: int(r.get("Dispatch_Id", 0)))

    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = rows_of(d, counter)
        ref = [float(r["Counter_Value"]) for r in rows if "bitwise_not" in r["Kernel_Name"]]
        if not ref:
            raise SystemExit("reference kernel counters missing")
        scale = COPY_BYTES / 1024.0 / float(np.median(ref)) * 1024.0  # bytes per counter unit
        for r in rows:
            name = r["Kernel_Name"]
            if not any(k in name for k in ("gemm_dma", "tail_reduce", "x_to_f16")):
                continue
            # the per-channel kernels: the w8pc GEMM and tail_reduce<true>
            pc = "w8pc_kernel" in name or "tail_reduce_kernel<true" in name
            kern = next(k for k in ("gemm_dma_w8pc_kernel", "gemm_dma_g128_kernel", "gemm_tail_reduce_kernel",
                                    "x_to_f16_rows_kernel") if k in name)
            res.setdefault(("w8pc" if pc else "w4g128", kern, counter), []).append(float(r["Counter_Value"]) * scale)
    lines = []
    for fmt, K, N, M, tile in PREFILL_PROFILE:
        alg = algorithmic_bytes(fmt, K, N, M)
        main = "gemm_dma_w8pc_kernel" if fmt == "w8pc" else "gemm_dma_g128_kernel"
        per_call = {}
        for kern in (main, "gemm_tail_reduce_kernel", "x_to_f16_rows_kernel"):
            f = res.get((fmt, kern, "FETCH_SIZE"))
            w = res.get((fmt, kern, "WRITE_SIZE"))
            if f and w:
                per_call[kern] = (float(np.median(f)), float(np.median(w)))
        tot = sum(f + w for f, w in per_call.values())
        parts = "; ".join(f"{k}: FETCH {f/1e6:.1f} MB + WRITE {w/1e6:.1f} MB" for k, (f, w) in per_call.items())
        lines.append(f"{fmt} K={K} N={N} M={M} tile={tile}: {parts}; call total {tot/1e6:.1f} MB = "
                     f"{tot/alg:.3f} x algorithmic {alg/1e6:.1f} MB")
    src = open(os.path.join(ROOT, "gemm_decode_amd", "csrc", "wq_gemm.hip"), "rb").read()
    lines.append(f"kernel source: gemm_decode_amd/csrc/wq_gemm.hip sha256 {hashlib.sha256(src).hexdigest()}")
    with open(out_txt, "a") as fo:
        fo.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_mfma(pmc_dir: str, out_txt: str):
    """Turn a rocprofv3 --pmc run of --profile-prefill (SQ_INSTS_MFMA,
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE) into per-kernel matrix-core figures: busy
    cycles per SIMD (the counter sums the 1024 SIMDs) and their ratio to GRBM_GUI_ACTIVE
    / 8 (the GPU's busy cycles, summed over the 8 XCDs; a shader-clock fraction only if
    that counter runs on the shader clock).  SQ_INSTS_MFMA x 32768 flops
    (v_mfma_f32_32x32x16) must equal the algorithmic 2 M K N."""
    import glob
    rows = []
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        rows += _read_csv_rows(f)
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "gemm_dma" not in name:
            continue
        kern = "gemm_dma_w8pc_kernel" if "w8pc" in name else "gemm_dma_g128_kernel"
        d = per.setdefault(kern, {}).setdefault(int(r.get("Dispatch_Id", 0)), {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    lines = []
    for (fmt, K, N, M, tile), kern in zip(PREFILL_PROFILE, ("gemm_dma_w8pc_kernel", "gemm_dma_g128_kernel")):
        ds = list(per.get(kern, {}).values())
        if not ds:
            continue
        mfma = float(np.mean([d["SQ_INSTS_MFMA"] for d in ds]))
        busy = float(np.mean([d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds])) / 1024.0
        gpu = float(np.mean([d["GRBM_GUI_ACTIVE"] for d in ds])) / 8.0
        lines.append(f"{kern} ({fmt} K={K} N={N} M={M} tile={tile}), {len(ds)} dispatches: "
                     f"{mfma:.0f} MFMA instructions = {mfma * 32768 / (2.0 * M * K * N):.4f} x 2MKN/32768; "
                     f"matrix cores busy {busy:.0f} cycles per SIMD (= {busy / 2.4e3:.1f} us at 2.4 GHz); "
                     f"GRBM_GUI_ACTIVE / 8 = {gpu:.0f} cycles, ratio {100 * busy / gpu:.1f} %")
    with open(out_txt, "a") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--replays", type=int, default=7, help="timed graph replays of the headline (median)")
    ap.add_argument("--settle", type=float, default=8.0,
                    help="seconds of untimed headline replays before timing (steady-state clocks)")
    ap.add_argument("--quick", action="store_true", help="headline only (no per-workload detail)")
    ap.add_argument("--detail", default="", help="comma list of detail groups to run (default: all)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tune-iters", type=int, default=1000)
    ap.add_argument("--profile-pass", action="store_true",
                    help="launch the copy reference and the headline GEMVs for a rocprofv3 counter run")
    ap.add_argument("--profile-topk", action="store_true",
                    help="run the LM head + top-k profile workload (for rocprofv3) and exit")
    ap.add_argument("--profile-prefill", action="store_true",
                    help="run the prefill GEMM profile workload (for rocprofv3) and exit")
    ap.add_argument("--summarize-prefill-traffic", nargs=3, metavar=("FETCH_DIR", "WRITE_DIR", "OUT_TXT"),
                    help="turn two rocprofv3 --pmc runs of --profile-prefill into HBM bytes per GEMM call")
    ap.add_argument("--profile-w4", action="store_true", help="kernels for rocprofv3: the W4 decode GEMV")
    ap.add_argument("--profile-fewtoken", action="store_true", help="kernels for rocprofv3: the few-token GEMM rows")
    ap.add_argument("--summarize-fewtoken", nargs=4, metavar=("TRACE_DIR", "FETCH_DIR", "WRITE_DIR", "OUT_TXT"),
                    help="per-row kernel time and HBM bytes of a --profile-fewtoken run")
    ap.add_argument("--summarize-valu", nargs=2, metavar=("PMC_DIR", "OUT_TXT"),
                    help="turn a rocprofv3 SQ counter pass of --profile-w4 into VALU figures")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "TRACE_DIR", "OUT_TXT"),
                    help="turn rocprofv3 runs of --profile-pass into the traffic record and a summary")
    ap.add_argument("--summarize-mfma", nargs=2, metavar=("PMC_DIR", "OUT_TXT"),
                    help="turn a rocprofv3 --pmc run of --profile-prefill into matrix-core busy fractions")
    args = ap.parse_args()
    if args.summarize_mfma:
        summarize_mfma(*args.summarize_mfma)
        return
    if args.profile_w4:
        profile_w4()
        return
    if args.profile_fewtoken:
        profile_fewtoken()
        return
    if args.summarize_valu:
        summarize_valu(*args.summarize_valu)
        return
    if args.summarize_prefill_traffic:
        summarize_prefill_traffic(*args.summarize_prefill_traffic)
        return
    if args.summarize_fewtoken:
        summarize_fewtoken(*args.summarize_fewtoken)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch
    import gemm_decode_amd.wq as wq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.profile_pass:
        profile_pass()
        return
    if args.profile_prefill:
        profile_prefill()
        return
    if args.profile_topk:
        profile_topk()
        return
    device_warmup(torch)
    log("warm-up done")

    # ---------------- headline: W8A16 per-channel decode projections at M = 1
    pools = [Pool(wq, torch, 2, "w8pc", K, N, 1) for K, N in DECODE_SHAPES]
    tuned = {}
    for p in pools:
        tuned[(p.K, p.N)] = tune(wq, p, args.tune_iters, args.tune_iters)
        log(f"tuned w8pc K={p.K} N={p.N} M=1: split_k={tuned[(p.K, p.N)][0]} lat_us={tuned[(p.K, p.N)][1]}")
    parity = {f"{p.K}x{p.N}": p.check(wq, torch) for p in pools}
    for k, st in parity.items():
        if st["fails"] or not st["copies_bit_identical"]:
            raise SystemExit(f"parity failure on {k}: {st}")

    def step():
        for p in pools:
            p.call(wq)

    bytes_step = sum(p.bytes_per_call() for p in pools)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    head_stats = {}
    ms = time_graph(torch, step, args.steps, reps=args.replays, stats=head_stats, settle_s=args.settle)
    ms_per_step = ms / args.steps
    value = bytes_step / (ms_per_step / 1e3) / 1e9
    log(f"headline: {ms_per_step * 1e3:.2f} us/step (median of {args.replays} replays of {args.steps} steps; "
        f"min {head_stats['min_ms'] / args.steps * 1e3:.2f}, max {head_stats['max_ms'] / args.steps * 1e3:.2f}), "
        f"{value:.1f} GB/s")

    detail = {"decode_w8pc_m1": {}}
    for p in pools:
        per = time_graph(torch, lambda p=p: p.call(wq), 2 * len(p.copies)) / (2 * len(p.copies))
        gbs = p.bytes_per_call() / (per / 1e3) / 1e9
        detail["decode_w8pc_m1"][f"{p.K}x{p.N}"] = {
            "us": round(per * 1e3, 3), "GB/s": round(gbs, 1), "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1),
            "split_k": tuned[(p.K, p.N)][0], "copies": len(p.copies), "parity": parity[f"{p.K}x{p.N}"],
            "tuned_value": wq.wq_tune_cache_get("w8pc", p.K, p.N, 1, wq.KIND_GEMV)}
    for p in pools:
        p.free()
    del pools
    torch.cuda.empty_cache()

    detail["streaming_ceiling"] = streaming_ceiling(torch)
    detail["streaming_ceiling"]["headline_pct_of_read"] = round(
        100 * value / detail["streaming_ceiling"]["read_GB/s"], 1)
    if not args.quick:
        detail.update(run_detail(wq, torch, args))

    src = open(os.path.join(ROOT, "gemm_decode_amd", "csrc", "wq_gemv.hip"), "rb").read()
    src_sha = hashlib.sha256(src).hexdigest()
    launches = 4 * args.steps
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "W8A16 per-channel decode GEMV step at M=1: (K,N) = (5120,27648) (13824,5120) "
                               "(5120,7168) (6144,5120), int8 codes + bf16 scales, x bf16 N(0,1), W N(0,0.02^2), "
                               "rotating weight copies, one HIP graph",
                   "M": 1, "launches_per_step": 4},
        "roofline": {"bound": "hbm", "achieved": round(value, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(value / HBM_PEAK_GBS, 4), "traffic": traffic_entry(src_sha),
                     "traffic_unit": "HBM bytes per launch (mean over the 4 shapes)",
                     "kernel": "gemv_kernel (W8 per-channel, M=1)",
                     "algorithmic_bytes_per_launch": round(bytes_step / 4),
                     "avg_launch_us": round(ms_per_step * 1e3 / 4, 3),
                     "timing": f"HIP events on the launching stream, median of {args.replays} graph replays "
                               f"of {launches} launches, after {args.settle:g} s of untimed replays"},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline(),
        "targets": compact_targets(detail, value, ms_per_step),
    }
    write_detail(detail, line)
    out = json.dumps(line, separators=(",", ":"))
    if len(out) > 4000:  # the result line stays short enough for a log tail to hold it whole
        line.pop("targets", None)
        out = json.dumps(line, separators=(",", ":"))
    print(out, flush=True)


DETAIL_FILE = os.path.join(ROOT, "gpurun_out", "bench_detail.json")


def write_detail(detail: dict, line: dict):
    """The per-workload detail (tuner latencies, parity statistics, every row) goes
    to a file and, one row per line, to stderr; stdout keeps the one result line."""
    try:
        os.makedirs(os.path.dirname(DETAIL_FILE), exist_ok=True)
        with open(DETAIL_FILE, "w") as f:
            json.dump({"result": line, "detail": detail}, f, indent=1)
        log(f"detail written to {DETAIL_FILE}")
    except OSError as e:  # pragma: no cover
        log(f"detail not written: {e}")
    for group, rows in detail.items():
        log(f"detail {group}: {json.dumps(rows, separators=(',', ':'))}")


def compact_targets(detail: dict, value: float, ms_per_step: float) -> dict:
    """The rows the goals are stated on: microseconds and % of the roofline for every
    M = 1 GEMV row (decode shapes, W4 decode, split-K stress shapes) and every M = 2048
    GEMM row, plus the parity outcome of all checked rows."""
    gemv, gemm, worst, fails = {}, {}, 0.0, 0
    for k, r in detail.get("decode_w8pc_m1", {}).items():
        gemv[f"w8pc_{k}"] = [r["us"], r["pct_hbm"]]
    for k, r in detail.get("decode_w4g128", {}).items():
        if k.endswith("_M1"):
            gemv[f"w4g128_{k[:-3]}"] = [r["us"], r["pct_hbm"]]
    for k, r in detail.get("splitk_stress", {}).items():
        gemv[k] = [r["us"], r["pct_hbm"]]
    for k, r in detail.get("prefill_gemm", {}).items():
        if k.endswith("_M2048"):
            gemm[k[:-6]] = [r["us"], r["pct_mfma"]]
    for group in detail.values():
        if not isinstance(group, dict):
            continue
        for r in group.values():
            st = r.get("parity") if isinstance(r, dict) else None
            if st:
                worst = max(worst, st["max_ratio"])
                fails += st["fails"]
    return {"goal": "GEMV M=1 >= 70 % of 8 TB/s; GEMM M=2048 >= 50 % of 2.5 PFLOP/s",
            "gemv_m1_us_pct_hbm": gemv, "gemm_m2048_us_pct_mfma": gemm,
            "parity_rows_worst_err_over_tol": round(worst, 4), "parity_fails": fails,
            "headline_us_per_step": round(ms_per_step * 1e3, 3)}


def streaming_ceiling(torch, nbytes: int = 2 << 30, reps: int = 10) -> dict:
    """Context for the GEMV's % of HBM: what plain vendor kernels stream on this device
    in the same run -- a bf16 matrix-vector product over a 2 GiB matrix (read only,
    torch.mv -> the vendor BLAS) and a 1 GiB elementwise copy (read + write), back to
    back, HIP events around `reps` calls."""
    K = 8192
    a = torch.ones((nbytes // 2 // K, K), dtype=torch.bfloat16, device="cuda")
    v = torch.ones(K, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(a.shape[0], dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        torch.mv(a, v, out=out)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mv(a, v, out=out)
    e1.record()
    e1.synchronize()
    read = nbytes * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del a, v, out
    b = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    c = torch.empty_like(b)
    for _ in range(2):
        torch.bitwise_not(b, out=c)
    e0.record()
    for _ in range(reps):
        torch.bitwise_not(b, out=c)
    e1.record()
    e1.synchronize()
    copy = 2 * (nbytes // 2) * reps / (e0.elapsed_time(e1) / 1e3) / 1e9
    del b, c
    torch.cuda.empty_cache()
    log(f"streaming ceiling: read {read:.0f} GB/s (bf16 mv over 2 GiB), copy {copy:.0f} GB/s (1 GiB in + out)")
    return {"read_GB/s": round(read, 1), "copy_GB/s": round(copy, 1),
            "how": "torch.mv of a 2 GiB bf16 matrix [262144, 8192] (vendor BLAS); torch.bitwise_not "
                   "1 GiB -> 1 GiB; HIP events over 10 back-to-back calls"}


def run_detail(wq, torch, args) -> dict:
    """Secondary workloads, each timed as graph replays over its rotation pool."""
    out = {}

    def measure(cfg, fmt, K, N, M, tune_it=True, check=True, act="bf16"):
        p = Pool(wq, torch, cfg, fmt, K, N, M, act=act)
        rec = {}
        if tune_it:
            rec["tuned"], rec["tune_lat_us"] = tune(wq, p, 200, 200)
        if check:
            rec["parity"] = p.check(wq, torch)
        n = 2 * len(p.copies)
        st = {}
        per = time_graph(torch, lambda: p.call(wq), n, stats=st) / n
        rec["us_min_max"] = [round(st["min_ms"] / n * 1e3, 3), round(st["max_ms"] / n * 1e3, 3)]
        gbs = p.bytes_per_call() / (per / 1e3) / 1e9
        tf = 2.0 * M * K * N / (per / 1e3) / 1e12
        rec.update({"us": round(per * 1e3, 3), "GB/s": round(gbs, 1),
                    "pct_hbm": round(100 * gbs / HBM_PEAK_GBS, 1), "TFLOP/s": round(tf, 2),
                    "pct_mfma": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 1)})
        log(f"cfg{cfg} {fmt}{' f16 x' if act == 'f16' else ''} K={K} N={N} M={M}: {rec['us']} us {rec['GB/s']} GB/s "
            f"{rec['TFLOP/s']} TF/s")
        p.free()
        del p
        torch.cuda.empty_cache()
        return rec

    groups = {
        "decode_w8pc_msweep": lambda: {f"{K}x{N}_M{M}": measure(2, "w8pc", K, N, M)
                                       for K, N in DECODE_SHAPES for M in (2, 4, 7)},
        "decode_w4g128": lambda: {f"{K}x{N}_M{M}": measure(3, "w4g128", K, N, M)
                                  for K, N in [(5120, 27648), (13824, 5120)] for M in (1, 4)},
        # INT4 per output channel: the group-128 kernels on its repeated metadata
        "w4_per_channel": lambda: {f"w4pc_{K}x{N}_M{M}": measure(3, "w4pc", K, N, M)
                                   for K, N in [(5120, 27648)] for M in (1, 2048)},
        # groups of 32 and 64: the dot2 GEMV and the LDS-DMA GEMM folding by the group size
        "small_groups": lambda: {f"{fmt}_{K}x{N}_M{M}": measure(3 if fmt.startswith("w4") else 2, fmt, K, N, M)
                                 for fmt in ("w8g32", "w8g64", "w4g32", "w4g64")
                                 for K, N in [(5120, 27648)] for M in (1, 2048)},
        # fp16 activations (tuned on bf16 x: the tuner times bf16 calls; the fp16 call takes its launch)
        "f16_activations": lambda: {f"{fmt}_{K}x{N}_M{M}": measure(2 if fmt == "w8pc" else 3, fmt, K, N, M,
                                                                   act="f16")
                                    for fmt in ("w8pc", "w4g128") for K, N in [(5120, 27648)] for M in (1, 2048)},
        "splitk_stress": lambda: {f"{fmt}_{K}x{N}": measure(4, fmt, K, N, 1)
                                  for K, N in [(27648, 5120), (5120, 151936)]
                                  for fmt in ("w8pc", "w8g128", "w4g128")},
        "prefill_gemm": lambda: {f"{fmt}_{K}x{N}_M{M}": measure(5, fmt, K, N, M, tune_it=M >= 8)
                                 for fmt in ("w8pc", "w4g128") for K, N in [(5120, 27648), (13824, 5120)]
                                 for M in (8, 64, 512, 2048)},
        # between the matrix-core GEMV tiles (<= 16 tokens) and the MFMA-bound sizes
        "mid_m_gemm": lambda: {f"{fmt}_{K}x{N}_M{M}": measure(5, fmt, K, N, M)
                               for fmt in ("w8pc", "w4g128") for K, N in [(5120, 27648), (13824, 5120)]
                               for M in (32, 128, 256)},
        "lm_head_topk": lambda: {f"{fmt}_{K}x{N}_M{M}": measure_lm_head_topk(wq, torch, 4, fmt, K, N, M)
                                 for fmt in ("w8g128", "w4g128") for K, N in [(5120, 151936)] for M in (1, 4)},
        "activation_permutation": lambda: {f"{fmt}_{K}x{N}_M{M}": measure_linear_perm(wq, torch, cfg, fmt, K, N, M)
                                           for cfg, fmt, M in ((3, "w4g128", 1), (1, "w8pc", 1), (5, "w8pc", 2048))
                                           for K, N in [(5120, 27648)]},
        "reference_bf16_gemm": lambda: reference_bf16_gemm(torch),
        "moe": lambda: {f"{fmt}_E{E}_{K}x{N}_T{T}{'_silu' if gated else ''}": measure_moe(wq, torch, fmt, E, K, N, T, gated)
                        for fmt, E, K, N, T, gated in MOE_ROWS},
    }
    want = list(groups) if not args.detail else args.detail.split(",")
    for name in want:
        if name not in groups:
            raise SystemExit(f"unknown detail group {name!r}; choose from {', '.join(groups)}")
        out[name] = groups[name]()
    return out


# MoE rows: 8 experts of a fused gate/up projection (K = 2048, N = 2 x 5632, SiLU-gated) and
# of a down projection (K = 5632, N = 2048), one token routed to two experts (T = 2 rows)
# and 16 tokens to two experts each (T = 32 rows, seeded counts)
MOE_ROWS = [("w4g128", 8, 2048, 11264, 2, True), ("w4g128", 8, 2048, 11264, 32, True),
            ("w8pc", 8, 5632, 2048, 2, False), ("w4g128", 8, 5632, 2048, 2, False),
            ("w4g128", 8, 2048, 11264, 2048, True), ("w8pc", 8, 5632, 2048, 2048, False)]


def measure_moe(wq, torch, fmt, E, K, N, T, gated) -> dict:
    """The grouped layer over E stacked experts (graph replay over rotating copies of the
    stacked weight), checked against the oracle on every output; GB/s counts the packed
    bytes of the experts that hold rows, x and y once."""
    import oracle
    import synth
    Ws = [synth.weight(60 + e, K, N, synth.uses_outliers(fmt)) for e in range(E)]
    base = wq.quantize_experts([torch.from_numpy(W).to("cuda") for W in Ws], fmt)
    per = sum(wq.wq_packed_sizes(fmt, wq.GFX950, K, N))
    copies = [base] + [base.clone() for _ in range(max(1, int(np.ceil(ROTATE_BYTES / (per * E)))) - 1)]
    off = synth.moe_offsets(61, T, E) if T > 2 else np.array([0] + [1] * 3 + [2] * (E - 3), dtype=np.int32)
    xb = synth.activation(62, K, T)
    x = torch.from_numpy(xb.view(np.int16)).to("cuda").view(torch.bfloat16)
    od = torch.from_numpy(off.astype(np.int32)).to("cuda")
    width = N // 2 if gated else N
    y = torch.empty((T, width), dtype=torch.bfloat16, device="cuda")
    epi = wq.EPILOGUE_SILU_MUL if gated else wq.EPILOGUE_NONE
    i = [0]

    def fn():
        wq.wq_moe_linear(copies[i[0]], x, od, y, epi)
        i[0] = (i[0] + 1) % len(copies)

    fn()
    torch.cuda.synchronize()
    Ps = [oracle.pack(fmt, W) for W in Ws]
    ref = oracle.ref_moe_silu_mul(xb, off, Ps) if gated else oracle.ref_moe_linear(xb, off, Ps)
    st = oracle.compare(y.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    if st["fails"]:
        raise SystemExit(f"moe parity failure {fmt} E={E} K={K} N={N} T={T}: {st}")
    n = 2 * len(copies)
    us = time_graph(torch, fn, n) / n * 1e3
    active = int(np.count_nonzero(np.diff(off)))
    alg = active * per + 2 * T * K + 2 * T * width
    rec = {"us": round(us, 3), "GB/s": round(alg / us / 1e3, 1), "pct_hbm": round(100 * alg / us / 1e3 / HBM_PEAK_GBS, 1),
           "TFLOP/s": round(2.0 * T * K * N / us / 1e6, 1), "experts_with_rows": active, "parity": st}
    log(f"moe {fmt} E={E} K={K} N={N} T={T} gated={gated}: {rec['us']} us, {rec['GB/s']} GB/s over "
        f"{active} experts with rows, {rec['TFLOP/s']} TFLOP/s")
    del copies, base
    torch.cuda.empty_cache()
    return rec


def measure_lm_head_topk(wq, torch, cfg, fmt, K, N, M, k: int = 50, temperature: float = 0.8) -> dict:
    """The LM head + top-k sampling call against the LM head alone (both tuned, graph
    replay over rotating weight copies): the cost the selection and the draw add."""
    p = Pool(wq, torch, cfg, fmt, K, N, M)
    tune(wq, p, 200, 200)
    n = 2 * len(p.copies)
    lin = time_graph(torch, lambda: p.call(wq), n) / n
    ws = wq.workspace(wq.wq_lm_head_topk_workspace_size(p.copies[0], M, k))
    u = torch.full((M,), 0.5, dtype=torch.float32, device="cuda")
    vals = torch.empty((M, k), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
    tok = torch.empty(M, dtype=torch.int32, device="cuda")

    def fn():
        w = p.copies[p.i]
        p.i = (p.i + 1) % len(p.copies)
        wq.wq_lm_head_topk(w, p.x, k, temperature, u, vals, idx, tok, ws)

    both = time_graph(torch, fn, n) / n
    rec = {"k": k, "temperature": temperature, "us_linear": round(lin * 1e3, 3),
           "us_linear_topk": round(both * 1e3, 3), "us_added": round((both - lin) * 1e3, 3),
           "GB/s_linear_topk": round(p.bytes_per_call() / (both / 1e3) / 1e9, 1)}
    log(f"lm head + top-k cfg{cfg} {fmt} K={K} N={N} M={M} k={k}: {rec['us_linear_topk']} us "
        f"(layer alone {rec['us_linear']} us, +{rec['us_added']} us)")
    p.free()
    del p
    torch.cuda.empty_cache()
    return rec


def measure_linear_perm(wq, torch, cfg, fmt, K, N, M) -> dict:
    """The layer with the full-K activation permutation (gather + layer) against the
    layer alone (both tuned, graph replay over rotating weight copies): the cost the
    gather adds."""
    p = Pool(wq, torch, cfg, fmt, K, N, M)
    tune(wq, p, 200, 200)
    n = 2 * len(p.copies)
    lin = time_graph(torch, lambda: p.call(wq), n) / n
    ws = wq.workspace(wq.wq_linear_perm_workspace_size(p.copies[0], M))
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(cfg)).to(torch.int32).to("cuda")

    def fn():
        w = p.copies[p.i]
        p.i = (p.i + 1) % len(p.copies)
        wq.wq_linear_perm(w, p.x, perm, p.y, ws)

    both = time_graph(torch, fn, n) / n
    rec = {"us_linear": round(lin * 1e3, 3), "us_linear_perm": round(both * 1e3, 3),
           "us_added": round((both - lin) * 1e3, 3)}
    log(f"activation permutation cfg{cfg} {fmt} K={K} N={N} M={M}: {rec['us_linear_perm']} us "
        f"(layer alone {rec['us_linear']} us, +{rec['us_added']} us)")
    p.free()
    del p
    torch.cuda.empty_cache()
    return rec


def reference_bf16_gemm(torch, M: int = 2048, K: int = 5120, N: int = 27648) -> dict:
    """Context, not this library: the vendor BLAS (torch.mm -> hipBLASLt) on a plain
    bf16 x bf16 product of the prefill shape, timed like the detail lines (graph replay
    over 4 distinct B matrices), as the matrix-core rate a library GEMM reaches on this
    device at this shape."""
    a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16)
    bs = [torch.randn(K, N, device="cuda", dtype=torch.bfloat16) for _ in range(4)]
    i = [0]

    def fn():
        torch.mm(a, bs[i[0]])
        i[0] = (i[0] + 1) % len(bs)

    per = time_graph(torch, fn, 8) / 8
    tf = 2.0 * M * K * N / (per / 1e3) / 1e12
    log(f"reference torch.mm bf16 M={M} K={K} N={N}: {per * 1e3:.1f} us {tf:.1f} TF/s")
    del a, bs
    torch.cuda.empty_cache()
    return {"what": "torch.mm bf16 (hipBLASLt), not this library", "M": M, "K": K, "N": N,
            "us": round(per * 1e3, 3), "TFLOP/s": round(tf, 2),
            "pct_mfma": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 1)}


if __name__ == "__main__":
    main()
