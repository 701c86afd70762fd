"""Benchmark of the smoothed, quantised attention path on one MI355X.

One step = sage_quant_qk + sage_quant_v + sage_attn_fwd over one batch of
seeded synthetic bf16 inputs already resident in HBM (default workload: the
FLUX.3 Action joint block, B2 H24 N4608 D128).  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 30] [--warmup 5] [--workload flux_joint]

`value` is attention TFLOPS over the whole step, 4*B*H*N^2*D / step time (the
quantisation kernels are inside the step).  A default run also measures the
metric's other two parts in the same process and reports them under `parts`:
attention on the long text-to-video shape (B1 H40 N32760 D128) and the
quantisers' HBM GB/s on the quant-only shape of the same size; and, for
reference, the video-early block (B2 H24 N3128 D128).  Each workload
first runs back-to-back steps for --prewarm-ms (the GPU clock ramps up over
the first tens of ms of load), then --warmup counted steps.  Per-kernel times
come from HIP events recorded on the stream the kernels run on.

    python bench.py --workload flux_joint --abba "producer=fused,producer=composed"

compares two step variants in one process, in ABBA groups.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized-attention TFLOPS at N=4608 & 32760 (1 GPU); quant-kernel HBM GB/s"
PEAK_MFMA_TFLOPS = 5000.0   # MI355X dense INT8 / FP8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def algorithmic(B, N, H, D, q_block=32, k_block=64):
    """Algorithmic work of each kernel (what the method must do; no padding,
    no second read of a two-pass design)."""
    E = B * N * H * D
    nq, nk = math.ceil(N / q_block), math.ceil(N / k_block)
    return {
        "attn_ops": 4.0 * B * H * N * N * D,
        # Q: 2 B read + 1 B write per element + 4 B per scale (per 32-token block or token)
        "quant_q_bytes": 3.0 * E + 4.0 * B * H * nq,
        # K: 2 B read + 1 B write per element + block scales + bf16 mean
        "quant_k_bytes": 3.0 * E + 4.0 * B * H * nk + 2.0 * B * H * D,
        # V: 2 B read + 1 B write per element + fp32 mean and scale per channel
        "quant_v_bytes": 3.0 * E + 8.0 * B * H * D,
    }


def source_hash(path):
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


def traffic_record(kernel_src, workload, q_block=32, k_block=64, kernel="attn_fwd"):
    """HBM traffic per launch from the committed counter summary of this
    kernel and workload, if it was taken on the current kernel source with the
    same scale granularities (else None)."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("source_sha256_16") != source_hash(kernel_src) or rec.get("workload") != workload \
            or rec.get("q_block", 32) != q_block or rec.get("k_block", 64) != k_block:
        return None
    return rec.get("hbm_bytes_per_launch")


def host_info():
    """The CPU the oracle baseline ran on: model name, logical CPUs, and the
    CPUs this process may use."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = os.cpu_count()
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "usable_cpus": usable}


# (query, key, head) pairs of tiled oracle attention in the baseline sample:
# about 14 s on 16 host cores at the rate measured for the FLUX sample
ORACLE_SAMPLE_PAIRS = 6.0e8


def cpu_baseline(workload_cfg, seed=0):
    """The oracle as it stands, on a bounded sample of the same workload: full
    Q/K and V quantisation, plus the tiled attention for every s-th 32-query
    block of every head, s chosen so the sample holds about
    ORACLE_SAMPLE_PAIRS (query, key, head) pairs; scaled to a whole-step
    estimate.  The quantisation is also timed on one thread."""
    import numpy as np
    import oracle
    import synth
    cfg = workload_cfg
    q, k, v = synth.make_qkv(cfg, seed)
    threads = oracle.num_threads()
    t0 = time.perf_counter()
    qk = oracle.quant_qk(q, k)
    vq = oracle.quant_v(v)
    t_quant = time.perf_counter() - t0
    oracle.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.quant_qk(q, k)
        oracle.quant_v(v)
        t_quant1 = time.perf_counter() - t0
    finally:
        oracle.set_num_threads(threads)
    nb = math.ceil(cfg.N / 32)
    pairs_per_block = 32.0 * cfg.N * cfg.B * cfg.H
    stride = max(1, math.ceil(nb * pairs_per_block / ORACLE_SAMPLE_PAIRS))
    blocks = list(range(0, nb, stride))
    rows = np.array([r for b in blocks for r in range(32 * b, min(cfg.N, 32 * b + 32))], np.int32)
    t0 = time.perf_counter()
    oracle.attn_tiled(qk, vq, rows=rows)
    t_attn = time.perf_counter() - t0
    est = t_quant + t_attn * cfg.N / rows.size
    ops = algorithmic(cfg.B, cfg.N, cfg.H, cfg.D)["attn_ops"]
    return {
        "value": round(ops / est / 1e12, 6),
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"full Q/K/V quantisation ({t_quant:.2f} s on {threads} threads, {t_quant1:.2f} s "
                   f"on 1) + tiled attention on one 32-query block in {stride}: {rows.size}/{cfg.N} "
                   f"query rows of all {cfg.B * cfg.H} heads ({t_attn:.2f} s), scaled to the whole "
                   f"step ({est:.1f} s est.)"),
        "quant_s": round(t_quant, 3),
        "quant_1thread_s": round(t_quant1, 3),
        "host": host_info(),
    }


class GpuStateSampler:
    """Samples the GPU's current shader clock, memory clock and socket power
    from sysfs every `period` seconds on a thread: the starred (current) level
    of pp_dpm_sclk / pp_dpm_mclk and hwmon power1_input (microwatts) of the
    first DRM card that has them.  No child process: the bench process holds
    the GPU."""

    def __init__(self, period=0.02):
        import glob
        import threading
        self.period = period
        cards = sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        self.dev = os.path.dirname(cards[0]) if cards else None
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    @staticmethod
    def _starred_mhz(path):
        with open(path) as f:
            for line in f:
                if line.rstrip().endswith("*"):
                    tok = line.split(":", 1)[1].strip().rstrip("*").strip().lower()
                    return float(tok.replace("mhz", ""))
        return None

    def _read(self):
        import glob
        sclk = self._starred_mhz(os.path.join(self.dev, "pp_dpm_sclk"))
        mclk = self._starred_mhz(os.path.join(self.dev, "pp_dpm_mclk"))
        power = None
        for h in sorted(glob.glob(os.path.join(self.dev, "hwmon", "hwmon*", "power1_input"))):
            with open(h) as f:
                power = int(f.read().strip()) * 1e-6
            break
        return sclk, mclk, power

    def _run(self):
        while not self._stop.is_set():
            try:
                self.samples.append(self._read())
            except (OSError, ValueError, IndexError):
                pass
            self._stop.wait(self.period)

    def __enter__(self):
        if self.dev:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        if self.dev:
            self._stop.set()
            self._thread.join()
        return False

    def summary(self):
        if not self.samples:
            return {"source": "sysfs", "samples": 0, "note": "no readable pp_dpm_sclk on this host"}

        def stats(i, nd=0):
            xs = sorted(x[i] for x in self.samples if x[i] is not None)
            if not xs:
                return None
            return {"min": round(xs[0], nd), "median": round(xs[len(xs) // 2], nd), "max": round(xs[-1], nd)}

        return {"source": f"sysfs {self.dev}: pp_dpm_sclk, pp_dpm_mclk (starred level), "
                          "hwmon power1_input", "samples": len(self.samples),
                "sclk_mhz": stats(0), "mclk_mhz": stats(1), "socket_power_w": stats(2)}


class GraphTimingEvent:
    """A HIP timing event that a captured graph records on every replay.

    While its stream is being captured, record() adds an event-record node to
    the capture graph after the stream's current dependencies and makes that
    node the stream's only dependency, so the node sits between the calls it
    brackets (hipStreamGetCaptureInfo_v2, hipGraphAddEventRecordNode,
    hipStreamUpdateCaptureDependencies).  Outside capture it is a plain
    hipEventRecord.  torch's Event refuses external=True on ROCm, and this HIP
    rejects hipEventRecordWithFlags(..., hipEventRecordExternal) during capture.
    Uses the HIP runtime already loaded in the process (torch's, soname
    libamdhip64.so.7)."""

    _hip = None

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            import ctypes as ct
            hip = ct.CDLL("libamdhip64.so.7")
            vp, pvp = ct.c_void_p, ct.POINTER(ct.c_void_p)
            hip.hipEventCreate.argtypes = [pvp]
            hip.hipEventRecord.argtypes = [vp, vp]
            hip.hipEventElapsedTime.argtypes = [ct.POINTER(ct.c_float), vp, vp]
            hip.hipStreamGetCaptureInfo_v2.argtypes = [vp, ct.POINTER(ct.c_int),
                                                       ct.POINTER(ct.c_ulonglong), pvp,
                                                       ct.POINTER(pvp), ct.POINTER(ct.c_size_t)]
            hip.hipGraphAddEventRecordNode.argtypes = [pvp, vp, pvp, ct.c_size_t, vp]
            hip.hipStreamUpdateCaptureDependencies.argtypes = [vp, pvp, ct.c_size_t, ct.c_uint]
            cls._hip = hip
        return cls._hip

    @staticmethod
    def _check(err, what):
        if err != 0:
            raise RuntimeError(f"{what} failed (hipError {err})")

    def __init__(self):
        import ctypes as ct
        self._ct = ct
        self.ev = ct.c_void_p()
        self._check(self._lib().hipEventCreate(ct.byref(self.ev)), "hipEventCreate")

    def record(self, stream):
        ct, hip = self._ct, self._lib()
        sp = ct.c_void_p(int(stream.cuda_stream))
        status, cid, graph = ct.c_int(), ct.c_ulonglong(), ct.c_void_p()
        deps, ndeps = ct.POINTER(ct.c_void_p)(), ct.c_size_t()
        self._check(hip.hipStreamGetCaptureInfo_v2(sp, ct.byref(status), ct.byref(cid), ct.byref(graph),
                                                   ct.byref(deps), ct.byref(ndeps)),
                    "hipStreamGetCaptureInfo_v2")
        if status.value == 0:  # hipStreamCaptureStatusNone
            self._check(hip.hipEventRecord(self.ev, sp), "hipEventRecord")
            return
        if status.value != 1:  # hipStreamCaptureStatusActive
            raise RuntimeError("stream capture invalidated")
        dep_list = (ct.c_void_p * max(1, ndeps.value))(*[deps[i] for i in range(ndeps.value)])
        node = ct.c_void_p()
        self._check(hip.hipGraphAddEventRecordNode(ct.byref(node), graph, dep_list, ndeps.value, self.ev),
                    "hipGraphAddEventRecordNode")
        self._check(hip.hipStreamUpdateCaptureDependencies(sp, ct.byref(node), 1, 1),
                    "hipStreamUpdateCaptureDependencies")

    def elapsed_time(self, end):
        ms = self._ct.c_float()
        self._check(self._lib().hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev),
                    "hipEventElapsedTime")
        return float(ms.value)


def gpu_state_during(run_step, torch, seconds=1.0):
    """Clock and power while the step runs back to back for `seconds` (a pass
    of its own, after the timed steps)."""
    with GpuStateSampler() as smp:
        t_end = time.perf_counter() + seconds
        while time.perf_counter() < t_end:
            for _ in range(4):
                run_step()
            torch.cuda.synchronize()
    return smp.summary()


def copy_calibration(torch, dev):
    """One 256 MiB device-to-device copy: a kernel of known HBM traffic for
    scaling FETCH_SIZE / WRITE_SIZE counter readings."""
    src = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


# multiply-accumulates of the oracle GEMM in the projection baseline sample:
# about 11 s on 16 host cores at the rate measured for a smaller sample
ORACLE_GEMM_SAMPLE_MACS = 2.5e11


def proj_cpu_baseline(M, K, N, seed=0):
    """The oracle on a bounded sample of the projection: the row quantisation of
    X and W in full, the scaled GEMM on every output row and every s-th
    column, s chosen so the sample holds about ORACLE_GEMM_SAMPLE_MACS
    multiply-accumulates; scaled to the whole step."""
    import numpy as np
    import oracle
    import synth
    x, w, b = synth.proj_inputs(M, K, N, seed)
    t0 = time.perf_counter()
    xc, xs = oracle.quant_rows_e4m3(x)
    t_q = time.perf_counter() - t0
    wc, ws = oracle.quant_rows_e4m3(w)
    stride = max(1, math.ceil(float(M) * N * K / ORACLE_GEMM_SAMPLE_MACS))
    rows = np.arange(0, M, dtype=np.int32)
    cols = np.arange(0, N, stride, dtype=np.int32)
    t0 = time.perf_counter()
    oracle.gemm_fp8_rowwise(xc, xs, wc, ws, bias=b, rows=rows, cols=cols)
    t_g = time.perf_counter() - t0
    est = t_q + t_g * (M * N) / (rows.size * cols.size)
    return {
        "value": round(2.0 * M * N * K / est / 1e12, 6),
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": (f"row quantisation of X in full ({t_q:.2f} s) + the scaled GEMM on "
                   f"{rows.size} x {cols.size} of the {M} x {N} outputs ({t_g:.2f} s), scaled "
                   f"to the whole step ({est:.1f} s est.)"),
        "host": host_info(),
    }


def run_projection(args, torch, synth, sage):
    """--workload vmlp_proj: the row-wise FP8 V + MLP projection of a FLUX-like
    block.  One step = sage_quant_rows_fp8 on the activation + the scaled FP8
    GEMM; the weight is quantised once, outside the timed region (the pages'
    FP8 packages ship E4M3 weights with their row scales)."""
    lib = sage.lib()
    M, K, N = synth.PROJ_SHAPES["vmlp_proj"]
    dev = torch.device("cuda:0")
    x, w, b = (t.to(dev) for t in synth.proj_inputs(M, K, N, args.seed))
    wc, ws = sage.quant_rows_fp8(w)
    xc = torch.empty((M, K), dtype=torch.uint8, device=dev)
    xs = torch.empty((M,), dtype=torch.float32, device=dev)
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    sp = int(torch.cuda.current_stream().cuda_stream)

    def step(evs=None):
        if evs:
            evs[0].record()
        st = lib.sage_quant_rows_fp8(x.data_ptr(), x.stride(0), M, K, xc.data_ptr(), xs.data_ptr(), sp)
        if evs:
            evs[1].record()
        st |= lib.sage_gemm_fp8_rowwise(xc.data_ptr(), xs.data_ptr(), M, wc.data_ptr(), ws.data_ptr(),
                                        N, K, b.data_ptr(), out.data_ptr(), out.stride(0), sp)
        if evs:
            evs[2].record()
        if st != 0:
            raise RuntimeError(f"libsage call failed with status {st}")

    pw = prewarm(step, torch, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps, each call bracketed by events on the stream it runs on
    evs_all = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record()
    for i in range(args.steps):
        step(evs_all[i])
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    per = {"quant_rows_x": [e[0].elapsed_time(e[1]) for e in evs_all],
           "gemm": [e[1].elapsed_time(e[2]) for e in evs_all]}
    stat = {k: {"avg": round(sum(v) / len(v), 5), "median": round(sorted(v)[len(v) // 2], 5),
                "min": round(min(v), 5), "p90": round(sorted(v)[min(len(v) - 1, 9 * len(v) // 10)], 5)}
            for k, v in per.items()}
    flops = 2.0 * M * N * K
    g_avg = stat["gemm"]["avg"]
    gemm_tflops = flops / (g_avg * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8-e4m3 x fp8-e4m3, fp32 accum, bf16 out",
        "data": "synthetic (seeded counter-based normals: X N(0,1), W N(0,1/K), bias N(0,0.01), bf16)",
        "config": {"workload": "vmlp_proj", "M": M, "K": K, "N": N, "seed": args.seed,
                   "weights": "quantised once outside the timed region"},
        "prewarm": pw,
        "kernels_ms": stat,
        "kernels_ms_source": "HIP events around each call inside the timed steps",
        "quant_rows_gbs": round(3.0 * M * K / (stat["quant_rows_x"]["avg"] * 1e-3) / 1e9, 1),
        "roofline": {"kernel": "sage_gemm_fp8_rowwise (gemm_fp8_kernel: 256 x 256 blocks, 8 waves)",
                     "bound": "mfma", "achieved": round(gemm_tflops, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(gemm_tflops / PEAK_MFMA_TFLOPS, 4),
                     "traffic": traffic_record(os.path.join(ROOT, "quantized_attention_video_smooth_amd",
                                                            "csrc", "sage_proj.hip"), "vmlp_proj",
                                               kernel="gemm_fp8")},
    }
    if args.gpu_state_seconds > 0:
        res["gpu_state"] = gpu_state_during(step, torch, args.gpu_state_seconds)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = proj_cpu_baseline(M, K, N, args.seed)
    return res


def sp_shard(N, P, rank):
    """Token range of `rank` when the sequence is split P ways in shards of a
    multiple of 64 tokens (the last shard takes the rest)."""
    size = math.ceil(N / P / 64) * 64
    a = rank * size
    return a, min(N, a + size)


def run_sp_share(args, torch, synth, sage, cfg):
    """One rank's share of a P-way sequence-parallel step on this GPU: the
    rank's Q shard quantised (sage_quant_q) and its queries against the K and V
    codes of the whole sequence (sage_attn_fwd_shard).  K and V are quantised
    once before the timed region: they stand for the codes the rank gathers.
    Not in the step: the rank's K/V shard quantisation with all-reduced
    statistics and the K/V all-gather, which need the other ranks."""
    lib = sage.lib()
    B, N, H, D = cfg.B, cfg.N, cfg.H, cfg.D
    P, rank = args.sp, args.sp_rank
    a, b = sp_shard(N, P, rank)
    if not (0 <= rank and a < N):
        raise SystemExit(f"--sp-rank {rank} holds no tokens of N={N} split {P} ways")
    Nq = b - a
    dev = torch.device("cuda:0")
    q, k, v = synth.make_qkv(cfg, args.seed, device=dev)
    qb, kbl = args.q_block, args.k_block
    kq = sage.quant_qk(q, k, q_block=qb, k_block=kbl)
    vq = sage.quant_v(v)
    qs = q[:, a:b]
    Npq = sage.sage_padded_tokens(Nq)
    q_i8 = torch.empty((B, H, Npq, D), dtype=torch.int8, device=dev)
    q_scale = torch.empty((B, H, Npq // qb), dtype=torch.float32, device=dev)
    out = torch.empty((B, Nq, H, D), dtype=torch.bfloat16, device=dev)
    sp_ = int(torch.cuda.current_stream().cuda_stream)
    os_ = out.stride()[:3]

    def step(evs=None):
        if evs:
            evs[0].record()
        st = lib.sage_quant_q(qs.data_ptr(), *qs.stride()[:3], B, Nq, H, D, q_i8.data_ptr(),
                              q_scale.data_ptr(), qb, sp_)
        if evs:
            evs[1].record()
        st |= lib.sage_attn_fwd_shard(q_i8.data_ptr(), q_scale.data_ptr(), Nq, kq[2].data_ptr(),
                                      kq[3].data_ptr(), vq[0].data_ptr(), vq[1].data_ptr(),
                                      vq[2].data_ptr(), N, B, H, D, 0.0, out.data_ptr(), *os_, qb, kbl,
                                      sp_)
        if evs:
            evs[2].record()
        if st != 0:
            raise RuntimeError(f"libsage call failed with status {st}")

    pw = prewarm(step, torch, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # timed steps, each call bracketed by events on its stream
    evs_all = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(evs_all[i])
    t1.record()
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps
    per = {"quant_q": [e[0].elapsed_time(e[1]) for e in evs_all],
           "attn_fwd_shard": [e[1].elapsed_time(e[2]) for e in evs_all]}
    stat = {k2: {"avg": round(sum(v2) / len(v2), 5), "median": round(sorted(v2)[len(v2) // 2], 5),
                 "min": round(min(v2), 5), "p90": round(sorted(v2)[min(len(v2) - 1, 9 * len(v2) // 10)], 5)}
            for k2, v2 in per.items()}
    ops = 4.0 * B * H * Nq * N * D
    at = ops / (stat["attn_fwd_shard"]["avg"] * 1e-3) / 1e12
    waves, wgs = sage.sage_attn_launch_shape(B, Nq, H, D)
    res = {
        "metric": METRIC,
        "value": round(ops / (ms_per_step * 1e-3) / 1e12, 3),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 QK / fp8-e4m3 PV, fp32 softmax+accum",
        "data": "synthetic (seeded counter-based normals, bf16 NHD)",
        "config": {"workload": f"{cfg.name}, rank {rank} of a {P}-way sequence split", "B": B, "N": N,
                   "H": H, "D": D, "queries": [a, b], "keys": N, "q_block": qb, "k_block": kbl,
                   "not_in_step": "K/V shard quantisation with all-reduced statistics, K/V all-gather"},
        "prewarm": pw,
        "kernels_ms": stat,
        "kernels_ms_source": "HIP events around each call inside the timed steps",
        "roofline": {"kernel": f"sage_attn_fwd_shard (attn_fwd_kernel<{D}, {waves}, {kbl}, {attn_sch(waves)}>: "
                               f"{waves}-wave workgroups, {wgs} per launch)",
                     "bound": "mfma", "achieved": round(at, 2), "peak": PEAK_MFMA_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(at / PEAK_MFMA_TFLOPS, 4), "traffic": None},
    }
    if args.gpu_state_seconds > 0:
        res["gpu_state"] = gpu_state_during(step, torch, args.gpu_state_seconds)
    return res


def prewarm(run_step, torch, ms):
    """Back-to-back steps for at least `ms` of wall time before the counted
    warm-up: the GPU clock ramps up over the first tens of ms of load, so a
    short --warmup alone would leave the timed steps inside the ramp."""
    if ms <= 0:
        return {"ms": 0.0, "steps": 0}
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(4):
            run_step()
        n += 4
        torch.cuda.synchronize()
        el = (time.perf_counter() - t0) * 1e3
        if el >= ms:
            return {"ms": round(el, 1), "steps": n}


def attn_sch(waves, schedule=0):
    """The attention kernel's schedule template argument for a launch of this
    workgroup size under sage_attn_schedule(schedule): interleaved (1) by
    default, the compiler's order (0) when forced with schedule 1."""
    return {0: 1, 1: 0, 2: 1}[schedule]


def parse_variant(spec):
    """'opt=val[;opt=val...]' -> {opt: val} over the step options an ABBA
    comparison may vary (streams, producer, q_block, k_block, attention
    workgroup size and key-step schedule, quantiser calls per step)."""
    allowed = {"streams": int, "producer": str, "q_block": int, "k_block": int, "waves": int,
               "sched": int, "events": str, "qgroups": int}
    out = {}
    if spec in ("", "default"):
        return out
    for part in spec.split(";"):
        key, _, val = part.partition("=")
        key = key.strip().replace("-", "_")
        if key not in allowed or not val:
            raise SystemExit(f"--abba: unknown variant option {part!r} (allowed: {sorted(allowed)})")
        out[key] = allowed[key](val.strip())
    if out.get("producer", "none") not in ("none", "fused", "composed"):
        raise SystemExit("--abba: producer is none, fused or composed")
    if out.get("events", "roofline") not in ("roofline", "all"):
        raise SystemExit("--abba: events is roofline (the timed call only) or all (every call)")
    if out.get("streams", 1) not in (1, 2) or out.get("q_block", 32) not in (1, 32) \
            or out.get("k_block", 64) not in (16, 64) or out.get("waves", 0) not in (0, 4, 8) \
            or out.get("sched", 0) not in (0, 1, 2) or not 1 <= out.get("qgroups", 1) <= 40:
        raise SystemExit("--abba: streams 1|2, q_block 1|32, k_block 16|64, waves 0|4|8, sched 0|1|2, "
                         "qgroups 1..40")
    return out


class AttentionPath:
    """Inputs, outputs and workspaces of one workload, resident in HBM, and the
    step of the path over them: sage_quant_qk (or the QK producer in front of
    it) + sage_quant_v + sage_attn_fwd (no attention for quant_long).  Scale
    buffers are sized for the finest granularities, so one instance serves
    every step variant."""

    def __init__(self, torch, synth, sage, cfg, seed, need_producer):
        self.torch, self.sage, self.cfg = torch, sage, cfg
        self.lib = sage.lib()
        B, N, H, D = cfg.B, cfg.N, cfg.H, cfg.D
        Np = sage.sage_padded_tokens(N)
        dev = self.dev = torch.device("cuda:0")
        self.q, self.k, self.v = synth.make_qkv(cfg, seed, device=dev)
        self.q_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
        self.q_scale = torch.empty((B, H, Np), dtype=torch.float32, device=dev)
        self.k_i8 = torch.empty((B, H, Np, D), dtype=torch.int8, device=dev)
        self.k_scale = torch.empty((B, H, Np // 16), dtype=torch.float32, device=dev)
        self.k_mean = torch.empty((B, H, D), dtype=torch.bfloat16, device=dev)
        self.v_fp8 = torch.empty((B, H, D, Np), dtype=torch.uint8, device=dev)
        self.v_scale = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        self.v_mean = torch.empty((B, H, D), dtype=torch.float32, device=dev)
        self.out = torch.empty((B, N, H, D), dtype=torch.bfloat16, device=dev)
        # zero-filled: the quantisers' arrival counters start at zero
        self.ws_qk = torch.zeros(max(sage.sage_quant_qk_workspace_size(B, N, H, D),
                                     sage.sage_norm_rope_quant_qk_workspace_size(B, N, H, D)),
                                 dtype=torch.uint8, device=dev)
        self.ws_v = torch.zeros(sage.sage_quant_v_workspace_size(B, N, H, D), dtype=torch.uint8, device=dev)
        if need_producer:
            self.wq = synth.norm_weight(cfg, "q").to(dev)
            self.wk = synth.norm_weight(cfg, "k").to(dev)
            self.rope = torch.from_numpy(synth.rope_table(N, D)).to(dev)
            self.yq = torch.empty_like(self.q)
            self.yk = torch.empty_like(self.k)
        self.stream = torch.cuda.current_stream()
        self.side = torch.cuda.Stream(device=dev)  # default priority
        self.ev_in = [torch.cuda.Event() for _ in range(2)]
        self.do_attn = cfg.name != "quant_long"

    def step_fn(self, streams, producer, qb, kbl, waves=None, sched=None, qgroups=1):
        """The step for these options.  step(evs=None, main=None): evs maps a
        call name to its (start, end) events, recorded on the stream the call
        runs on; main is the step's stream (the capture stream under --graph).
        With streams == 2, sage_quant_v runs on a side stream beside the Q/K
        segment and the attention waits for both.  qgroups > 1 (B = 1 only)
        runs each quantiser as that many calls over consecutive head groups,
        each call's statistics pass followed by its quantisation: the second
        read of a group's K or V then follows its first closely."""
        lib, cfg = self.lib, self.cfg
        B, N, H, D = cfg.B, cfg.N, cfg.H, cfg.D
        q, k, v, out = self.q, self.k, self.v, self.out
        qs, ks, vs, os_ = q.stride()[:3], k.stride()[:3], v.stride()[:3], out.stride()[:3]
        side, side_p, ev_in = self.side, int(self.side.cuda_stream), self.ev_in
        eps = 1e-6
        pq = (self.q_i8.data_ptr(), self.q_scale.data_ptr(), self.k_i8.data_ptr(), self.k_scale.data_ptr(),
              self.k_mean.data_ptr())
        pv = (self.v_fp8.data_ptr(), self.v_scale.data_ptr(), self.v_mean.data_ptr())
        ws_qk, ws_v = self.ws_qk, self.ws_v
        if qgroups > 1 and (B != 1 or producer != "none" or qgroups > H):
            raise SystemExit("qgroups > 1 needs B = 1, no producer and at most H groups")
        hg = [(H * g // qgroups, H * (g + 1) // qgroups) for g in range(qgroups)]
        Np = self.sage.sage_padded_tokens(N)

        def heads(h0):
            """Pointer offsets of head h0 (B = 1): inputs by their head stride,
            outputs head-major and contiguous."""
            return ((q.data_ptr() + 2 * h0 * qs[2], k.data_ptr() + 2 * h0 * ks[2], v.data_ptr() + 2 * h0 * vs[2]),
                    (pq[0] + h0 * Np * D, pq[1] + 4 * h0 * (Np // qb), pq[2] + h0 * Np * D,
                     pq[3] + 4 * h0 * (Np // kbl), pq[4] + 2 * h0 * D),
                    (pv[0] + h0 * D * Np, pv[1] + 4 * h0 * D, pv[2] + 4 * h0 * D))

        def qk_call(sp_):
            if qgroups > 1:
                st_ = 0
                for h0, h1 in hg:
                    (pq_in, pk_in, _), pq_out, _ = heads(h0)
                    st_ |= lib.sage_quant_qk_ex(pq_in, *qs, pk_in, *ks, B, N, h1 - h0, D, *pq_out,
                                                ws_qk.data_ptr(), ws_qk.numel(), qb, kbl, sp_)
                return st_
            if producer == "fused":
                return lib.sage_norm_rope_quant_qk(
                    q.data_ptr(), *qs, k.data_ptr(), *ks, B, N, H, D, self.wq.data_ptr(), self.wk.data_ptr(),
                    self.rope.data_ptr(), eps, *pq, ws_qk.data_ptr(), ws_qk.numel(), qb, kbl, sp_)
            src_q, src_k = q, k
            st_ = 0
            if producer == "composed":
                yq, yk = self.yq, self.yk
                st_ |= lib.sage_norm_rope(q.data_ptr(), *qs, B, N, H, D, self.wq.data_ptr(),
                                          self.rope.data_ptr(), eps, yq.data_ptr(), *yq.stride()[:3], sp_)
                st_ |= lib.sage_norm_rope(k.data_ptr(), *ks, B, N, H, D, self.wk.data_ptr(),
                                          self.rope.data_ptr(), eps, yk.data_ptr(), *yk.stride()[:3], sp_)
                src_q, src_k = yq, yk
            st_ |= lib.sage_quant_qk_ex(src_q.data_ptr(), *src_q.stride()[:3], src_k.data_ptr(),
                                        *src_k.stride()[:3], B, N, H, D, *pq, ws_qk.data_ptr(),
                                        ws_qk.numel(), qb, kbl, sp_)
            return st_

        def step(evs=None, main=None):
            if waves is not None:
                lib.sage_attn_tuning(waves)
            if sched is not None:
                lib.sage_attn_schedule(sched)
            two = streams == 2
            stream_ = self.stream if main is None else main
            sp_ = int(stream_.cuda_stream)

            def rec(name, i, s_):
                if evs and name in evs:
                    evs[name][i].record(s_)

            st = 0
            if two:
                ev_in[0].record(stream_)
                side.wait_event(ev_in[0])
            vs_, vp_ = (side, side_p) if two else (stream_, sp_)
            rec("quant_qk", 0, stream_)
            st |= qk_call(sp_)
            rec("quant_qk", 1, stream_)
            rec("quant_v", 0, vs_)
            for h0, h1 in hg:
                (_, _, pv_in), _, pv_out = heads(h0)
                st |= lib.sage_quant_v(pv_in, *vs, B, N, h1 - h0, D, *pv_out, ws_v.data_ptr(), ws_v.numel(), vp_)
            rec("quant_v", 1, vs_)
            if two:
                ev_in[1].record(side)
                stream_.wait_event(ev_in[1])
            if self.do_attn:
                rec("attn_fwd", 0, stream_)
                st |= lib.sage_attn_fwd_ex(pq[0], pq[1], pq[2], pq[3], *pv, B, N, H, D, 0.0,
                                           out.data_ptr(), *os_, qb, kbl, sp_)
                rec("attn_fwd", 1, stream_)
            if st != 0:
                raise RuntimeError(f"libsage call failed with status {st}")

        return step


def _stats(v2):
    s = sorted(v2)
    return {"avg": round(sum(v2) / len(v2), 5), "median": round(s[len(s) // 2], 5),
            "min": round(s[0], 5), "p90": round(s[min(len(s) - 1, (9 * len(s)) // 10)], 5)}


def measure_path(args, cfg, torch, synth, sage, streams):
    """The workload's step: pre-warm, warm-up, K timed steps with per-call HIP
    events.  Returns the fields of its JSON result (no cpu_baseline)."""
    B, N, H, D = cfg.B, cfg.N, cfg.H, cfg.D
    qb, kbl, prod = args.q_block, args.k_block, args.producer
    path = AttentionPath(torch, synth, sage, cfg, args.seed, prod != "none")
    step = path.step_fn(streams, prod, qb, kbl)
    stream, dev, do_attn = path.stream, path.dev, path.do_attn
    pw = prewarm(step, torch, args.prewarm_ms)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    names = ["quant_qk", "quant_v"] + (["attn_fwd"] if do_attn else [])
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    if args.graph:
        # The K timed steps captured as one HIP graph, the roofline's call
        # bracketed in each step by timing events that the graph records on
        # that call's stream.  After the eager warm-up one untimed replay warms
        # the graph; the timed region is one replay.  The library allocates
        # nothing and issues no memset, so the graph holds only the steps'
        # kernels and events.  Only the roofline's call is bracketed: each
        # event node costs about as much as replay saves over eager launches.
        timed = ["attn_fwd"] if do_attn else ["quant_qk"]
        evs_all = [{k2: (GraphTimingEvent(), GraphTimingEvent()) for k2 in timed}
                   for _ in range(args.steps)]
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream(device=dev)  # default priority
        cap.wait_stream(stream)
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(evs_all[i], main=cap)
        stream.wait_stream(cap)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        t_start.record(stream)
        graph.replay()
        t_end.record(stream)
        torch.cuda.synchronize()
        kernels_src = (f"HIP events around {timed[0]} inside the timed steps (event-record nodes of the "
                       "replayed graph, on the call's stream)")
    else:
        # Only the roofline's calls are bracketed inside the timed steps: each
        # recorded event adds a dependency gap of several us to the stream
        # (FLUX step 411 us without events, 417 with them around the attention,
        # 433 around all three calls).  With attention, the quantisers' per-call
        # times come from as many further steps with events around every call.
        timed = ["attn_fwd"] if do_attn else names
        evs_all = [{k2: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for k2 in timed} for _ in range(args.steps)]
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(args.steps):
            step(evs_all[i])
        t_end.record(stream)
        torch.cuda.synchronize()
        kernels_src = ("HIP events around " + ", ".join(timed) + " inside the timed steps, on the call's "
                       "stream")
        if do_attn:
            evs_more = [{k2: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                         for k2 in ("quant_qk", "quant_v")} for _ in range(args.steps)]
            for i in range(args.steps):
                step(evs_more[i])
            torch.cuda.synchronize()
            for i in range(args.steps):
                evs_all[i].update(evs_more[i])
            kernels_src += ("; quant_qk and quant_v from as many further steps with events around every "
                            "call")
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    per = {k2: [e[k2][0].elapsed_time(e[k2][1]) for e in evs_all] for k2 in evs_all[0]}
    kstats = {k2: _stats(v2) for k2, v2 in per.items()}
    avg = {k2: s["avg"] for k2, s in kstats.items()}

    work = algorithmic(B, N, H, D, qb, kbl)
    if prod != "none":
        # the rotation table, read once per step (the weights are negligible);
        # the Q/K segment's bytes are otherwise those of the quantiser
        work["quant_q_bytes"] += 4.0 * N * D
    step_s = ms_per_step * 1e-3
    res = {"ms_per_step": round(ms_per_step, 5), "prewarm": pw}
    if do_attn:
        waves, wgs = sage.sage_attn_launch_shape(B, N, H, D)
        attn_tflops = work["attn_ops"] / (avg["attn_fwd"] * 1e-3) / 1e12
        res["value"] = round(work["attn_ops"] / step_s / 1e12, 3)
        res["unit"] = "TFLOPS"
        res["roofline"] = {
            "kernel": f"sage_attn_fwd (attn_fwd_kernel<{D}, {waves}, {kbl}, {attn_sch(waves)}>: {waves}-wave "
                      f"workgroups, {wgs} per launch)",
            "bound": "mfma",
            "achieved": round(attn_tflops, 2),
            "peak": PEAK_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_MFMA_TFLOPS, 4),
            "traffic": traffic_record(os.path.join(ROOT, "quantized_attention_video_smooth_amd",
                                                   "csrc", "sage_attn.hip"), cfg.name, qb, kbl),
        }
        res["attn_tflops"] = round(attn_tflops, 2)
    else:
        qv_bytes = work["quant_q_bytes"] + work["quant_k_bytes"] + work["quant_v_bytes"]
        res["value"] = round(qv_bytes / step_s / 1e9, 3)
        res["unit"] = "GB/s"
        gbs = (work["quant_q_bytes"] + work["quant_k_bytes"]) / (avg["quant_qk"] * 1e-3) / 1e9
        gbs_v = work["quant_v_bytes"] / (avg["quant_v"] * 1e-3) / 1e9
        src = os.path.join(ROOT, "quantized_attention_video_smooth_amd", "csrc", "sage_quant.hip")
        res["roofline"] = {"kernel": "sage_quant_qk (its statistics kernel, which also finalises "
                                     "each head, and its quantisation kernel; one call)",
                           "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(gbs / PEAK_HBM_GBS, 4),
                           "traffic": traffic_record(src, cfg.name, qb, kbl, kernel="quant_qk")}
        res["roofline_quant_v"] = {"kernel": "sage_quant_v (its statistics kernel, which also finalises "
                                             "each head, and its quantisation kernel; one call)",
                                   "bound": "hbm", "achieved": round(gbs_v, 1), "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": round(gbs_v / PEAK_HBM_GBS, 4),
                                   "traffic": traffic_record(src, cfg.name, qb, kbl, kernel="quant_v")}
        res["quant_qk_gbs"] = round(gbs, 1)
        res["quant_v_gbs"] = round(gbs_v, 1)
    res["config"] = {"workload": cfg.name, "B": B, "N": N, "H": H, "D": D, "causal": False,
                     "layout": "NHD bf16 in, bf16 out", "seed": args.seed,
                     "streams": streams, "graph": bool(args.graph), "q_block": qb, "k_block": kbl,
                     "producer": prod}
    res["kernels_ms"] = kstats
    res["kernels_ms_source"] = kernels_src
    res["_step"] = step
    return res


def run_abba(args, cfg, torch, synth, sage):
    """Same-process ABBA comparison of two step variants on one workload (the
    pages' protocol for their last gains): every group times K steps of A, K
    of B, K of B, K of A, each block bracketed by events; a group gives the
    mean step time of each variant and their ratio B/A."""
    specs = args.abba.split(",")
    if len(specs) != 2:
        raise SystemExit("--abba takes two variants: A,B (each 'opt=val[;opt=val]' or 'default')")
    base = {"streams": args.streams, "producer": args.producer, "q_block": args.q_block,
            "k_block": args.k_block, "waves": 0, "sched": 0, "events": "roofline", "qgroups": 1}
    var = []
    for s in specs:
        o = dict(base)
        o.update(parse_variant(s))
        var.append(o)
    need_prod = any(o["producer"] != "none" for o in var)
    path = AttentionPath(torch, synth, sage, cfg, args.seed, need_prod)
    steps = [path.step_fn(o["streams"], o["producer"], o["q_block"], o["k_block"], o["waves"], o["sched"],
                          o["qgroups"]) for o in var]
    key = "attn_fwd" if path.do_attn else "quant_qk"
    every = ["quant_qk", "quant_v"] + (["attn_fwd"] if path.do_attn else [])

    def block(step, events):
        # events "all": every call bracketed, as the timed steps once were
        names = every if events == "all" else [key]
        evs = [{k2: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                for k2 in names} for _ in range(args.steps)]
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record(path.stream)
        for i in range(args.steps):
            step(evs[i])
        t1.record(path.stream)
        torch.cuda.synchronize()
        call = [e[key][0].elapsed_time(e[key][1]) for e in evs]
        return t0.elapsed_time(t1) / args.steps, sum(call) / len(call)

    pw = prewarm(lambda: (steps[0](), steps[1]()), torch, args.prewarm_ms)
    for _ in range(args.warmup):
        steps[0]()
        steps[1]()
    torch.cuda.synchronize()
    groups = []
    for _ in range(args.abba_groups):
        ea, eb = var[0]["events"], var[1]["events"]
        a1, b1, b2, a2 = block(steps[0], ea), block(steps[1], eb), block(steps[1], eb), block(steps[0], ea)
        ga = ((a1[0] + a2[0]) / 2, (a1[1] + a2[1]) / 2)
        gb = ((b1[0] + b2[0]) / 2, (b1[1] + b2[1]) / 2)
        groups.append({"A_step_ms": round(ga[0], 5), "B_step_ms": round(gb[0], 5),
                       f"A_{key}_ms": round(ga[1], 5), f"B_{key}_ms": round(gb[1], 5),
                       "ratio_step": round(gb[0] / ga[0], 5), f"ratio_{key}": round(gb[1] / ga[1], 5)})

    def med(xs):
        s = sorted(xs)
        return s[len(s) // 2]

    return {
        "mode": "abba",
        "workload": cfg.name,
        "A": var[0], "B": var[1],
        "groups": args.abba_groups, "steps_per_block": args.steps, "warmup": args.warmup, "prewarm": pw,
        "median_A_step_ms": med([g["A_step_ms"] for g in groups]),
        "median_B_step_ms": med([g["B_step_ms"] for g in groups]),
        f"median_A_{key}_ms": med([g[f"A_{key}_ms"] for g in groups]),
        f"median_B_{key}_ms": med([g[f"B_{key}_ms"] for g in groups]),
        "median_ratio_step": med([g["ratio_step"] for g in groups]),
        f"median_ratio_{key}": med([g[f"ratio_{key}"] for g in groups]),
        "ratio_step_range": [min(g["ratio_step"] for g in groups), max(g["ratio_step"] for g in groups)],
        "per_group": groups,
    }


# The metric's other parts, measured after the main workload in a default run
# (attention at N = 32760, quantiser GB/s on the quant-only shape).
DEFAULT_PARTS = ("video_early", "long_t2v", "quant_long")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prewarm-ms", type=float, default=300.0,
                    help="back-to-back untimed steps for at least this many ms before the counted "
                         "warm-up of each workload (the GPU clock ramps up over the first tens of ms "
                         "of load); reported as 'prewarm'")
    ap.add_argument("--workload", default="flux_joint",
                    choices=["tiny", "flux_joint", "video_early", "long_t2v", "quant_long", "vmlp_proj"])
    ap.add_argument("--parts", default=None,
                    help="comma-separated further workloads measured in the same run and reported under "
                         "'parts' (default: video_early,long_t2v,quant_long when the workload is flux_joint, none "
                         "otherwise; 'none' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--streams", type=int, choices=[1, 2], default=1,
                    help="1 (default): the three calls in order on one stream, so each call's event "
                         "window is its own. 2: sage_quant_v runs on a second stream beside "
                         "sage_quant_qk (they are independent) and the attention waits for both "
                         "(same-process ABBA: no faster at FLUX or Long T2V, 2%% slower at video early)")
    ap.add_argument("--q-block", type=int, choices=[32, 1], default=32,
                    help="Q scale granularity: one scale per 32-token block (default) or per token")
    ap.add_argument("--k-block", type=int, choices=[64, 16], default=64,
                    help="K scale granularity: one scale per 64-token key tile (default) or per 16 tokens")
    ap.add_argument("--producer", choices=["none", "fused", "composed"], default="none",
                    help="inputs are pre-norm Q and K of a QK RMSNorm + RoPE producer: 'fused' runs "
                         "sage_norm_rope_quant_qk, 'composed' runs sage_norm_rope on Q and on K "
                         "(bf16 NHD stores) and then sage_quant_qk_ex; 'none' (default) quantises "
                         "Q and K as given")
    ap.add_argument("--gpu-state-seconds", type=float, default=1.0,
                    help="length of the pass of back-to-back steps during which the GPU clock and power "
                         "are sampled (0: no such pass, e.g. under a profiler)")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps as one HIP graph, with timing events around the "
                         "roofline's call only; after the eager warm-up, replay it once untimed and "
                         "once timed")
    ap.add_argument("--sp", type=int, default=1,
                    help="P > 1: time one rank's share of a P-way sequence-parallel step (its Q shard "
                         "against the whole gathered K/V; no collectives), for --sp-rank")
    ap.add_argument("--sp-rank", type=int, default=0)
    ap.add_argument("--abba", default=None,
                    help="A,B: same-process ABBA comparison of two step variants on --workload, each "
                         "'opt=val[;opt=val]' over streams, producer, q_block, k_block, waves (attention "
                         "workgroup size 0|4|8), sched (attention key-step schedule 0|1|2), events "
                         "(roofline|all: which calls the timed steps bracket with events), qgroups (B = 1: "
                         "each quantiser as that many calls over head groups) (or 'default'); "
                         "--steps steps per block, --abba-groups groups")
    ap.add_argument("--abba-groups", type=int, default=15)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the run, copy 256 MiB device to device once: a kernel of known "
                         "HBM traffic for scaling FETCH_SIZE / WRITE_SIZE counter readings")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path shards over (batch, head) with no "
              "exchange, and this build runs on a single MI355X; use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.parts is None:
        parts = list(DEFAULT_PARTS) if (args.workload == "flux_joint" and args.sp == 1 and not args.abba
                                        and args.producer == "none") else []
    else:
        parts = [p for p in args.parts.split(",") if p and p != "none"]
    for p in parts:
        if p not in ("tiny", "flux_joint", "video_early", "long_t2v", "quant_long"):
            raise SystemExit(f"--parts: unknown workload {p!r}")

    import torch
    import synth
    import quantized_attention_video_smooth_amd as sage

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    sage.lib()
    if args.workload == "vmlp_proj":
        res = run_projection(args, torch, synth, sage)
        if args.copy_calibration:
            copy_calibration(torch, torch.device("cuda:0"))
        print(json.dumps(res), flush=True)
        return
    cfg = synth.config(args.workload)
    if args.sp > 1:
        if args.workload == "quant_long" or args.producer != "none":
            raise SystemExit("--sp times the attention share: use an attention workload, no --producer")
        print(json.dumps(run_sp_share(args, torch, synth, sage, cfg)), flush=True)
        return
    if args.abba:
        print(json.dumps(run_abba(args, cfg, torch, synth, sage)), flush=True)
        return

    main_res = measure_path(args, cfg, torch, synth, sage, args.streams)
    step = main_res.pop("_step")
    res = {
        "metric": METRIC,
        "value": main_res.pop("value"),
        "unit": main_res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 QK / fp8-e4m3 PV, fp32 softmax+accum",
        "data": "synthetic (seeded counter-based normals, bf16 NHD)",
    }
    res.update(main_res)
    if args.gpu_state_seconds > 0:
        res["gpu_state"] = gpu_state_during(step, torch, args.gpu_state_seconds)
    del step
    if parts:
        res["parts"] = {}
        for p in parts:
            pcfg = synth.config(p)
            pres = measure_path(args, pcfg, torch, synth, sage, 1 if p == "quant_long" else args.streams)
            pres.pop("_step")
            pres["steps"], pres["warmup"] = args.steps, args.warmup
            res["parts"][p] = pres
            torch.cuda.empty_cache()
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(cfg, args.seed)
    if args.copy_calibration:
        copy_calibration(torch, torch.device("cuda:0"))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
