"""Benchmark: paged relative-bias attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-extra] [--no-cpu]

A step is one rpa_attn_varlen call (attention kernel + split combine) over
one batch.  The headline workload is the batched decode batch (32 requests
with 1024..8192 cached tokens, 32 q heads / 8 kv heads, head_dim 128, block
size 16, rel_extent 128, planner-chosen splits); `value` is its algorithmic
KV-and-operand bytes per second.  The same JSON line also carries, each with
its roofline block (and HBM traffic from the committed rocprofv3 summaries
while the kernel source matches them): the chunked-prefill batch (TFLOP/s
against the bf16 MFMA peak), the 1M-token decode (planner and 16..128
splits), the continuous-batching mix, the E4M3-cache, ALiBi and bf16
rel_logits variants, the paged KV write, the headline decode as a HIP graph,
the measured HBM streaming-read ceiling, and the CPU oracle timed on bounded
samples (--no-cpu skips it).  Inputs are resident in HBM before timing; KV
pools are rotated over three copies so that the 256 MB last-level cache
cannot serve repeated steps.  The extra workloads are timed after about 0.3 s
of untimed calls, once the shader clock has settled (from idle it takes some
50 ms of prefill work to ramp up, and a prefill step timed during the ramp
reads up to 20 % slow); the headline runs exactly the --warmup steps before
its timed steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode KV GB/s (% of HBM peak) and prefill TFLOP/s (% of bf16 MFMA peak)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
SETTLE_S = 0.3  # untimed calls before timing the extra workloads
KERNEL_SOURCES = ["relative_bias_amd/csrc/rpa_kernels.hip", "relative_bias_amd/csrc/rpa_internal.h"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(workload: str):
    """HBM traffic per launch from committed rocprofv3 --pmc summaries, if they
    were taken on the current kernel source (else None)."""
    hits = [f for f in os.listdir(os.path.join(ROOT, "profiles")) if f.endswith(f"_{workload}_traffic.json")
            and f[: -len(f"_{workload}_traffic.json")].endswith("_kernel")]
    if len(hits) != 1:
        return None
    path = os.path.join(ROOT, "profiles", hits[0])
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def load_mfma(workload: str):
    """MFMA busy fraction and executed/algorithmic flop ratio from the
    committed rocprofv3 counter summary of a prefill workload, if taken on
    the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", f"attn_kernel_{workload}_mfma.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash():
        return None
    return {"mfma_busy_fraction": t["mfma_busy_fraction"], "executed_over_algorithmic": t["executed_over_algorithmic"]}


def time_calls(fn, steps, warmup, stream):
    import torch
    for _ in range(warmup):
        fn(0)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    stop = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for i in range(steps):
        fn(i)
    stop.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps  # ms


class Runner:
    """Holds device buffers for one workload and times rpa_attn_varlen on it."""

    def __init__(self, w, num_splits, pools=1):
        import torch
        from relative_bias_amd import binding as bnd
        self.bnd = bnd
        self.w = w
        self.S = int(num_splits)
        T, H, D = w.q.shape
        dev = w.q.device
        self.out = torch.empty((T, H, D), dtype=torch.bfloat16, device=dev)
        self.lse = torch.empty((T, H), dtype=torch.float32, device=dev)
        nb = bnd.rpa_workspace_bytes(self.S, T, H, D)
        self.ws = torch.empty((max(nb, 1),), dtype=torch.uint8, device=dev)
        self.kv = [(w.key_cache, w.value_cache)]
        for _ in range(pools - 1):
            self.kv.append((w.key_cache.clone(), w.value_cache.clone()))

    alibi = None  # fp32 [H] ALiBi slopes on the device, or None

    def call(self, i=0):
        w = self.w
        k, v = self.kv[i % len(self.kv)]
        self.bnd.rpa_attn_varlen(
            w.q, k, v, block_table=w.block_table, cache_seqlens=w.cache_seqlens,
            cu_seqlens_q=w.cu_seqlens_q, max_seqlen_q=w.max_seqlen_q, softmax_scale=w.softmax_scale,
            causal=w.causal, window_size=w.window_size, rel_extent=w.rel_extent,
            rel_logits=w.rel_logits, num_splits=self.S, out=self.out, lse=self.lse, workspace=self.ws,
            alibi_slopes=self.alibi)

    def combine_only(self, i=0):
        """The split combine alone, on partial buffers of this call's shape."""
        if not hasattr(self, "_po"):
            import torch
            T, H, D = self.w.q.shape
            g = torch.Generator(device=self.w.q.device).manual_seed(1)
            self._po = torch.randn((self.S, T, H, D), generator=g, device=self.w.q.device)
            self._pl = torch.randn((self.S, T, H), generator=g, device=self.w.q.device)
        self.bnd.rpa_split_combine(self._po, self._pl, out=self.out, lse=self.lse)


class Fp8Runner(Runner):
    """Times rpa_attn_varlen_fp8 on a workload whose K/V are held as E4M3
    codes of the bf16 caches divided by the scales (the codes a
    quantise-at-store write of the same rows would hold)."""

    K_SCALE, V_SCALE = 1.0 / 32, 1.0 / 16

    def __init__(self, w, num_splits, pools=1):
        import torch
        super().__init__(w, num_splits, pools=1)
        kv = []
        for i in range(pools):
            k = w.key_cache if i == 0 else w.key_cache.clone()
            v = w.value_cache if i == 0 else w.value_cache.clone()
            kv.append(((k.float() / self.K_SCALE).to(torch.float8_e4m3fn).view(torch.uint8),
                       (v.float() / self.V_SCALE).to(torch.float8_e4m3fn).view(torch.uint8)))
            del k, v
        self.kv = kv
        torch.cuda.empty_cache()

    def call(self, i=0):
        w = self.w
        k, v = self.kv[i % len(self.kv)]
        self.bnd.rpa_attn_varlen_fp8(
            w.q, k, v, k_scale=self.K_SCALE, v_scale=self.V_SCALE, block_table=w.block_table,
            cache_seqlens=w.cache_seqlens, cu_seqlens_q=w.cu_seqlens_q, max_seqlen_q=w.max_seqlen_q,
            softmax_scale=w.softmax_scale, causal=w.causal, window_size=w.window_size,
            rel_extent=w.rel_extent, rel_logits=w.rel_logits, num_splits=self.S, out=self.out, lse=self.lse,
            workspace=self.ws)


def settle(fn, seconds):
    """Untimed calls for about `seconds` of wall time (clock ramp-up)."""
    import torch
    t_end = time.perf_counter() + seconds
    i = 0
    while time.perf_counter() < t_end:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def measure(runner, steps, warmup, settle_s=0.0):
    import torch
    from relative_bias_amd import metrics
    stream = torch.cuda.current_stream()
    if settle_s > 0:
        settle(runner.call, settle_s)
    ms = time_calls(runner.call, steps, warmup, stream)
    ms_comb = 0.0
    if runner.S > 1:
        ms_comb = time_calls(runner.combine_only, steps, warmup, stream)
    wk = metrics.work(runner.w, kv_elem_bytes=1 if isinstance(runner, Fp8Runner) else 2)
    return ms, ms_comb, wk


def measure_graph(runner, steps, warmup):
    """The same step captured once per KV pool in a HIP graph and replayed:
    device time per step (back-to-back replays) and host latency of one
    step (launch or replay, then synchronize), median of 50, against the
    eager call's."""
    import statistics
    import torch
    graphs = []
    for i in range(len(runner.kv)):
        runner.call(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            runner.call(i)
        graphs.append(g)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ms = time_calls(lambda i: graphs[i % len(graphs)].replay(), steps, warmup, stream)
    lat_e, lat_g = [], []
    for i in range(50):
        t0 = time.perf_counter()
        runner.call(i)
        torch.cuda.synchronize()
        lat_e.append(time.perf_counter() - t0)
        t0 = time.perf_counter()
        graphs[i % len(graphs)].replay()
        torch.cuda.synchronize()
        lat_g.append(time.perf_counter() - t0)
    del graphs
    return ms, statistics.median(lat_e) * 1e6, statistics.median(lat_g) * 1e6


def measure_kv_write(steps, warmup):
    """The paged KV write of the chunked-prefill batch's 8173 new tokens (8 kv
    heads, head_dim 128): rpa_slot_mapping then rpa_kv_cache_write, timed
    together.  Algorithmic bytes: the K and V rows read and written, the
    slots written and read, and the metadata the slot kernel reads."""
    import torch
    from relative_bias_amd import binding as bnd
    from relative_bias_amd import workloads as wl
    w = wl.chunked_prefill(device="cpu").to("cuda")
    T, Hkv, D = w.num_tokens, w.num_kv_heads, w.head_dim
    g = torch.Generator(device="cuda").manual_seed(3)
    key = torch.randn((T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    val = torch.randn((T, Hkv, D), generator=g, device="cuda").to(torch.bfloat16)
    slots = torch.empty((T,), dtype=torch.int64, device="cuda")

    def step(i=0):
        bnd.rpa_slot_mapping(w.block_table, w.cache_seqlens, w.cu_seqlens_q, w.block_size, out=slots)
        bnd.rpa_kv_cache_write(key, val, slots, w.key_cache, w.value_cache)

    settle(step, SETTLE_S)
    ms = time_calls(step, steps, warmup, torch.cuda.current_stream())
    row = Hkv * D * 2
    nbytes = 2 * T * row * 2 + T * 8 * 2 + T * 4 + (2 * w.batch + 1) * 4
    info = {"workload": "kv_write (chunked_prefill tokens)", "num_tokens": T, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": w.block_size, "alg_bytes": nbytes}
    del w, key, val, slots
    torch.cuda.empty_cache()
    return ms, dict(info, bytes=nbytes)


def hbm_read_ceiling(gib=4, reps=10):
    """Streaming-read rate of the device: one pass of 16-byte nontemporal
    loads over a `gib` GiB buffer (larger than the 256 MB last-level cache),
    one contiguous chunk per workgroup, by libhbmprobe.so's kernel, best and
    median of `reps` passes."""
    import ctypes
    import statistics
    import torch
    from relative_bias_amd import build as bld
    if not os.path.exists(bld.PROBE_LIB):
        raise RuntimeError(f"{bld.PROBE_LIB} is missing: build it with `python -m relative_bias_amd.build`")
    L = ctypes.CDLL(bld.PROBE_LIB)
    L.hbm_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p]
    L.hbm_stream_read.restype = ctypes.c_int
    nbytes = gib << 30
    buf = torch.ones((nbytes // 2,), dtype=torch.bfloat16, device="cuda")
    blocks = 256 * 8
    sink = torch.empty((blocks,), dtype=torch.int32, device="cuda")
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    times = []
    for i in range(reps + 2):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        rc = L.hbm_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()), blocks, st)
        e1.record()
        torch.cuda.synchronize()
        if rc != 0:
            raise RuntimeError(f"hbm_stream_read failed: {rc}")
        if i >= 2:
            times.append(e0.elapsed_time(e1))
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": "stream_read_kernel (libhbmprobe.so)", "bytes": nbytes,
            "best_gbs": round(nbytes / min(times) / 1e6, 1), "median_gbs": round(nbytes / statistics.median(times) / 1e6, 1)}


def cpu_baseline_one_thread(w, budget_s=4.0):
    """The same oracle on one host thread (a shorter sample), for the
    per-core rate."""
    import torch
    n = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        r = cpu_baseline(w, budget_s)
    finally:
        torch.set_num_threads(n)
    return r


def cpu_baseline(w, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the decode batch: whole requests
    in order, passing over the batch again until about budget_s of CPU time
    has been spent, in GB/s of the same algorithmic bytes."""
    import torch
    from oracle import attention as orc
    from relative_bias_amd import metrics
    wc = w.to("cpu")
    cu = wc.cu_seqlens_q.tolist()
    done_bytes, spent, nreq = 0, 0.0, 0
    while spent < budget_s:
        for b in range(wc.batch):
            toks = list(range(cu[b], cu[b + 1]))
            t0 = time.perf_counter()
            orc.attention(wc.q, wc.key_cache, wc.value_cache, wc.block_table, wc.cache_seqlens,
                          wc.cu_seqlens_q, wc.softmax_scale, wc.causal, wc.window_size, wc.rel_extent,
                          wc.rel_logits, tokens=toks)
            spent += time.perf_counter() - t0
            sub = type("W", (), {})()
            for k in ("num_heads", "num_kv_heads", "head_dim", "block_size", "rel_extent", "window_size",
                      "causal"):
                setattr(sub, k, getattr(wc, k))
            sub.q_lens, sub.k_lens = [wc.q_lens[b]], [wc.k_lens[b]]
            done_bytes += metrics.work(sub)["bytes"]
            nreq += 1
            if spent >= budget_s:
                break
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{nreq} request evaluations ({nreq / wc.batch:.1f} passes over the {wc.batch} requests) "
                      f"of the batched decode batch, all {wc.num_heads} heads, {spent:.1f} s of fp64 CPU work"}


def host_cpu():
    """Model name and thread counts of the host the oracle runs on."""
    import torch
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"model": model, "logical_cpus": os.cpu_count(), "torch_threads": torch.get_num_threads()}


def _rows_flops(w, b, local, heads):
    """4 * D * (visible (row, key) pairs) over the given rows of request b and heads."""
    from relative_bias_amd import metrics
    lq, lk = w.q_lens[b], w.k_lens[b]
    pairs = 0
    for i in local:
        lo, hi = metrics._row_bounds(i + lk - lq, lk, w.causal, *w.window_size)
        pairs += max(hi - lo + 1, 0)
    return 4 * w.head_dim * len(heads) * pairs


def cpu_baseline_rows(w, rows_per_request, budget_s, what):
    """The fp64 oracle on a bounded sample of a prefill-type workload: the
    last `rows_per_request` query rows of each request (all heads), request
    after request until about budget_s of CPU time, in GFLOP/s of the same
    algorithmic flops (4 * D * visible pairs * heads)."""
    import torch
    from oracle import attention as orc
    wc = w if w.q.device.type == "cpu" else w.to("cpu")
    cu = wc.cu_seqlens_q.tolist()
    heads = list(range(wc.num_heads))
    flops, spent, nrows, nreq = 0, 0.0, 0, 0
    while spent < budget_s:
        for b in range(wc.batch):
            lq = wc.q_lens[b]
            local = list(range(max(lq - rows_per_request, 0), lq))
            if not local:
                continue
            toks = [cu[b] + i for i in local]
            t0 = time.perf_counter()
            orc.attention(wc.q, wc.key_cache, wc.value_cache, wc.block_table, wc.cache_seqlens, wc.cu_seqlens_q,
                          wc.softmax_scale, wc.causal, wc.window_size, wc.rel_extent, wc.rel_logits, tokens=toks)
            spent += time.perf_counter() - t0
            flops += _rows_flops(wc, b, local, heads)
            nrows += len(local)
            nreq += 1
            if spent >= budget_s:
                break
    return {"value": round(flops / spent / 1e9, 3), "unit": "GFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{what}: the last {rows_per_request} query rows of each request, all {wc.num_heads} heads; "
                      f"{nreq} request evaluations, {nrows} rows, {flops / 1e9:.1f} GFLOP in {spent:.1f} s of "
                      f"fp64 CPU work"}


def cpu_baseline_whole(w, budget_s, what):
    """The fp64 oracle on a whole small workload, repeated for about budget_s,
    in GB/s of the same algorithmic bytes."""
    import torch
    from oracle import attention as orc
    from relative_bias_amd import metrics
    wc = w if w.q.device.type == "cpu" else w.to("cpu")
    nbytes = metrics.work(wc)["bytes"]
    passes, spent = 0, 0.0
    while spent < budget_s:
        t0 = time.perf_counter()
        orc.attention(wc.q, wc.key_cache, wc.value_cache, wc.block_table, wc.cache_seqlens, wc.cu_seqlens_q,
                      wc.softmax_scale, wc.causal, wc.window_size, wc.rel_extent, wc.rel_logits)
        spent += time.perf_counter() - t0
        passes += 1
    return {"value": round(passes * nbytes / spent / 1e9, 4), "unit": "GB/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{what}: {passes} passes over the whole workload in {spent:.1f} s of fp64 CPU work"}


def cpu_baseline_heads(w, budget_s, what):
    """The fp64 oracle on the q heads of one kv head at a time (kv head 0,
    then 1, ...) of a decode workload, until about budget_s of CPU time, in
    GB/s of those heads' algorithmic bytes (their kv head's K and V, their
    q, out, lse and rel_logits rows, the block table)."""
    import torch
    from oracle import attention as orc
    from relative_bias_amd import metrics
    wc = w if w.q.device.type == "cpu" else w.to("cpu")
    G = wc.num_heads // wc.num_kv_heads
    sub = type("W", (), {})()
    for k in ("q_lens", "k_lens", "head_dim", "block_size", "rel_extent", "window_size", "causal"):
        setattr(sub, k, getattr(wc, k))
    sub.num_heads, sub.num_kv_heads = G, 1
    slice_bytes = metrics.work(sub)["bytes"]
    done, spent, g = 0, 0.0, 0
    while spent < budget_s and g < wc.num_kv_heads:
        t0 = time.perf_counter()
        orc.attention(wc.q, wc.key_cache, wc.value_cache, wc.block_table, wc.cache_seqlens, wc.cu_seqlens_q,
                      wc.softmax_scale, wc.causal, wc.window_size, wc.rel_extent, wc.rel_logits,
                      heads=range(g * G, (g + 1) * G))
        spent += time.perf_counter() - t0
        done += slice_bytes
        g += 1
    return {"value": round(done / spent / 1e9, 4), "unit": "GB/s", "cores": torch.get_num_threads(),
            "kind": "oracle",
            "sample": f"{what}: {g} of {wc.num_kv_heads} kv heads (each with its {G} q heads), "
                      f"{done / 1e9:.2f} GB of algorithmic bytes in {spent:.1f} s of fp64 CPU work"}


def roofline_of(name, w, ms, wk, kv_elem_bytes=2):
    """Roofline block of one workload: its bound (the larger of its HBM time
    at 8 TB/s and its MFMA time at 2.5 PFLOP/s), the achieved rate over the
    whole timed step and its fraction of the peak, and the HBM traffic from
    committed counter summaries of the current kernel source (else None)."""
    t_hbm = wk["bytes"] / (HBM_PEAK_GBS * 1e6)          # ms
    t_mfma = wk["flops"] / (MFMA_BF16_PEAK_TFLOPS * 1e9)  # ms
    if t_mfma >= t_hbm:
        achieved = wk["flops"] / ms / 1e9
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
    else:
        achieved = wk["bytes"] / ms / 1e6
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["roofline_ms"] = round(max(t_hbm, t_mfma), 5)
    roof["bound_over_measured"] = round(max(t_hbm, t_mfma) / ms, 4)
    roof["kernel_ms"] = round(ms, 5)
    roof["alg_bytes_per_launch"] = wk["bytes"]
    roof["alg_flops_per_launch"] = wk["flops"]
    roof["traffic"] = load_traffic(name)
    if roof["traffic"]:
        roof["traffic_over_alg_bytes"] = round(roof["traffic"] / wk["bytes"], 4)
    return roof


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-extra", action="store_true", help="only the headline decode batch")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", default=None, help="run one workload: batched_decode, chunked_prefill, "
                                                  "long_decode, continuous_batch, batched_decode_fp8, "
                                                  "chunked_prefill_fp8, long_decode_fp8, batched_decode_alibi, "
                                                  "chunked_prefill_alibi, chunked_prefill_relbf16, kv_write")
    ap.add_argument("--splits", type=int, default=None,
                    help="override the planner's num_splits (0 = balanced decode) for the headline decode batch "
                         "(or for long_decode with --only long_decode)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 10 times (for scaling the "
                         "FETCH_SIZE / WRITE_SIZE counters) and exit")
    a = ap.parse_args(argv)
    if a.copy_calibration:
        import torch
        src = torch.ones((1 << 29,), dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": src.numel() * 2, "copy_bytes_written": dst.numel() * 2,
                          "launches": 10}))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(see the sharding notes in the design document); run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    from relative_bias_amd import binding as bnd
    from relative_bias_amd import workloads as wl
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    bnd.lib()
    torch.manual_seed(0)
    dev = "cuda"
    results = {}
    kv_summary = None
    graph_summary = None
    split_sweep = {}
    cpu_extra = {}
    want_cpu = not a.no_cpu and a.only is None and not a.no_extra

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    # Headline: batched decode.
    run_main = a.only in (None, "batched_decode")
    if run_main:
        w = wl.batched_decode(device="cpu").to(dev)
        S = bnd.rpa_choose_splits(w.batch, 1, w.num_heads, w.num_kv_heads, max(w.k_lens))
        if a.splits is not None:
            S = a.splits
        r = Runner(w, S, pools=3)
        ms, ms_c, wk = measure(r, a.steps, a.warmup)
        results["batched_decode"] = (w, S, ms, ms_c, wk)
        log(f"batched_decode S={S}: {ms * 1e3:.1f} us/step (combine {ms_c * 1e3:.1f} us), "
            f"{wk['bytes'] / ms / 1e6:.1f} GB/s")
        if not a.no_extra and a.only is None:
            try:
                gms, lat_e, lat_g = measure_graph(r, a.steps, a.warmup)
                graph_summary = {"workload": "batched_decode, one HIP graph per KV pool",
                                 "ms_per_step": round(gms, 5), "eager_ms_per_step": round(ms, 5),
                                 "host_latency_us_eager": round(lat_e, 1),
                                 "host_latency_us_graph": round(lat_g, 1)}
                log(f"batched_decode graph replay: {gms * 1e3:.1f} us/step; one-step latency "
                    f"eager {lat_e:.1f} us, graph {lat_g:.1f} us")
            except Exception as e:  # reported in the line; never hides the headline
                log(f"graph replay failed: {e!r}")
                graph_summary = {"workload": "batched_decode graph", "error": repr(e)}
        del r
    if not a.no_extra or a.only:
        if a.only in (None, "chunked_prefill"):
            w3 = wl.chunked_prefill(device="cpu").to(dev)
            r3 = Runner(w3, 1, pools=3)
            ms, ms_c, wk = measure(r3, max(5, a.steps // 2), a.warmup, SETTLE_S)
            results["chunked_prefill"] = (w3, 1, ms, ms_c, wk)
            log(f"chunked_prefill: {ms * 1e3:.1f} us/step, {wk['flops'] / ms / 1e9:.1f} TFLOP/s")
            if want_cpu:
                cpu_extra["chunked_prefill"] = cpu_baseline_rows(w3, 8, 8.0, "chunked prefill batch")
                log(f"  oracle: {cpu_extra['chunked_prefill']['value']} GFLOP/s")
            del r3, w3
        if a.only in (None, "long_decode"):
            w4 = wl.long_decode(device=dev)
            S4 = bnd.rpa_choose_splits(1, 1, w4.num_heads, w4.num_kv_heads, max(w4.k_lens))
            if a.splits is not None and a.only == "long_decode":
                S4 = a.splits
            r4 = Runner(w4, S4)
            ms, ms_c, wk = measure(r4, max(5, a.steps // 2), a.warmup, SETTLE_S)
            results["long_decode"] = (w4, S4, ms, ms_c, wk)
            log(f"long_decode S={S4}: {ms * 1e3:.1f} us/step, {wk['bytes'] / ms / 1e6:.1f} GB/s")
            del r4
            if a.only is None:
                # The split counts the walkthrough's planner caps at for this
                # range (16 to 128 partitions), beside the planner's choice.
                for Sx in (16, 32, 64, 128):
                    rx = Runner(w4, Sx)
                    msx, msx_c, wkx = measure(rx, max(5, a.steps // 2), a.warmup, 0.05)
                    split_sweep[str(Sx)] = {"num_splits": Sx, "ms_per_step": round(msx, 5),
                                            "combine_ms": round(msx_c, 5),
                                            "gbs": round(wkx["bytes"] / msx / 1e6, 2),
                                            "hbm_frac": round(wkx["bytes"] / msx / 1e6 / HBM_PEAK_GBS, 4)}
                    log(f"long_decode S={Sx}: {msx * 1e3:.1f} us/step (combine {msx_c * 1e3:.1f} us), "
                        f"{wkx['bytes'] / msx / 1e6:.1f} GB/s")
                    del rx
            if want_cpu:
                cpu_extra["long_decode"] = cpu_baseline_heads(w4, 8.0, "1M-token decode")
                log(f"  oracle: {cpu_extra['long_decode']['value']} GB/s")
            del w4
            torch.cuda.empty_cache()
        if a.only in (None, "continuous_batch"):
            w5 = wl.continuous_batch(device=dev)
            r5 = Runner(w5, 1, pools=3)
            ms, ms_c, wk = measure(r5, max(5, a.steps // 2), a.warmup, SETTLE_S)
            results["continuous_batch"] = (w5, 1, ms, ms_c, wk)
            log(f"continuous_batch: {ms * 1e3:.1f} us/step, {wk['bytes'] / ms / 1e6:.1f} GB/s, "
                f"{wk['flops'] / ms / 1e9:.1f} TFLOP/s")
            del r5
            if want_cpu:
                cpu_extra["continuous_batch"] = cpu_baseline_rows(w5, 8, 8.0, "continuous-batching mix")
                log(f"  oracle: {cpu_extra['continuous_batch']['value']} GFLOP/s")
            del w5
            torch.cuda.empty_cache()
        if a.only in (None, "batched_decode_fp8"):
            w6 = wl.batched_decode(device="cpu").to(dev)
            r6 = Fp8Runner(w6, 0, pools=3)
            ms, ms_c, wk = measure(r6, a.steps, a.warmup, SETTLE_S)
            results["batched_decode_fp8"] = (w6, 0, ms, ms_c, wk)
            log(f"batched_decode_fp8: {ms * 1e3:.1f} us/step, {wk['bytes'] / ms / 1e6:.1f} GB/s")
            del r6, w6
            torch.cuda.empty_cache()
        if a.only in (None, "chunked_prefill_fp8"):
            w8 = wl.chunked_prefill(device="cpu").to(dev)
            r8 = Fp8Runner(w8, 1, pools=3)
            ms, ms_c, wk = measure(r8, max(5, a.steps // 2), a.warmup, SETTLE_S)
            results["chunked_prefill_fp8"] = (w8, 1, ms, ms_c, wk)
            log(f"chunked_prefill_fp8: {ms * 1e3:.1f} us/step, {wk['flops'] / ms / 1e9:.1f} TFLOP/s")
            del r8, w8
            torch.cuda.empty_cache()
        if a.only in (None, "long_decode_fp8"):
            w7 = wl.long_decode(device=dev)
            r7 = Fp8Runner(w7, 0)
            w7.key_cache = w7.value_cache = None  # the bf16 caches are not needed any more
            torch.cuda.empty_cache()
            ms, ms_c, wk = measure(r7, max(5, a.steps // 2), a.warmup, SETTLE_S)
            results["long_decode_fp8"] = (w7, 0, ms, ms_c, wk)
            log(f"long_decode_fp8: {ms * 1e3:.1f} us/step, {wk['bytes'] / ms / 1e6:.1f} GB/s")
            del r7, w7
            torch.cuda.empty_cache()
        for name, make, S_a in (("batched_decode_alibi", wl.batched_decode, 0),
                                ("chunked_prefill_alibi", wl.chunked_prefill, 1),
                                ("chunked_prefill_relbf16", wl.chunked_prefill, 1)):
            if a.only not in (None, name):
                continue
            wa = make(device="cpu").to(dev)
            ra = Runner(wa, S_a, pools=3)
            H = wa.num_heads
            if name.endswith("_alibi"):
                ra.alibi = torch.tensor([2.0 ** (-8.0 * (i + 1) / H) for i in range(H)], dtype=torch.float32,
                                        device=dev)
            else:
                wa.rel_logits = wa.rel_logits.to(torch.bfloat16)
            ms, ms_c, wk = measure(ra, max(5, a.steps // 2), a.warmup, SETTLE_S)
            results[name] = (wa, S_a, ms, ms_c, wk)
            log(f"{name}: {ms * 1e3:.1f} us/step, {wk['bytes'] / ms / 1e6:.1f} GB/s, "
                f"{wk['flops'] / ms / 1e9:.1f} TFLOP/s")
            del ra, wa
            torch.cuda.empty_cache()
        if a.only in (None, "kv_write"):
            try:
                ms_kv, kvinfo = measure_kv_write(max(5, a.steps // 2), a.warmup)
                log(f"kv_write: {ms_kv * 1e3:.1f} us/step, {kvinfo['bytes'] / ms_kv / 1e6:.1f} GB/s")
                kv_summary = dict(kvinfo, ms_per_step=round(ms_kv, 5),
                                  gbs=round(kvinfo["bytes"] / ms_kv / 1e6, 2),
                                  hbm_frac=round(kvinfo["bytes"] / ms_kv / 1e6 / HBM_PEAK_GBS, 4))
            except Exception as e:  # reported in the line; never hides the headline
                log(f"kv_write failed: {e!r}")
                kv_summary = {"workload": "kv_write (chunked_prefill tokens)", "error": repr(e)}

    def summary(name):
        w, S, ms, ms_c, wk = results[name]
        extra = {}
        if name.endswith("_alibi"):
            extra = {"alibi_slopes": "2^(-8 (h + 1) / H)"}
        if name.endswith("_relbf16"):
            extra = {"rel_logits": "bf16"}
        if name.endswith("_fp8"):
            kern = ("attn_kernel<128, false, true>" if S == 1 else
                    "decode_heads_kernel<128, true, true> + combine_heads_kernel<128>")
            extra = {"kv_cache": "e4m3", "k_scale": Fp8Runner.K_SCALE, "v_scale": Fp8Runner.V_SCALE,
                     "kernel": kern}
        return {**extra, "workload": name, "batch": w.batch, "num_tokens": w.num_tokens, "num_heads": w.num_heads,
                "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                "rel_extent": w.rel_extent, "window": list(w.window_size), "num_splits": S,
                "ms_per_step": round(ms, 5), "combine_ms": round(ms_c, 5),
                "gbs": round(wk["bytes"] / ms / 1e6, 2), "tflops": round(wk["flops"] / ms / 1e9, 2),
                "hbm_frac": round(wk["bytes"] / ms / 1e6 / HBM_PEAK_GBS, 4),
                "mfma_frac": round(wk["flops"] / ms / 1e9 / MFMA_BF16_PEAK_TFLOPS, 4),
                "alg_bytes": wk["bytes"], "alg_flops": wk["flops"],
                "roofline": roofline_of(name, w, ms, wk),
                **({"mfma_counters": load_mfma(name)} if load_mfma(name) else {}),
                **({"cpu_baseline": cpu_extra[name]} if name in cpu_extra else {}),
                **({"split_sweep": split_sweep} if name == "long_decode" and split_sweep else {})}

    if a.only == "kv_write":
        print(json.dumps({"kv_write": kv_summary, "kernel_hash": kernel_hash()}))
        return 0
    head = a.only if a.only else "batched_decode"
    w, S, ms, ms_c, wk = results[head]
    kernel_ms = ms - ms_c
    prefill_like = head.startswith("chunked_prefill")
    if prefill_like:
        achieved = wk["flops"] / kernel_ms / 1e9
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_BF16_PEAK_TFLOPS, 4)}
        value, unit = wk["flops"] / ms / 1e9, "TFLOP/s"
    else:
        achieved = wk["bytes"] / kernel_ms / 1e6
        roof = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
        value, unit = wk["bytes"] / ms / 1e6, "GB/s"
    if S == 0:
        # Balanced decode: the attention kernel and the combine of the
        # requests cut between workgroups; kernel_ms is the whole step (both
        # kernels).  Eight kv heads take the form with one kv head per wave.
        if head.endswith("_fp8"):
            roof["kernel"] = "decode_heads_kernel<128, true, true> + combine_heads_kernel<128>"
        elif w.num_kv_heads == 8:
            roof["kernel"] = "decode_heads_kernel<128> + combine_heads_kernel<128>"
        else:
            roof["kernel"] = "decode_balanced_kernel<128> + combine_balanced_kernel<128>"
    else:
        roof["kernel"] = "attn_kernel<128, false, true>" if head.endswith("_fp8") else "attn_kernel<128>"
    roof["kernel_ms"] = round(kernel_ms, 5)
    roof["alg_bytes_per_launch"] = wk["bytes"]
    roof["traffic"] = load_traffic(head)
    line = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": summary(head), "roofline": roof,
    }
    for name in results:
        if name != head:
            line[name] = summary(name)
    if kv_summary is not None:
        line["kv_write"] = kv_summary
    if graph_summary is not None:
        line["batched_decode_graph"] = graph_summary
    if not a.no_extra and a.only is None:
        try:
            hc = hbm_read_ceiling()
            hc["decode_frac_of_ceiling"] = round(roof["achieved"] / hc["best_gbs"], 4) if not prefill_like else None
            line["hbm_read_ceiling"] = hc
            log(f"HBM streaming-read ceiling: best {hc['best_gbs']} GB/s, median {hc['median_gbs']} GB/s")
        except Exception as e:  # reported in the line; never hides the headline
            line["hbm_read_ceiling"] = {"error": repr(e)}
    if not a.no_cpu and head == "batched_decode":
        log("timing the CPU oracle on a sample ...")
        line["cpu_baseline"] = cpu_baseline(w)
        line["cpu_baseline"]["host_cpu"] = host_cpu()
        line["cpu_baseline_one_thread"] = cpu_baseline_one_thread(w)
        if want_cpu:
            line["tiny_mixed_cpu_baseline"] = cpu_baseline_whole(wl.tiny(), 3.0, "tiny mixed batch")
    line["kernel_hash"] = kernel_hash()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
