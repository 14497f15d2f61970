#!/usr/bin/env python3
"""Benchmark: one decode step = the append of each sequence's new token + paged
decode attention, on one MI355X.

The step is one pkv_decode_step call (the append runs inside the partition
kernel, then the merge kernel); `--step two-call` times kv_append followed by
pkv_paged_decode_attention instead (three launches, bit-identical results).
Both are timed and reported; `value` is the one `--step` selects.

Default workload: the Llama-3-8B-shaped layer (B=64, Hq=32, Hkv=8, D=128,
block 16, context lengths uniform in [512, 4096], bf16 KV).  Prints ONE JSON
line.  `value` is KV bytes read per step (sum over sequences of
L * 2 * Hkv * D * bytes per element) divided by the measured step time.

Inputs are resident in HBM before timing starts.  R copies of the KV cache
(same contents, different addresses) are cycled so that no step finds the
previous step's pages in the 256 MB memory-side cache.  The K timed steps
run with nothing else in the stream; the same K steps are then run again
with a HIP event pair around every partition launch (recorded on the stream
the kernel runs on), whose mean gives the roofline entry.  The oracle timed
on the host cores gives the CPU baseline.

The default run also times every other configuration's step (fewer
steps each) for `detail.configs`, and a streaming read of a 2 GiB buffer
(pkv_read_probe) for the device's read ceiling.

  python bench.py [--steps K] [--warmup W] [--config NAME] [--step fused|two-call] [--no-cpu]
                  [--no-configs] [--only-step]
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

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, 8 TB/s
ARITHMETIC = ("bf16 q and KV (fp8 / int8 codes widened exactly to bf16) as MFMA operands, "
              "softmax weights as two bf16 terms (to 2^-16), fp32 accumulation and softmax, "
              "bf16 output")
ARITHMETIC_VALU = "bf16 q and KV widened to fp32, fp32 FMA, fp32 softmax, bf16 output"


def visible_keys(wl):
    """Per sequence, the keys some query sees: every position without a
    window; otherwise the first `sinks` plus those from L - q_len - window + 1
    on.  And the blocks those keys sit in."""
    L = wl.lengths.astype(np.int64)
    BS = wl.BS
    if wl.window <= 0:
        return L, (L + BS - 1) // BS
    ql = wl.q_lens.astype(np.int64)
    lo = np.maximum(L - ql - wl.window + 1, 0)
    keys = np.where(wl.sinks >= lo, L, np.minimum(wl.sinks, L) + (L - lo))
    pe = (L + BS - 1) // BS
    ps = np.minimum((wl.sinks + BS - 1) // BS, pe)
    pw = lo // BS
    pages = np.where(pw <= ps, pe, ps + (pe - pw))
    return keys, pages


def kv_bytes(wl) -> int:
    """Algorithmic KV bytes of one step: K and V of every key some query sees
    (and the per-block scales of a quantised cache)."""
    elem = 2 if wl.kv_dtype == "bf16" else 1
    keys, pages = visible_keys(wl)
    tot = int(keys.sum()) * 2 * wl.Hkv * wl.D * elem
    if wl.kv_dtype != "bf16":
        tot += int(pages.sum()) * wl.Hkv * 2 * 4
    return tot


PARTITION_SOURCES = ["decode_mfma.hip", "decode_valu.hip", "decode_common.hpp", "pkv_device.hpp",
                     "pkv_internal.hpp"]


def partition_source_hash() -> str:
    """sha256 over the sources the partition kernels are built from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_decode_06_amd", "csrc")
    for name in PARTITION_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(config: str, kernel: str):
    """HBM bytes per partition launch from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, scaled by a plain copy of known
    size), or None when there is none for this workload or the kernel
    sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            entries = json.load(f)
    except (OSError, ValueError):
        return None
    for ent in entries:
        if ent.get("config") == config and ent.get("kernel") == kernel:
            if ent.get("source_sha256") != partition_source_hash():
                return None
            return ent["traffic_bytes_per_launch"]
    return None


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_step_seconds(wl, nthreads: int, budget_s: float, max_runs: int):
    """Mean wall time of the oracle's attention over the whole batch (after
    its own append of the step's tokens, in position order), repeated until
    about `budget_s` of wall time has passed; (mean seconds, runs)."""
    import oracle
    from paged_kv_decode_06_amd import workloads as W

    k = W.cache_host(wl.k_cache).copy()
    v = W.cache_host(wl.v_cache).copy()
    ks = None if wl.k_scale is None else wl.k_scale.cpu().numpy().copy()
    vs = None if wl.v_scale is None else wl.v_scale.cpu().numpy().copy()
    pos = np.concatenate([np.arange(q) for q in wl.q_lens])
    for i in range(int(wl.q_lens.max())):
        slots = np.where(pos == i, wl.slot_mapping_np, -1).astype(np.int32)
        oracle.kv_append(W.bf16_bits(wl.k_new), W.bf16_bits(wl.v_new), slots, k, v, ks, vs)
    q = W.bf16_bits(wl.q)
    cl = wl.lengths.astype(np.int32)
    general = int(wl.q_lens.max()) > 1 or wl.window > 0
    times = []
    t_all = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if general:
            oracle.paged_attention(q, k, v, wl.block_tables_np, cl, wl.scale, q_start=wl.q_start_np,
                                   sinks=wl.sinks, window=wl.window, k_scale=ks, v_scale=vs,
                                   nthreads=nthreads)
        else:
            oracle.paged_decode_attention(q, k, v, wl.block_tables_np, cl, wl.scale, k_scale=ks,
                                          v_scale=vs, nthreads=nthreads)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_all > budget_s or len(times) >= max_runs:
            break
    return sum(times) / len(times), len(times)


def cpu_baseline(wl, budget_s=10.0, max_runs=100, single_thread=True):
    """The oracle, as it stands, on the host cores: one full step's attention
    over the same batch, repeated for about `budget_s` of wall time on every
    core the process may use; beside it the same oracle on one thread, for
    this batch and for the tiny configuration (one run or more each)."""
    from paged_kv_decode_06_amd import workloads as W

    try:
        threads = len(os.sched_getaffinity(0))
    except AttributeError:
        threads = os.cpu_count() or 1
    threads = min(threads, int(os.environ.get("OMP_NUM_THREADS", threads) or threads))
    t, runs = oracle_step_seconds(wl, threads, budget_s, max_runs)
    res = {"value": round(kv_bytes(wl) / t / 1e9, 4), "unit": "GB/s", "cores": threads,
           "kind": "oracle",
           "sample": f"full {wl.name} batch (B={wl.B}), fp64 attention of one step, "
                     f"{runs} run(s), mean {t:.3f} s per step",
           "cpu_model": cpu_model()}
    if single_thread:
        one = {}
        t1, r1 = oracle_step_seconds(wl, 1, 0.0, 1)
        one[wl.name] = {"s_per_step": round(t1, 4), "GB/s": round(kv_bytes(wl) / t1 / 1e9, 4),
                        "runs": r1}
        tiny = W.make_config_workload("tiny", device="cpu")
        tt, rt = oracle_step_seconds(tiny, 1, 1.0, 1000)
        one["tiny"] = {"s_per_step": round(tt, 7), "GB/s": round(kv_bytes(tiny) / tt / 1e9, 4),
                       "runs": rt}
        res["single_thread"] = one
    return res


class TimingEvents:
    """HIP events for timing only, created with hipEventDisableSystemFence so
    that recording one does not write back and invalidate the caches (HIP's
    own documentation of the flag: it makes timings between events more
    accurate).  Bound through ctypes to the HIP runtime already mapped in
    this process (the one torch and libpkv use), never a second copy."""

    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def lib(cls):
        if cls._lib is None:
            import ctypes
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64.so" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded in this process")
            L = ctypes.CDLL(path)
            vp = ctypes.c_void_p
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(vp), ctypes.c_uint]
            L.hipEventRecord.argtypes = [vp, vp]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
            L.hipEventDestroy.argtypes = [vp]
            for fn in (L.hipEventCreateWithFlags, L.hipEventRecord, L.hipEventElapsedTime,
                       L.hipEventDestroy):
                fn.restype = ctypes.c_int
            cls._lib = L
        return cls._lib

    def __init__(self, n: int):
        import ctypes
        L = self.lib()
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            if L.hipEventCreateWithFlags(ctypes.byref(e), self.DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def record(self, i: int, stream) -> None:
        import ctypes
        if self.lib().hipEventRecord(self.ev[i], ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        import ctypes
        ms = ctypes.c_float()
        if self.lib().hipEventElapsedTime(ctypes.byref(ms), self.ev[i], self.ev[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def close(self) -> None:
        for e in self.ev:
            self.lib().hipEventDestroy(e)
        self.ev = []


def settle(runs, seconds: float) -> int:
    """Keep the GPU busy with the workload's own steps for `seconds` of wall
    time before the warmup steps: clocks ramp under load, and a timed region
    started from idle read up to 3% slow for its first tens of milliseconds
    (the first of two step kinds timed back to back was the one to suffer).
    Returns the steps run; none of them is timed."""
    import torch
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(16):
            for run in runs:
                run(n)
            n += 1
        torch.cuda.synchronize()
    return n


def general_result(args, cfg, wl, dev, nbytes):
    """Several query tokens per sequence and/or a sliding window: a step is
    the append of every new token (kv_append, in position order) followed by
    pkv_paged_attention; the roofline entry times that attention call
    (partition + merge) with event pairs."""
    import torch
    from paged_kv_decode_06_amd import ops

    pool_bytes = 2 * wl.k_cache.numel() * wl.k_cache.element_size()
    copies = args.copies or max(2, int(np.ceil(2.0e9 / pool_bytes)))
    stream = torch.cuda.Stream(device=dev)
    kvd = {"bf16": ops.KV_BF16, "fp8": ops.KV_FP8, "int8": ops.KV_INT8}[wl.kv_dtype]
    mq = int(wl.q_lens.max())
    ws = torch.zeros(ops.attention_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd,
                                                   mq), dtype=torch.uint8, device=dev)
    out = torch.empty_like(wl.q)
    pos = np.concatenate([np.arange(q) for q in wl.q_lens])
    # a quantised cache needs the tokens of one sequence appended in order
    groups = [wl.slot_mapping] if wl.kv_dtype == "bf16" else [
        torch.from_numpy(np.where(pos == i, wl.slot_mapping_np, -1).astype(np.int32)).to(dev)
        for i in range(mq)]
    caches = [(wl.k_cache, wl.v_cache, wl.k_scale, wl.v_scale)]
    for _ in range(copies - 1):
        caches.append(tuple(None if t is None else t.clone() for t in caches[0]))
    steps = []
    for kc, vc, ks, vs in caches:
        apps = [ops.PreparedAppend(wl.k_new, wl.v_new, g, kc, vc, ks, vs, stream=stream)
                for g in groups]
        att = ops.PreparedGeneralAttention(wl.q, kc, vc, wl.block_tables, wl.context_lens,
                                           wl.scale, out, q_start=wl.q_start, max_q_len=mq,
                                           sinks=wl.sinks, window=wl.window, k_scale=ks,
                                           v_scale=vs, workspace=ws, stream=stream)
        steps.append((apps, att))
    torch.cuda.synchronize()
    K, Wm = args.steps, args.warmup

    def run(i):
        apps, att = steps[i % copies]
        for a in apps:
            a()
        att()

    with torch.cuda.stream(stream):
        settled = settle([run], args.settle)
        for i in range(Wm):
            run(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            run(Wm + i)
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / K
        if args.only_step:
            return only_step_line(args, cfg, nbytes, ms_per_step)
        tev = TimingEvents(2 * K)   # (timing-only events: no system-scope fence)
        for i in range(K):
            apps, att = steps[(Wm + i) % copies]
            for a in apps:
                a()
            tev.record(2 * i, stream)
            att()
            tev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
    att_ms = float(np.mean([tev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)]))
    tev.close()
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (att_ms * 1e-3) / 1e9
    keys, _ = visible_keys(wl)
    result = {
        "metric": "KV-read GB/s per decode-attention step (1 MI355X)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}", "kv_dtype": wl.kv_dtype,
            "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "block_size": wl.BS,
            "q_len": mq, "sinks": wl.sinks, "window": wl.window,
            "sum_context": int(wl.lengths.sum()), "keys_seen": int(keys.sum()),
            "num_blocks": wl.NB, "kv_bytes_per_step": nbytes, "kv_cache_copies_cycled": copies,
            "step": "kv_append of the new tokens + paged_attention (partition + merge)",
            "arithmetic": ARITHMETIC,
        },
        "roofline": {
            "bound": "hbm", "kernel": "paged_attention call (mfma_partition_kernel + merge)",
            "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
        },
        "detail": {
            "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
            "attention_call_us_mean": round(att_ms * 1e3, 2),
            "query_rows_heads_per_s": round(int(wl.q_start_np[-1]) * wl.Hq / (ms_per_step * 1e-3), 1),
            "settle_steps_untimed": settled,
        },
    }
    return result


def only_step_line(args, cfg, nbytes, ms_per_step):
    """The line of an --only-step run (for profiler runs: the timed steps and
    nothing else on the GPU)."""
    return {"metric": "KV-read GB/s per decode-attention step (1 MI355X)",
            "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "ms_per_step": round(ms_per_step, 5), "config": {"workload": cfg.name},
            "only_step": True}


def decode_detail(name, args, dev):
    """One decode configuration for detail.configs: K one-call steps (wall
    clock), then the same K steps with timing-only events around the
    partition launch (append inside) and the merge, each step followed by
    the attention call's partition alone on another cache copy (the cost of
    the fused append is the difference of the two partition means)."""
    import torch
    from paged_kv_decode_06_amd import ops
    from paged_kv_decode_06_amd import workloads as W

    wl = W.make_config_workload(name, device=dev, poison=False)
    nbytes = kv_bytes(wl)
    kvd = {"bf16": ops.KV_BF16, "fp8": ops.KV_FP8, "int8": ops.KV_INT8}[wl.kv_dtype]
    pool_bytes = 2 * wl.k_cache.numel() * wl.k_cache.element_size()
    copies = min(16, max(2, int(np.ceil(2.0e9 / pool_bytes))))   # (tiny: latency-bound anyway)
    stream = torch.cuda.Stream(device=dev)
    ws = torch.zeros(ops.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(wl.q)
    caches = [(wl.k_cache, wl.v_cache, wl.k_scale, wl.v_scale)]
    for _ in range(copies - 1):
        caches.append(tuple(None if t is None else t.clone() for t in caches[0]))
    steps = [ops.PreparedStep(wl.q, wl.k_new, wl.v_new, kc, vc, wl.block_tables, wl.context_lens,
                              wl.scale, out, ks, vs, ws, stream=stream)
             for kc, vc, ks, vs in caches]
    atts = [ops.PreparedAttention(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale, out,
                                  ks, vs, ws, stream=stream)
            for kc, vc, ks, vs in caches]
    K, Wm = args.detail_steps, max(3, args.warmup // 2)
    with torch.cuda.stream(stream):
        settle([lambda i: steps[i % copies]()], args.settle)
        for i in range(Wm):
            steps[i % copies]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            steps[(Wm + i) % copies]()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / K
        tev = TimingEvents(6 * K)
        for i in range(K):
            st = steps[(Wm + i) % copies]
            tev.record(6 * i, stream)
            st.partition()
            tev.record(6 * i + 1, stream)
            tev.record(6 * i + 2, stream)
            st.merge()
            tev.record(6 * i + 3, stream)
            at = atts[(Wm + i + copies // 2) % copies]
            tev.record(6 * i + 4, stream)
            at.partition()
            tev.record(6 * i + 5, stream)
            at.merge()
        torch.cuda.synchronize()
    part = float(np.mean([tev.elapsed_ms(6 * i, 6 * i + 1) for i in range(K)]))
    merge = float(np.mean([tev.elapsed_ms(6 * i + 2, 6 * i + 3) for i in range(K)]))
    apart = float(np.mean([tev.elapsed_ms(6 * i + 4, 6 * i + 5) for i in range(K)]))
    tev.close()
    res = {"kv_bytes_per_step": nbytes, "kv_dtype": wl.kv_dtype,
           "shape": f"B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} D{wl.D} BS{wl.BS}",
           "step_us": round(ms * 1e3, 2), "step_GBs": round(nbytes / (ms * 1e-3) / 1e9, 1),
           "step_pct_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
           "partition_us": round(part * 1e3, 2), "merge_us": round(merge * 1e3, 2),
           "attention_partition_us": round(apart * 1e3, 2),
           "fused_append_us": round((part - apart) * 1e3, 2),
           "partition_frac": round(nbytes / (part * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "seq_heads_per_s": round(wl.B * wl.Hq / (ms * 1e-3), 1),
           "steps": K, "kernel_heads_per_wave": ops.decode_unit_heads(wl.B, wl.Hq, wl.Hkv, wl.D,
                                                                      wl.BS, kvd)}
    del steps, atts, caches, ws, out, wl
    torch.cuda.empty_cache()
    return res


def general_detail(name, args, dev):
    """One generalised configuration for detail.configs (general_result with
    the detail step count)."""
    import torch
    from paged_kv_decode_06_amd import workloads as W

    cfg = W.CONFIGS[name]
    wl = W.make_config_workload(name, device=dev, poison=False)
    nbytes = kv_bytes(wl)
    sub = argparse.Namespace(**vars(args))
    sub.steps, sub.warmup, sub.only_step = args.detail_steps, max(3, args.warmup // 2), False
    r = general_result(sub, cfg, wl, dev, nbytes)
    res = {"kv_bytes_per_step": nbytes, "kv_dtype": wl.kv_dtype,
           "shape": (f"B{wl.B} Hq{wl.Hq} Hkv{wl.Hkv} D{wl.D} BS{wl.BS} q_len {cfg.q_len} "
                     f"window {cfg.window} sinks {cfg.sinks}"),
           "step_us": round(r["ms_per_step"] * 1e3, 2), "step_GBs": r["value"],
           "step_pct_peak": r["detail"]["pct_hbm_peak_step"],
           "attention_call_us": r["detail"]["attention_call_us_mean"],
           "attention_call_frac": r["roofline"]["frac"], "steps": sub.steps}
    del wl
    torch.cuda.empty_cache()
    return res


def probe_ceiling(dev, nbytes=2 << 30, reps=20):
    """Read bandwidth of pkv_read_probe over a 2 GiB buffer (timing-only
    events around each of `reps` launches, after 3 untimed ones)."""
    import torch
    from paged_kv_decode_06_amd import ops

    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    sink = torch.zeros(ops.read_probe_waves(), dtype=torch.int32, device=dev)
    stream = torch.cuda.Stream(device=dev)
    tev = TimingEvents(2 * reps)
    with torch.cuda.stream(stream):
        for _ in range(3):
            ops.read_probe(buf, sink, stream=stream)
        for i in range(reps):
            tev.record(2 * i, stream)
            ops.read_probe(buf, sink, stream=stream)
            tev.record(2 * i + 1, stream)
        torch.cuda.synchronize()
    ms = float(np.mean([tev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]))
    tev.close()
    del buf, sink
    torch.cuda.empty_cache()
    return {"GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1), "bytes": nbytes, "us": round(ms * 1e3, 2),
            "waves": ops.read_probe_waves()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--settle", type=float, default=0.3,
                    help="seconds of untimed steps before the warmup (clock settling)")
    ap.add_argument("--config", default="llama3_8b")
    ap.add_argument("--copies", type=int, default=0, help="KV cache copies cycled (0 = auto)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--kernel", choices=["mfma", "valu"], default="mfma",
                    help="partition-kernel variant")
    ap.add_argument("--step", choices=["fused", "two-call"], default="fused",
                    help="decode_step (one call) or kv_append + attention (two calls)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (detail.configs) and the read probe")
    ap.add_argument("--detail-steps", type=int, default=20,
                    help="timed steps per configuration in detail.configs")
    ap.add_argument("--only-step", action="store_true",
                    help="time the selected step only (no events, comparisons, other "
                         "configurations or CPU baseline): for profiler runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reads 1 GiB, writes "
                         "1 GiB) a few times, to scale hardware byte counters")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from paged_kv_decode_06_amd import ops
    from paged_kv_decode_06_amd import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": src.numel(), "copies": 3}), flush=True)
        return
    ops.select_partition_kernel(ops.PARTITION_MFMA if args.kernel == "mfma" else ops.PARTITION_VALU)
    cfg = W.CONFIGS[args.config]
    wl = W.make_config_workload(args.config, device=dev, poison=False)
    nbytes = kv_bytes(wl)
    if cfg.q_len > 1 or cfg.window > 0:
        result = general_result(args, cfg, wl, dev, nbytes)
        if not args.only_step and not args.no_cpu:
            result["cpu_baseline"] = cpu_baseline(wl)
        print(json.dumps(result), flush=True)
        return
    pool_bytes = 2 * wl.k_cache.numel() * wl.k_cache.element_size()
    copies = args.copies or max(2, int(np.ceil(2.0e9 / pool_bytes)))

    stream = torch.cuda.Stream(device=dev)
    kvd = {"bf16": ops.KV_BF16, "fp8": ops.KV_FP8, "int8": ops.KV_INT8}[wl.kv_dtype]
    # (also large enough for the RoPE step, which always runs the MFMA kernel)
    ws = torch.zeros(max(ops.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd),
                         ops.decode_step_rope_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS,
                                                              wl.MBS, kvd)),
                     dtype=torch.uint8, device=dev)
    out = torch.empty_like(wl.q)
    caches = [(wl.k_cache, wl.v_cache, wl.k_scale, wl.v_scale)]
    for _ in range(copies - 1):
        caches.append(tuple(None if t is None else t.clone() for t in caches[0]))
    fused, split = [], []
    for kc, vc, ks, vs in caches:
        fused.append(ops.PreparedStep(wl.q, wl.k_new, wl.v_new, kc, vc, wl.block_tables,
                                      wl.context_lens, wl.scale, out, ks, vs, ws, stream=stream))
        split.append((ops.PreparedAppend(wl.k_new, wl.v_new, wl.slot_mapping, kc, vc, ks, vs,
                                         stream=stream),
                      ops.PreparedAttention(wl.q, kc, vc, wl.block_tables, wl.context_lens,
                                            wl.scale, out, ks, vs, ws, stream=stream)))

    def run_fused(i):
        fused[i % copies]()

    def run_split(i):
        app, att = split[i % copies]
        app()
        att()

    def timed(run, first):
        """Wall time per step of K back-to-back steps (ms)."""
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(K):
            run(first + i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / K

    K, Wm = args.steps, args.warmup
    main_run, other_run = (run_fused, run_split) if args.step == "fused" else (run_split, run_fused)
    with torch.cuda.stream(stream):
        settled = settle([main_run, other_run], args.settle)
        for i in range(Wm):
            other_run(i)
        for i in range(Wm):
            main_run(i)
        # timed region: exactly K steps, nothing else in the stream
        ms_per_step = timed(main_run, Wm)
        if args.only_step:
            print(json.dumps(only_step_line(args, cfg, nbytes, ms_per_step)), flush=True)
            return
        ms_per_step_other = timed(other_run, Wm)

    # the same K steps again with a HIP event pair around every partition
    # launch, recorded on the stream the kernel runs on (the event records
    # themselves add a few microseconds to each bracketed launch)
    def halves(i):
        if args.step == "fused":
            st = fused[i % copies]
            return (lambda: None), st.partition, st.merge
        app, att = split[i % copies]
        return app, att.partition, att.merge

    # (timing-only events: no system-scope fence at each record)
    tev = TimingEvents(2 * K)
    with torch.cuda.stream(stream):
        torch.cuda.synchronize()
        t2 = time.perf_counter()
        for i in range(K):
            pre, part, merge = halves(Wm + i)
            pre()
            tev.record(2 * i, stream)
            part()
            tev.record(2 * i + 1, stream)
            merge()
        torch.cuda.synchronize()
        t3 = time.perf_counter()
    ms_per_step_events = (t3 - t2) * 1e3 / K
    part_ms = [tev.elapsed_ms(2 * i, 2 * i + 1) for i in range(K)]
    part_avg_ms = float(np.mean(part_ms))
    tev.close()
    # the same with torch's default events (a system-scope fence at each
    # record), reported beside it
    ev0 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    ev1 = [torch.cuda.Event(enable_timing=True) for _ in range(K)]
    with torch.cuda.stream(stream):
        for i in range(K):
            pre, part, merge = halves(Wm + i)
            pre()
            ev0[i].record(stream)
            part()
            ev1[i].record(stream)
            merge()
    torch.cuda.synchronize()
    part_avg_ms_fenced = float(np.mean([a.elapsed_time(b) for a, b in zip(ev0, ev1)]))

    # breakdown of one step, each launch between its own pair of events
    nb = min(K, 50)
    e = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(nb)]
    with torch.cuda.stream(stream):
        for i in range(nb):
            pre, part, merge = halves(i)
            e[i][0].record(stream)
            pre()
            e[i][1].record(stream)
            part()
            e[i][2].record(stream)
            merge()
            e[i][3].record(stream)
    torch.cuda.synchronize()
    app_us = float(np.median([x[0].elapsed_time(x[1]) for x in e])) * 1e3
    part_med_us = float(np.median([x[1].elapsed_time(x[2]) for x in e])) * 1e3
    merge_us = float(np.median([x[2].elapsed_time(x[3]) for x in e])) * 1e3

    # the RoPE-fused append at the same batch (rotating q into a scratch
    # tensor and appending the rotated keys into the first cache copy), 50
    # launches between events.  A bounded spin on the stream first lets the
    # host queue all 50 before the first runs, so the events time the GPU,
    # not the launch rate of a few-microsecond kernel.
    q_rot = torch.empty_like(wl.q)
    pos = (wl.context_lens - 1).to(torch.int32)
    kc, vc, ks, vs = caches[0]
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        for i in range(10):
            ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, kc, vc, ks, vs,
                               q_out=q_rot, stream=stream)
        if hasattr(torch.cuda, "_sleep"):
            torch.cuda._sleep(20_000_000)          # ~10 ms of GPU clock cycles
        r0.record(stream)
        for i in range(50):
            ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, kc, vc, ks, vs,
                               q_out=q_rot, stream=stream)
        r1.record(stream)
    torch.cuda.synchronize()
    rope_us = r0.elapsed_time(r1) * 1e3 / 50

    # The decode step with RoPE: one call (rotation inside the partition
    # kernel) against RoPE append + attention, K steps each, wall clock.
    rope_fused = [ops.PreparedStep(wl.q, wl.k_new, wl.v_new, kc_, vc_, wl.block_tables,
                                   wl.context_lens, wl.scale, out, ks_, vs_, ws, stream=stream,
                                   rope={})
                  for kc_, vc_, ks_, vs_ in caches]
    rope_att = [ops.PreparedAttention(q_rot, kc_, vc_, wl.block_tables, wl.context_lens,
                                      wl.scale, out, ks_, vs_, ws, stream=stream)
                for kc_, vc_, ks_, vs_ in caches]

    def run_rope_fused(i):
        rope_fused[i % copies]()

    def run_rope_split(i):
        kc_, vc_, ks_, vs_ = caches[i % copies]
        ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, kc_, vc_, ks_, vs_,
                           q_out=q_rot, stream=stream)
        rope_att[i % copies]()

    # The two are timed in alternating blocks of 5 steps (wall clock around
    # each block), so that a drift of the GPU's clocks over the run weighs on
    # both alike.
    with torch.cuda.stream(stream):
        for i in range(Wm):
            run_rope_fused(i)
            run_rope_split(i)
        spent = {run_rope_fused: 0.0, run_rope_split: 0.0}
        n_blocks = max(1, K // 5)
        for blk in range(n_blocks):
            for run in (run_rope_fused, run_rope_split):
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                for i in range(5):
                    run(Wm + 5 * blk + i)
                torch.cuda.synchronize()
                spent[run] += time.perf_counter() - t0
        rope_step_ms = spent[run_rope_fused] * 1e3 / (5 * n_blocks)
        rope_split_ms = spent[run_rope_split] * 1e3 / (5 * n_blocks)

    value = nbytes / (ms_per_step * 1e-3) / 1e9
    achieved = nbytes / (part_avg_ms * 1e-3) / 1e9
    waves = ops.attention_waves(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, kvd)
    unit_heads = ops.decode_unit_heads(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, kvd)
    result = {
        "metric": "KV-read GB/s per decode-attention step (1 MI355X)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": Wm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "kv_dtype": wl.kv_dtype,
            "B": wl.B, "Hq": wl.Hq, "Hkv": wl.Hkv, "D": wl.D, "block_size": wl.BS,
            "sum_context": int(wl.lengths.sum()), "num_blocks": wl.NB,
            "kv_bytes_per_step": nbytes, "kv_cache_copies_cycled": copies,
            "step": ("decode_step: partition with the append inside + merge"
                     if args.step == "fused" else "kv_append + partition + merge"),
            "arithmetic": ARITHMETIC if args.kernel == "mfma" else ARITHMETIC_VALU,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"{args.kernel}_partition_kernel",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.config, args.kernel),
        },
        "detail": {
            "pct_hbm_peak_step": round(100 * value / HBM_PEAK_GBS, 2),
            "ms_per_step_with_partition_events": round(ms_per_step_events, 5),
            "partition_us_mean": round(part_avg_ms * 1e3, 2),
            "partition_us_mean_default_events": round(part_avg_ms_fenced * 1e3, 2),
            "partition_us_median": round(part_med_us, 2),
            "merge_us_median": round(merge_us, 2),
            "kv_append_us_median": round(app_us, 2) if args.step == "two-call" else None,
            "ms_per_step_" + ("two_call" if args.step == "fused" else "fused"):
                round(ms_per_step_other, 5),
            "seq_heads_per_s": round(wl.B * wl.Hq / (ms_per_step * 1e-3), 1),
            "rope_kv_append_us_mean": round(rope_us, 2),
            "decode_step_rope_us": round(rope_step_ms * 1e3, 2),
            "rope_append_then_attention_us": round(rope_split_ms * 1e3, 2),
            "persistent_waves": waves,
            "settle_steps_untimed": settled,
            "kv_heads_per_wave": unit_heads,
        },
    }
    if not args.no_configs:
        # every other configuration, fewer steps each, and the read ceiling
        probe = probe_ceiling(dev)
        result["detail"]["read_probe"] = probe
        result["detail"]["partition_pct_of_read_probe"] = round(100 * achieved / probe["GB/s"], 2)
        configs = {}
        for name in W.CONFIG_ORDER:
            if name == args.config:
                continue
            c = W.CONFIGS[name]
            if c.q_len > 1 or c.window > 0:
                configs[name] = general_detail(name, args, dev)
            else:
                configs[name] = decode_detail(name, args, dev)
            if name != "tiny":
                frac = configs[name].get("partition_frac", configs[name].get("attention_call_frac"))
                configs[name]["pct_of_read_probe"] = round(100 * frac * HBM_PEAK_GBS / probe["GB/s"], 2)
        result["detail"]["configs"] = configs
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
