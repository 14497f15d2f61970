"""Helpers for the GPU parity tests: run a decode step through the C ABI and
the same step through the oracle, on the same seeded inputs.

The oracle only ever sees generator output (the pre-append cache, q and the
new token), never anything the HIP path produced.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W

BF16_ATOL = 4e-3
BF16_RTOL = 8e-3
FP8_ATOL = 3e-2


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


KV_KIND = {"bf16": ops.KV_BF16, "fp8": ops.KV_FP8, "int8": ops.KV_INT8}


def workspace_for(wl: W.Workload) -> torch.Tensor:
    kvd = KV_KIND[wl.kv_dtype]
    n = ops.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd)
    assert n > 0
    return torch.zeros(n, dtype=torch.uint8, device=wl.q.device)   # zero-filled once


def gpu_step(wl: W.Workload, out=None, workspace=None, append=True) -> torch.Tensor:
    """kv_append of this step's token, then attention; returns out (bf16)."""
    if append:
        ops.kv_append(wl.k_new, wl.v_new, wl.slot_mapping, wl.k_cache, wl.v_cache,
                      wl.k_scale, wl.v_scale)
    if out is None:
        out = torch.empty_like(wl.q)
    if workspace is None:
        workspace = workspace_for(wl)
    ops.paged_decode_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                               wl.scale, out, wl.k_scale, wl.v_scale, workspace)
    return out


class HostProblem:
    """Host (numpy) copy of a workload, or of a subset of its sequences with
    their pages renumbered into a compact pool, taken before the GPU runs."""

    def __init__(self, wl: W.Workload, seqs=None):
        BS = wl.BS
        seqs = list(range(wl.B)) if seqs is None else list(seqs)
        self.seqs = seqs
        pages = [wl.block_tables_np[b, : (int(wl.lengths[b]) + BS - 1) // BS] for b in seqs]
        old = np.concatenate(pages).astype(np.int64)
        self.old_blocks = old
        remap = {int(p): i for i, p in enumerate(old)}
        idx = torch.from_numpy(old).to(wl.k_cache.device)
        self.k = W.cache_host(wl.k_cache.index_select(0, idx)).copy()
        self.v = W.cache_host(wl.v_cache.index_select(0, idx)).copy()
        if wl.k_scale is not None:
            self.ks = wl.k_scale.index_select(0, idx).cpu().numpy().copy()
            self.vs = wl.v_scale.index_select(0, idx).cpu().numpy().copy()
        else:
            self.ks = self.vs = None
        mbs = max(len(p) for p in pages)
        self.bt = np.full((len(seqs), mbs), -1, np.int32)
        for i, p in enumerate(pages):
            self.bt[i, : len(p)] = [remap[int(x)] for x in p]
        self.cl = wl.lengths[seqs].astype(np.int32)
        sel = torch.tensor(seqs, device=wl.q.device)
        self.q = W.bf16_bits(wl.q.index_select(0, sel))
        self.k_new = W.bf16_bits(wl.k_new.index_select(0, sel))
        self.v_new = W.bf16_bits(wl.v_new.index_select(0, sel))
        slots = []
        for i, b in enumerate(seqs):
            blk, off = divmod(int(wl.slot_mapping_np[b]), BS)
            slots.append(remap[blk] * BS + off)
        self.slots = np.array(slots, np.int32)
        self.scale = wl.scale
        self.BS = BS

    def append(self):
        oracle.kv_append(self.k_new, self.v_new, self.slots, self.k, self.v, self.ks, self.vs)

    def attention(self, nthreads=0):
        return oracle.paged_decode_attention(self.q, self.k, self.v, self.bt, self.cl, self.scale,
                                             k_scale=self.ks, v_scale=self.vs,
                                             nthreads=nthreads)


def error_report(gpu: np.ndarray, ref: np.ndarray, kv_dtype: str | None = None) -> dict:
    """Max and RMS absolute error, the max error relative to |ref| over the
    elements with |ref| >= 1e-2 (near-zero outputs make the plain ratio
    meaningless), and, given the cache kind, the largest fraction of the
    tolerance bar any element uses."""
    err = np.abs(gpu - ref)
    big = np.abs(ref) >= 1e-2
    rep = dict(max_abs=float(err.max()), rms=float(np.sqrt((err ** 2).mean())),
               max_rel=float((err[big] / np.abs(ref[big])).max()) if big.any() else 0.0)
    if kv_dtype is not None:
        rep["bar_used"] = float((err / tolerance_bar(ref, kv_dtype)).max())
    return rep


def tolerance_bar(ref: np.ndarray, kv_dtype: str) -> np.ndarray:
    """Elementwise bound on |gpu - ref| for the cache kind (see
    assert_attention_close)."""
    if kv_dtype == "fp8":
        return np.full(ref.shape, FP8_ATOL)
    return BF16_ATOL + BF16_RTOL * np.abs(ref)


def assert_attention_close(gpu: np.ndarray, ref: np.ndarray, kv_dtype: str, what: str = ""):
    """bf16 and int8 caches: |gpu - ref| <= 4e-3 + 8e-3 |ref| elementwise;
    fp8: <= 3e-2 absolute (both against the oracle on the stored values: the
    dequantised codes for fp8 and int8).  The int8 cache is held to the bf16
    bar: its codes and scales are exact inputs to both sides, as bf16 values
    are."""
    assert gpu.shape == ref.shape
    assert np.isfinite(gpu).all(), f"{what}: non-finite output"
    err = np.abs(gpu - ref)
    bad = err > tolerance_bar(ref, kv_dtype)
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {bad.sum()} elements out of tolerance, first at {tuple(i)}: "
            f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}; {error_report(gpu, ref, kv_dtype)}")


class GeneralHost:
    """Host (numpy) copy of a workload with several query tokens per sequence,
    or of a subset of its sequences with their pages renumbered into a compact
    pool, taken before the GPU runs.  The oracle appends the step's tokens in
    position order, then runs the generalised attention."""

    def __init__(self, wl: W.Workload, seqs=None):
        BS = wl.BS
        seqs = list(range(wl.B)) if seqs is None else list(seqs)
        pages = [wl.block_tables_np[b, : (int(wl.lengths[b]) + BS - 1) // BS] for b in seqs]
        old = np.concatenate(pages).astype(np.int64)
        self.old_blocks = old
        remap = {int(p): i for i, p in enumerate(old)}
        idx = torch.from_numpy(old).to(wl.k_cache.device)
        self.k = W.cache_host(wl.k_cache.index_select(0, idx)).copy()
        self.v = W.cache_host(wl.v_cache.index_select(0, idx)).copy()
        if wl.k_scale is not None:
            self.ks = wl.k_scale.index_select(0, idx).cpu().numpy().copy()
            self.vs = wl.v_scale.index_select(0, idx).cpu().numpy().copy()
        else:
            self.ks = self.vs = None
        mbs = max(len(p) for p in pages)
        self.bt = np.full((len(seqs), mbs), -1, np.int32)
        for i, p in enumerate(pages):
            self.bt[i, : len(p)] = [remap[int(x)] for x in p]
        self.cl = wl.lengths[seqs].astype(np.int32)
        qs = wl.q_start_np
        rows = np.concatenate([np.arange(qs[b], qs[b + 1]) for b in seqs])
        self.rows = rows                                 # q rows of the subset, in order
        self.q_start = np.zeros(len(seqs) + 1, np.int32)
        self.q_start[1:] = np.cumsum([qs[b + 1] - qs[b] for b in seqs])
        sel = torch.from_numpy(rows).to(wl.q.device)
        self.q = W.bf16_bits(wl.q.index_select(0, sel))
        self.k_new = W.bf16_bits(wl.k_new.index_select(0, sel))
        self.v_new = W.bf16_bits(wl.v_new.index_select(0, sel))
        slots = []
        for r in rows:
            blk, off = divmod(int(wl.slot_mapping_np[r]), BS)
            slots.append(remap[blk] * BS + off)
        self.slots = np.array(slots, np.int32)
        self.pos_in_seq = np.concatenate([np.arange(qs[b + 1] - qs[b]) for b in seqs])
        self.scale = wl.scale
        self.window, self.sinks = wl.window, wl.sinks

    def append(self):
        """In position order: a token that opens a block comes before the
        tokens that land in it."""
        for i in range(int(self.pos_in_seq.max()) + 1):
            s = np.where(self.pos_in_seq == i, self.slots, -1).astype(np.int32)
            oracle.kv_append(self.k_new, self.v_new, s, self.k, self.v, self.ks, self.vs)

    def attention(self, sinks=None, window=None, nthreads=0):
        return oracle.paged_attention(
            self.q, self.k, self.v, self.bt, self.cl, self.scale, q_start=self.q_start,
            sinks=self.sinks if sinks is None else sinks,
            window=self.window if window is None else window,
            k_scale=self.ks, v_scale=self.vs, nthreads=nthreads)


def append_in_order(wl: W.Workload):
    """kv_append of the step's tokens on the GPU, one position at a time (a
    token that opens an fp8/int8 block comes before the tokens landing in it)."""
    ql = wl.q_lens
    pos = np.concatenate([np.arange(q) for q in ql])
    for i in range(int(ql.max())):
        s = torch.from_numpy(np.where(pos == i, wl.slot_mapping_np, -1).astype(np.int32))
        ops.kv_append(wl.k_new, wl.v_new, s.to(wl.q.device), wl.k_cache, wl.v_cache,
                      wl.k_scale, wl.v_scale)


def general_step(wl: W.Workload, sinks=None, window=None, out=None, workspace=None,
                 append=True) -> torch.Tensor:
    """The step's appends, then the generalised attention; returns out."""
    if append:
        append_in_order(wl)
    kvd = KV_KIND[wl.kv_dtype]
    mq = int(wl.q_lens.max())
    if workspace is None:
        n = ops.attention_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd, mq)
        assert n > 0
        workspace = torch.zeros(n, dtype=torch.uint8, device=wl.q.device)
    if out is None:
        out = torch.empty_like(wl.q)
    ops.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.scale,
                        out, q_start=wl.q_start, max_q_len=mq,
                        sinks=wl.sinks if sinks is None else sinks,
                        window=wl.window if window is None else window,
                        k_scale=wl.k_scale, v_scale=wl.v_scale, workspace=workspace)
    return out
