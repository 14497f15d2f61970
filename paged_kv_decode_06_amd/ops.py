"""Thin ctypes binding of libpkv.so (declared in include/pkv.h).

Argument marshalling only: shape/dtype checks on the torch tensors, raw
device pointers and the current HIP stream go into the C calls, and every
step of the computation runs in the library's kernels.  The library is
loaded on first use; if it is missing or fails to load, the call raises --
there is no CPU or PyTorch fallback.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

KV_BF16 = 0
KV_FP8 = 1
KV_INT8 = 2

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libpkv.so"
_lib = None
_lock = threading.Lock()


class PkvError(RuntimeError):
    """A libpkv call returned a non-zero status."""

    def __init__(self, fn: str, status: int, text: str, detail: str):
        super().__init__(f"{fn} failed with status {status} ({text}){': ' + detail if detail else ''}")
        self.status = status


def library_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()'). "
                "There is no fallback implementation.")
        lib = ctypes.CDLL(path)
        P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        lib.pkv_kv_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, P]
        lib.pkv_kv_append.restype = I
        lib.pkv_paged_decode_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        lib.pkv_paged_decode_workspace_bytes.restype = S
        attn_args = [P, P, P, P, P, P, P, F, P, I, I, I, I, I, I, I, I, P, S, P]
        for name in ("pkv_paged_decode_attention", "pkv_paged_decode_partition",
                     "pkv_paged_decode_merge", "pkv_validate_inputs"):
            fn = getattr(lib, name)
            fn.argtypes = attn_args
            fn.restype = I
        lib.pkv_paged_decode_attention_noalloc.argtypes = attn_args[:17] + [P]
        lib.pkv_paged_decode_attention_noalloc.restype = I
        Dd = ctypes.c_double
        lib.pkv_rope_kv_append.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I,
                                           Dd, Dd, Dd, Dd, Dd, P]
        lib.pkv_rope_kv_append.restype = I
        lib.pkv_paged_attention.argtypes = [P, P, I, P, P, P, P, P, P, F, I, I, P, I, I, I, I,
                                            I, I, I, I, P, S, P]
        lib.pkv_paged_attention.restype = I
        lib.pkv_paged_attention_workspace_bytes.argtypes = [I, I, I, I, I, I, I, I]
        lib.pkv_paged_attention_workspace_bytes.restype = S
        lib.pkv_decode_step_rope_workspace_bytes.argtypes = [I, I, I, I, I, I, I]
        lib.pkv_decode_step_rope_workspace_bytes.restype = S
        for name in ("pkv_decode_step", "pkv_decode_step_partition"):
            fn = getattr(lib, name)
            fn.argtypes = [P, P, P, P, P, P, P, P, P, F, P, I, I, I, I, I, I, I, I, P, S, P]
            fn.restype = I
        Dbl = ctypes.c_double
        lib.pkv_decode_step_rope.argtypes = ([P] * 9 + [F] + [Dbl] * 5 + [P] + [I] * 8
                                             + [P, S, P])
        lib.pkv_decode_step_rope.restype = I
        lib.pkv_status_string.argtypes = [I]
        lib.pkv_status_string.restype = ctypes.c_char_p
        lib.pkv_last_error.argtypes = []
        lib.pkv_last_error.restype = ctypes.c_char_p
        lib.pkv_attention_waves.argtypes = [I, I, I, I, I, I]
        lib.pkv_attention_waves.restype = I
        lib.pkv_decode_unit_heads.argtypes = [I, I, I, I, I, I]
        lib.pkv_decode_unit_heads.restype = I
        lib.pkv_read_probe_waves.argtypes = []
        lib.pkv_read_probe_waves.restype = I
        lib.pkv_read_probe.argtypes = [P, S, P, S, P]
        lib.pkv_read_probe.restype = I
        lib.pkv_select_share_combine.argtypes = [I]
        lib.pkv_select_share_combine.restype = I
        lib.pkv_select_result_parking.argtypes = [I]
        lib.pkv_select_result_parking.restype = I
        lib.pkv_select_run_cost.argtypes = [I]
        lib.pkv_select_run_cost.restype = I
        lib.pkv_select_unit_heads.argtypes = [I]
        lib.pkv_select_unit_heads.restype = I
        lib.pkv_select_partition_kernel.argtypes = [I]
        lib.pkv_select_partition_kernel.restype = I
        lib.pkv_partition_kernel.argtypes = []
        lib.pkv_partition_kernel.restype = I
        _lib = lib
    return _lib


def lib():
    """The loaded ctypes library (raises if it is not built)."""
    return _load()


def _check(fn: str, status: int):
    if status != 0:
        L = _load()
        raise PkvError(fn, status, L.pkv_status_string(status).decode(),
                       L.pkv_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: int):
    """Type, dtype, rank and layout of one argument (the device is checked
    last, by _on_gpu, once every shape agrees)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_gpu(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be on the GPU")


def _cache_args(k_cache, v_cache, k_scale, v_scale):
    """The caches ([NB, BS, Hkv, D], K and V alike) and, for a quantised
    cache, the scales ([NB, Hkv] fp32 each: the kernels index them by block
    and kv head).  Returns (kv_dtype, NB, BS, Hkv, D)."""
    kvd = _kv_dtype(k_cache)
    _need(k_cache, "k_cache", k_cache.dtype, 4)
    _need(v_cache, "v_cache", k_cache.dtype, 4)
    if tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError(f"v_cache shape {tuple(v_cache.shape)} differs from k_cache "
                         f"{tuple(k_cache.shape)}")
    NB, BS, Hkv, D = k_cache.shape
    if kvd != KV_BF16:
        _need(k_scale, "k_scale", torch.float32, 2)
        _need(v_scale, "v_scale", torch.float32, 2)
        for t, name in ((k_scale, "k_scale"), (v_scale, "v_scale")):
            if tuple(t.shape) != (NB, Hkv):
                raise ValueError(f"{name} must be [NB, Hkv] = {(NB, Hkv)}, got {tuple(t.shape)}")
    elif k_scale is not None or v_scale is not None:
        raise ValueError("a bf16 cache takes no scales")
    return kvd, NB, BS, Hkv, D


def _kv_dtype(k_cache: torch.Tensor) -> int:
    if k_cache.dtype == torch.bfloat16:
        return KV_BF16
    if k_cache.dtype in (torch.uint8, torch.float8_e4m3fn):
        return KV_FP8
    if k_cache.dtype == torch.int8:
        return KV_INT8
    raise TypeError(f"cache dtype must be bfloat16, uint8/float8_e4m3fn or int8, got {k_cache.dtype}")


def _append_args(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream):
    kvd, NB, BS, Hkv, D = _cache_args(k_cache, v_cache, k_scale, v_scale)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    N = k_new.shape[0]
    if tuple(k_new.shape) != (N, Hkv, D) or tuple(v_new.shape) != (N, Hkv, D):
        raise ValueError(f"k_new and v_new must be [N, Hkv, D] with the cache's Hkv, D = "
                         f"{Hkv}, {D}; got {tuple(k_new.shape)}, {tuple(v_new.shape)}")
    if slot_mapping.shape[0] != N:
        raise ValueError("slot_mapping must have one entry per token of k_new")
    _on_gpu(k_new=k_new, v_new=v_new, slot_mapping=slot_mapping, k_cache=k_cache,
            v_cache=v_cache, k_scale=k_scale, v_scale=v_scale)
    return (_ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
            _ptr(k_scale), _ptr(v_scale), N, Hkv, D, BS, NB, kvd, _stream(stream))


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None,
              stream=None) -> None:
    """pkv_kv_append: store each sequence's new K/V token into its slot."""
    args = _append_args(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale, stream)
    _check("pkv_kv_append", _load().pkv_kv_append(*args))


LLAMA3_ROPE = dict(theta=500000.0, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
                   original_max_len=8192.0)


def rope_kv_append(q, k_new, v_new, positions, slot_mapping, k_cache, v_cache, k_scale=None,
                   v_scale=None, q_out=None, theta=500000.0, factor=32.0, low_freq_factor=1.0,
                   high_freq_factor=4.0, original_max_len=8192.0, stream=None) -> None:
    """pkv_rope_kv_append: rotate q (into q_out; in place when q_out is None)
    and the new keys at `positions`, then append the rotated keys and the
    values into their slots.  Defaults are the Llama 3 RoPE parameters."""
    kvd, NB, BS, Hkv, D = _cache_args(k_cache, v_cache, k_scale, v_scale)
    if q_out is None:
        q_out = q
    for t, name in ((q, "q"), (q_out, "q_out"), (k_new, "k_new"), (v_new, "v_new")):
        _need(t, name, torch.bfloat16, 3)
    _need(positions, "positions", torch.int32, 1)
    _need(slot_mapping, "slot_mapping", torch.int32, 1)
    N, Hq = q.shape[0], q.shape[1]
    if (tuple(q.shape) != (N, Hq, D) or tuple(q_out.shape) != (N, Hq, D)
            or tuple(k_new.shape) != (N, Hkv, D) or tuple(v_new.shape) != (N, Hkv, D)
            or positions.shape[0] != N or slot_mapping.shape[0] != N):
        raise ValueError("q, q_out, k_new, v_new, positions, slot_mapping and the caches disagree")
    _on_gpu(q=q, q_out=q_out, k_new=k_new, v_new=v_new, positions=positions,
            slot_mapping=slot_mapping, k_cache=k_cache, v_cache=v_cache, k_scale=k_scale,
            v_scale=v_scale)
    st = _load().pkv_rope_kv_append(
        _ptr(q), _ptr(q_out), _ptr(k_new), _ptr(v_new), _ptr(positions), _ptr(slot_mapping),
        _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale), N, Hq, Hkv, D, BS, NB, kvd,
        float(theta), float(factor), float(low_freq_factor), float(high_freq_factor),
        float(original_max_len), _stream(stream))
    _check("pkv_rope_kv_append", st)


PARTITION_VALU = 0
PARTITION_MFMA = 1


def select_partition_kernel(variant: int) -> None:
    """pkv_select_partition_kernel: 0 = VALU, 1 = MFMA (process-wide; resize
    workspaces afterwards)."""
    _check("pkv_select_partition_kernel", _load().pkv_select_partition_kernel(int(variant)))


def partition_kernel() -> int:
    return int(_load().pkv_partition_kernel())


UNITS_AUTO = 0
UNITS_ONE_HEAD = 1


def select_unit_heads(mode: int) -> None:
    """pkv_select_unit_heads: 0 = several kv heads per MFMA wave where the
    call allows it, 1 = one kv head per wave (process-wide; resize
    workspaces afterwards)."""
    _check("pkv_select_unit_heads", _load().pkv_select_unit_heads(int(mode)))


def select_share_combine(mode: int) -> None:
    """pkv_select_share_combine: 1 = the waves of a workgroup combine their
    partial results in LDS where the call allows it (default), 0 = one partial
    row per wave (process-wide; resize workspaces afterwards)."""
    _check("pkv_select_share_combine", _load().pkv_select_share_combine(int(mode)))


def select_result_parking(mode: int) -> None:
    """pkv_select_result_parking: 1 = generalised calls with one kv head and
    one column tile per wave keep a mid-piece result in LDS until the piece
    ends (default), 0 = store it when its run ends (process-wide; same bits
    either way)."""
    _check("pkv_select_result_parking", _load().pkv_select_result_parking(int(mode)))


def select_run_cost(slots: int) -> None:
    """pkv_select_run_cost: positions of no pages the MFMA work split counts
    ahead of each run (0..8, default 2; process-wide)."""
    _check("pkv_select_run_cost", _load().pkv_select_run_cost(int(slots)))


def decode_unit_heads(B: int, Hq: int, Hkv: int, D: int, BS: int, kv_dtype: int) -> int:
    """Kv heads per partition wave a decode call with these sizes uses
    (kv_dtype: KV_BF16, KV_FP8 or KV_INT8)."""
    return int(_load().pkv_decode_unit_heads(B, Hq, Hkv, D, BS, int(kv_dtype)))


def attention_waves(B: int, Hq: int, Hkv: int, D: int, BS: int, kv_dtype: int) -> int:
    """Persistent waves of a decode call's partition grid with these sizes."""
    return int(_load().pkv_attention_waves(B, Hq, Hkv, D, BS, int(kv_dtype)))


def read_probe_waves() -> int:
    """Waves of the streaming-read probe's grid (the words its sink needs)."""
    return int(_load().pkv_read_probe_waves())


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """pkv_read_probe: read every whole 1 KB unit of `buf` (a contiguous GPU
    tensor) with 16-byte non-temporal loads; one XOR fold per wave in `sink`
    (int32 / uint32 GPU tensor of at least read_probe_waves() words)."""
    if not (isinstance(buf, torch.Tensor) and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous tensor")
    if not (isinstance(sink, torch.Tensor) and sink.is_contiguous() and sink.element_size() == 4):
        raise ValueError("sink must be a contiguous tensor of 32-bit words")
    _on_gpu(buf=buf, sink=sink)
    _check("pkv_read_probe", _load().pkv_read_probe(
        _ptr(buf), ctypes.c_size_t(buf.numel() * buf.element_size()), _ptr(sink),
        ctypes.c_size_t(sink.numel()), _stream(stream)))


def workspace_bytes(B, Hq, Hkv, D, BS, MBS, kv_dtype=KV_BF16) -> int:
    return int(_load().pkv_paged_decode_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kv_dtype))


_NO_WORKSPACE = object()


def _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale, v_scale,
               workspace, stream):
    kvd, NB, BS, Hkv, D2 = _cache_args(k_cache, v_cache, k_scale, v_scale)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B, Hq, D = q.shape
    MBS = block_tables.shape[1]
    if D2 != D or tuple(out.shape) != (B, Hq, D):
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != B or context_lens.shape[0] != B:
        raise ValueError("block_tables/context_lens must have B rows")
    _on_gpu(q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
            context_lens=context_lens, k_scale=k_scale, v_scale=v_scale)
    if workspace is _NO_WORKSPACE:   # (the static-scratch call: no workspace arguments)
        return (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale), _ptr(out),
                B, Hq, Hkv, D, BS, NB, MBS, kvd, _stream(stream))
    if workspace is None:
        raise ValueError("workspace is required (see workspace_bytes)")
    if workspace.dtype != torch.uint8 or not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 GPU tensor")
    return (_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
            _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale), _ptr(out),
            B, Hq, Hkv, D, BS, NB, MBS, kvd, _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), _stream(stream))


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                           k_scale=None, v_scale=None, workspace=None, stream=None) -> None:
    """pkv_paged_decode_attention: out[b, h] = softmax(scale q K^T) V over the paged history."""
    args = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale,
                      v_scale, workspace, stream)
    _check("pkv_paged_decode_attention", _load().pkv_paged_decode_attention(*args))


STATIC_SCRATCH_BYTES = 32 << 20   # PKV_STATIC_SCRATCH_BYTES


def paged_decode_attention_noalloc(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                   k_scale=None, v_scale=None, stream=None) -> None:
    """pkv_paged_decode_attention_noalloc: paged_decode_attention without a
    workspace argument; the library's static per-GPU scratch holds the partial
    results (calls on one GPU must not overlap in time)."""
    args = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale,
                      v_scale, _NO_WORKSPACE, stream)
    _check("pkv_paged_decode_attention_noalloc",
           _load().pkv_paged_decode_attention_noalloc(*args))


def validate_inputs(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                    k_scale=None, v_scale=None, workspace=None, stream=None) -> None:
    """pkv_validate_inputs: check the device-resident inputs of
    paged_decode_attention (lengths, block ids of the used pages, fp8 / int8
    scales of those blocks); synchronises the stream; raises PkvError
    (PKV_ERR_INPUT) naming the first violation."""
    args = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale,
                      v_scale, workspace, stream)
    _check("pkv_validate_inputs", _load().pkv_validate_inputs(*args))


def paged_decode_partition(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                           k_scale=None, v_scale=None, workspace=None, stream=None) -> None:
    """First half of paged_decode_attention (the partition kernel)."""
    args = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale,
                      v_scale, workspace, stream)
    _check("pkv_paged_decode_partition", _load().pkv_paged_decode_partition(*args))


def paged_decode_merge(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                       k_scale=None, v_scale=None, workspace=None, stream=None) -> None:
    """Second half of paged_decode_attention (the log-sum-exp merge kernel)."""
    args = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale,
                      v_scale, workspace, stream)
    _check("pkv_paged_decode_merge", _load().pkv_paged_decode_merge(*args))


def decode_step_rope_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kv_dtype=KV_BF16) -> int:
    return int(_load().pkv_decode_step_rope_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kv_dtype))


def attention_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kv_dtype=KV_BF16, max_q_len=1) -> int:
    return int(_load().pkv_paged_attention_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kv_dtype,
                                                           max_q_len))


def _general_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, q_start,
                  max_q_len, sinks, window, k_scale, v_scale, workspace, stream):
    kvd, NB, BS, Hkv, D2 = _cache_args(k_cache, v_cache, k_scale, v_scale)
    _need(q, "q", torch.bfloat16, 3)
    _need(out, "out", torch.bfloat16, 3)
    _need(block_tables, "block_tables", torch.int32, 2)
    _need(context_lens, "context_lens", torch.int32, 1)
    B = context_lens.shape[0]
    if q_start is not None:
        _need(q_start, "q_start", torch.int32, 1)
        if q_start.shape[0] != B + 1:
            raise ValueError("q_start must have B + 1 entries")
    elif q.shape[0] != B:
        raise ValueError("without q_start, q has one row per sequence")
    TQ, Hq, D = q.shape
    MBS = block_tables.shape[1]
    if D2 != D or tuple(out.shape) != (TQ, Hq, D):
        raise ValueError("q/out/cache shapes disagree")
    if block_tables.shape[0] != B:
        raise ValueError("block_tables must have B rows")
    _on_gpu(q=q, out=out, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
            context_lens=context_lens, q_start=q_start, k_scale=k_scale, v_scale=v_scale)
    if workspace is None or workspace.dtype != torch.uint8 or not workspace.is_cuda:
        raise ValueError("workspace must be a uint8 GPU tensor (see attention_workspace_bytes)")
    return (_ptr(q), _ptr(q_start), int(max_q_len), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale),
            _ptr(v_scale), _ptr(block_tables), _ptr(context_lens), ctypes.c_float(scale),
            int(sinks), int(window), _ptr(out), B, Hq, Hkv, D, BS, NB, MBS, kvd,
            _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, scale, out, q_start=None,
                    max_q_len=1, sinks=0, window=0, k_scale=None, v_scale=None, workspace=None,
                    stream=None) -> None:
    """pkv_paged_attention: q_start[b] .. q_start[b+1]-1 are sequence b's query
    rows (bottom-right causal over its L_b keys); window > 0 keeps only keys
    within the window of each query plus the first `sinks` keys."""
    args = _general_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, q_start,
                         max_q_len, sinks, window, k_scale, v_scale, workspace, stream)
    _check("pkv_paged_attention", _load().pkv_paged_attention(*args))


class PreparedGeneralAttention:
    """paged_attention with its arguments marshalled once (see PreparedAttention)."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, out, q_start=None,
                 max_q_len=1, sinks=0, window=0, k_scale=None, v_scale=None, workspace=None,
                 stream=None):
        self._args = _general_args(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                   q_start, max_q_len, sinks, window, k_scale, v_scale,
                                   workspace, stream)
        self._lib = _load()

    def __call__(self):
        _check("pkv_paged_attention", self._lib.pkv_paged_attention(*self._args))


def _step_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
               k_scale, v_scale, workspace, stream):
    a = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out, k_scale, v_scale,
                   workspace, stream)
    _need(k_new, "k_new", torch.bfloat16, 3)
    _need(v_new, "v_new", torch.bfloat16, 3)
    B, Hkv, D = q.shape[0], k_cache.shape[2], q.shape[2]
    if tuple(k_new.shape) != (B, Hkv, D) or tuple(v_new.shape) != (B, Hkv, D):
        raise ValueError("k_new and v_new must be [B, Hkv, D]")
    _on_gpu(k_new=k_new, v_new=v_new)
    # (q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, ...)
    return (a[0], _ptr(k_new), _ptr(v_new)) + a[1:]


def decode_step(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                k_scale=None, v_scale=None, workspace=None, stream=None) -> None:
    """pkv_decode_step: append each sequence's new token at position
    context_lens[b] - 1, then attend (one call, bit-identical to kv_append
    followed by paged_decode_attention)."""
    args = _step_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                      k_scale, v_scale, workspace, stream)
    _check("pkv_decode_step", _load().pkv_decode_step(*args))


def _rope_args(rope) -> tuple:
    r = dict(LLAMA3_ROPE)
    r.update(rope or {})
    return tuple(float(r[k]) for k in ("theta", "factor", "low_freq_factor", "high_freq_factor",
                                       "original_max_len"))


def decode_step_rope(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                     k_scale=None, v_scale=None, workspace=None, stream=None, rope=None) -> None:
    """pkv_decode_step_rope: the decode step with RoPE of q and the new keys
    at position context_lens[b] - 1 inside the partition kernel (q is not
    changed).  `rope`: overrides of LLAMA3_ROPE.  Size the workspace with
    decode_step_rope_workspace_bytes."""
    a = _step_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                   k_scale, v_scale, workspace, stream)
    _check("pkv_decode_step_rope",
           _load().pkv_decode_step_rope(*(a[:10] + _rope_args(rope) + a[10:])))


class PreparedStep:
    """decode_step (or, with `rope`, decode_step_rope) with its arguments
    marshalled once (see PreparedAttention)."""

    def __init__(self, q, k_new, v_new, k_cache, v_cache, block_tables, context_lens, scale, out,
                 k_scale=None, v_scale=None, workspace=None, stream=None, rope=None):
        self._args = _step_args(q, k_new, v_new, k_cache, v_cache, block_tables, context_lens,
                                scale, out, k_scale, v_scale, workspace, stream)
        a = self._args
        self._merge_args = (a[0],) + a[3:]     # the attention call's arguments
        self._lib = _load()
        self._rope_args = None if rope is None else a[:10] + _rope_args(rope) + a[10:]

    def __call__(self):
        if self._rope_args is not None:
            _check("pkv_decode_step_rope", self._lib.pkv_decode_step_rope(*self._rope_args))
            return
        _check("pkv_decode_step", self._lib.pkv_decode_step(*self._args))

    def partition(self):
        """First half: the append and the partition kernel."""
        _check("pkv_decode_step_partition", self._lib.pkv_decode_step_partition(*self._args))

    def merge(self):
        """Second half: the merge kernel."""
        _check("pkv_paged_decode_merge", self._lib.pkv_paged_decode_merge(*self._merge_args))


class PreparedAttention:
    """The attention call with its arguments marshalled once, for loops that
    launch the same shapes repeatedly (benchmarks, serving loops).  The
    tensors must stay alive and in place for as long as this object is used."""

    def __init__(self, q, k_cache, v_cache, block_tables, context_lens, scale, out,
                 k_scale=None, v_scale=None, workspace=None, stream=None):
        self._args = _attn_args(q, k_cache, v_cache, block_tables, context_lens, scale, out,
                                k_scale, v_scale, workspace, stream)
        self._lib = _load()

    def __call__(self):
        _check("pkv_paged_decode_attention", self._lib.pkv_paged_decode_attention(*self._args))

    def partition(self):
        _check("pkv_paged_decode_partition", self._lib.pkv_paged_decode_partition(*self._args))

    def merge(self):
        _check("pkv_paged_decode_merge", self._lib.pkv_paged_decode_merge(*self._args))


class PreparedAppend:
    """kv_append with its arguments marshalled once (see PreparedAttention)."""

    def __init__(self, k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None,
                 stream=None):
        self._args = _append_args(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale,
                                  stream)
        self._lib = _load()

    def __call__(self):
        _check("pkv_kv_append", self._lib.pkv_kv_append(*self._args))
