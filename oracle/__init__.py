"""fp64 CPU oracle for decode-phase paged attention and the one-token KV append.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``paged_kv_decode_06_amd``) never imports it, and this package imports nothing
from the product path: the two share no code.

The arithmetic lives in ``pkv_oracle.c`` (plain C, built with gcc, no fast-math,
no FMA contraction).  This module only builds it, loads it with ctypes and
marshals numpy arrays.  bf16 tensors travel as their raw 16-bit patterns
(``uint16``), e4m3fn caches as raw bytes (``uint8``).

Sources of each computation (page titles; see the C file for the details):
  * attention: "Decode Phase Attention Forward Pass", sections 2-5 (gather the
    history through the block list, GQA head grouping, no causal mask,
    softmax_scale), with the padding caveat at the end of that page read as
    "positions past the context length take no part";
  * kv_append: "tiny-vllm part 5", section on scattering the new token's K/V
    into 16-token blocks (block = pos / block_size, offset = pos % block_size);
  * fp8: the "Decode Phase" glossary's KV-cache quantisation bullet, with the
    OCP e4m3fn format and a per-(block, kv head) scale amax/448;
  * int8: the same bullet (and the glossary's mixed-precision bullet): a
    symmetric per-(block, kv head) scale amax/127, codes rint(x/scale)
    clamped to +-127;
  * generalised attention: "Prefill Forward Prefix Caching Explained", the
    bottom-right causal mask (query i of q_len new tokens sees key j iff
    j <= i + kv_len - q_len), plus the glossary's sliding-window and
    attention-sink bullets (keys older than the window are hidden except the
    first `sinks` tokens);
  * RoPE: "tiny-vllm part 5", the RoPE section (adjacent-pair rotation,
    theta^(-2i/D) frequencies with the Llama 3 scaling of the table path).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pkv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

KV_BF16 = 0
KV_FP8 = 1
KV_INT8 = 2

_lib = None


def build(force: bool = True) -> str:
    """Compile ``pkv_oracle.c`` into ``liboracle.so`` with gcc."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = [
        "gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
        "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
        "-o", tmp, _SRC, "-lm",
    ]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    override = os.environ.get("PKV_ORACLE_LIB")   # a deliberately broken copy, for the mutation test
    if override:
        lib = ctypes.CDLL(override)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.pkvo_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.pkvo_bf16_to_f64.restype = ctypes.c_double
    lib.pkvo_e4m3fn_to_f64.argtypes = [ctypes.c_uint8]
    lib.pkvo_e4m3fn_to_f64.restype = ctypes.c_double
    lib.pkvo_e4m3fn_from_f32.argtypes = [ctypes.c_float]
    lib.pkvo_e4m3fn_from_f32.restype = ctypes.c_uint8
    lib.pkvo_e4m3fn_decode_array.argtypes = [P, P, ctypes.c_int64]
    lib.pkvo_e4m3fn_decode_array.restype = None
    lib.pkvo_e4m3fn_encode_array.argtypes = [P, P, ctypes.c_int64]
    lib.pkvo_e4m3fn_encode_array.restype = None
    lib.pkvo_paged_decode_attention.argtypes = [
        P, P, P, P, P, P, P, ctypes.c_float, P, P, I, I, I, I, I, I, I, I, I]
    lib.pkvo_paged_decode_attention.restype = I
    lib.pkvo_kv_append.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I]
    lib.pkvo_kv_append.restype = I
    lib.pkvo_int8_from_f32.argtypes = [ctypes.c_float]
    lib.pkvo_int8_from_f32.restype = ctypes.c_int8
    lib.pkvo_paged_attention.argtypes = [
        P, P, P, P, P, P, P, P, ctypes.c_float, I, I, P, P, I, I, I, I, I, I, I, I, I]
    lib.pkvo_paged_attention.restype = I
    D_ = ctypes.c_double
    lib.pkvo_rope_freqs.argtypes = [I, D_, D_, D_, D_, D_, P]
    lib.pkvo_rope_freqs.restype = None
    lib.pkvo_rope_apply.argtypes = [P, P, I, I, I, P, P, P]
    lib.pkvo_rope_apply.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def e4m3fn_decode(codes: np.ndarray) -> np.ndarray:
    """Exact value of each e4m3fn byte, as fp64 (NaN for the NaN codes)."""
    codes = _c(codes, np.uint8)
    out = np.empty(codes.shape, np.float64)
    _load().pkvo_e4m3fn_decode_array(_ptr(codes), _ptr(out), codes.size)
    return out


def e4m3fn_encode(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even, saturating e4m3fn encode of fp32 values."""
    x = _c(x, np.float32)
    out = np.empty(x.shape, np.uint8)
    _load().pkvo_e4m3fn_encode_array(_ptr(x), _ptr(out), x.size)
    return out


def _cache_dtype(k_cache, v_cache, k_scale, v_scale):
    if k_cache.dtype == np.uint16:
        return KV_BF16, _c(k_cache, np.uint16), _c(v_cache, np.uint16), None, None
    if k_cache.dtype == np.uint8:
        return (KV_FP8, _c(k_cache, np.uint8), _c(v_cache, np.uint8),
                _c(k_scale, np.float32), _c(v_scale, np.float32))
    if k_cache.dtype == np.int8:
        return (KV_INT8, _c(k_cache, np.int8), _c(v_cache, np.int8),
                _c(k_scale, np.float32), _c(v_scale, np.float32))
    raise TypeError("cache must be uint16 (bf16 bits), uint8 (e4m3fn) or int8")


def int8_encode(x: np.ndarray) -> np.ndarray:
    """int8 code of fp32 quotients: rint (halves to even), clamped to +-127."""
    x = _c(x, np.float32)
    f = _load().pkvo_int8_from_f32
    return np.array([f(float(v)) for v in x.ravel()], np.int8).reshape(x.shape)


def paged_attention(q, k_cache, v_cache, block_tables, context_lens, scale, q_start=None,
                    sinks=0, window=0, k_scale=None, v_scale=None, num_blocks=None,
                    return_weights=False, nthreads=0):
    """fp64 reference of the generalised attention, ``[total_q, Hq, D]``.

    q: uint16 bf16 bits [total_q, Hq, D]; q_start: int32 [B + 1] cumulative
    query counts (None: one query per sequence, total_q = B).  Query i of
    sequence b sees key j iff j <= L_b - q_len_b + i and (window <= 0 or
    j > that limit - window or j < sinks).
    """
    q = _c(q, np.uint16)
    kv_dtype, k_cache, v_cache, k_scale, v_scale = _cache_dtype(k_cache, v_cache, k_scale, v_scale)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    B = context_lens.shape[0]
    if q_start is not None:
        q_start = _c(q_start, np.int32)
        assert q_start.shape == (B + 1,) and q_start[-1] == q.shape[0]
    else:
        assert q.shape[0] == B
    TQ, Hq, D = q.shape
    NB, BS, Hkv, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    MBS = block_tables.shape[1]
    out = np.zeros((TQ, Hq, D), np.float64)
    w = np.zeros((TQ, Hq, MBS * BS), np.float64) if return_weights else None
    st = _load().pkvo_paged_attention(
        _ptr(q), _ptr(q_start), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), float(scale), int(sinks), int(window),
        _ptr(out), _ptr(w), B, Hq, Hkv, D, BS, NB if num_blocks is None else num_blocks, MBS,
        kv_dtype, int(nthreads))
    if st != 0:
        raise ValueError(f"oracle attention rejected its inputs (status {st})")
    return (out, w) if return_weights else out


def rope_freqs(D, theta=500000.0, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
               original_max=8192.0) -> np.ndarray:
    """The D/2 rotary frequencies (fp64), Llama 3 scaling (factor 1: none)."""
    f = np.zeros(D // 2, np.float64)
    _load().pkvo_rope_freqs(int(D), float(theta), float(factor), float(low_freq_factor),
                            float(high_freq_factor), float(original_max), _ptr(f))
    return f


def rope_apply(x, positions, freqs):
    """Rotate x (bf16 bits [N, H, D]) at positions [N]; returns (bf16 bits,
    the unrounded fp64 rotation)."""
    x = _c(x, np.uint16)
    positions = _c(positions, np.int32)
    freqs = _c(freqs, np.float64)
    N, H, D = x.shape
    assert positions.shape == (N,) and freqs.shape == (D // 2,)
    y = np.empty_like(x)
    y64 = np.empty(x.shape, np.float64)
    _load().pkvo_rope_apply(_ptr(x), _ptr(positions), N, H, D, _ptr(freqs), _ptr(y), _ptr(y64))
    return y, y64


def paged_decode_attention(q, k_cache, v_cache, block_tables, context_lens, scale,
                           k_scale=None, v_scale=None, num_blocks=None,
                           return_weights=False, nthreads=0):
    """fp64 reference output ``[B, Hq, D]`` (and optionally the weights).

    q: uint16 bf16 bits [B, Hq, D]; k_cache/v_cache: uint16 [NB, BS, Hkv, D]
    (bf16), uint8 (e4m3fn) or int8 [NB, BS, Hkv, D] (then k_scale/v_scale
    are fp32 [NB, Hkv]); block_tables int32 [B, MBS]; context_lens int32 [B].
    """
    q = _c(q, np.uint16)
    kv_dtype, k_cache, v_cache, k_scale, v_scale = _cache_dtype(k_cache, v_cache, k_scale, v_scale)
    block_tables = _c(block_tables, np.int32)
    context_lens = _c(context_lens, np.int32)
    B, Hq, D = q.shape
    NB, BS, Hkv, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    MBS = block_tables.shape[1]
    out = np.zeros((B, Hq, D), np.float64)
    w = np.zeros((B, Hq, MBS * BS), np.float64) if return_weights else None
    st = _load().pkvo_paged_decode_attention(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(context_lens), float(scale), _ptr(out), _ptr(w),
        B, Hq, Hkv, D, BS, NB if num_blocks is None else num_blocks, MBS, kv_dtype,
        int(nthreads))
    if st != 0:
        raise ValueError(f"oracle attention rejected its inputs (status {st})")
    return (out, w) if return_weights else out


def kv_append(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale=None, v_scale=None):
    """Append in place into host (numpy) caches; returns nothing."""
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    slot_mapping = _c(slot_mapping, np.int32)
    for a in (k_cache, v_cache, k_scale, v_scale):
        if a is not None and not a.flags["C_CONTIGUOUS"]:
            raise ValueError("caches must be C-contiguous (updated in place)")
    if k_cache.dtype == np.uint16:
        kv_dtype = KV_BF16
    elif k_cache.dtype in (np.uint8, np.int8):
        kv_dtype = KV_FP8 if k_cache.dtype == np.uint8 else KV_INT8
        assert k_scale.dtype == np.float32 and v_scale.dtype == np.float32
    else:
        raise TypeError("cache must be uint16, uint8 (e4m3fn) or int8")
    N, Hkv, D = k_new.shape
    NB, BS = k_cache.shape[0], k_cache.shape[1]
    st = _load().pkvo_kv_append(
        _ptr(k_new), _ptr(v_new), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
        _ptr(k_scale), _ptr(v_scale), N, Hkv, D, BS, NB, kv_dtype)
    if st != 0:
        raise ValueError(f"oracle kv_append rejected its inputs (status {st})")
