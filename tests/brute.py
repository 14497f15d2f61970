"""Dense reference computations used to pin the oracle.

Written independently of the oracle: the paged cache is first gathered into a
dense [L, Hkv, D] history per sequence with numpy fancy indexing (the
"gather the whole history" step of "Decode Phase Attention Forward Pass",
section 2, but cut to each sequence's own length), then attention is the
textbook softmax(q K^T * scale) V, either in numpy fp64 or through torch's
CPU scaled_dot_product_attention in fp64 (a library routine).
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_to_f64_torch(codes: np.ndarray) -> np.ndarray:
    """Library decode of e4m3fn bytes (torch's float8_e4m3fn)."""
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def dequant_cache(cache: np.ndarray, scales: np.ndarray | None) -> np.ndarray:
    """[NB, BS, Hkv, D] cache (uint16 bf16 bits or uint8 e4m3fn) -> fp64 values."""
    if cache.dtype == np.uint16:
        return bf16_bits_to_f64(cache)
    vals = e4m3fn_to_f64_torch(cache)
    return vals * scales.astype(np.float64)[:, None, :, None]


def gather_history(cache_f64: np.ndarray, block_table_row: np.ndarray, L: int, BS: int) -> np.ndarray:
    """Dense [L, Hkv, D] history of one sequence."""
    t = np.arange(L)
    blocks = block_table_row[t // BS]
    return cache_f64[blocks, t % BS]


def dense_attention_numpy(q_bits, k_cache, v_cache, block_tables, context_lens, scale,
                          k_scale=None, v_scale=None) -> np.ndarray:
    q = bf16_bits_to_f64(q_bits)
    B, Hq, D = q.shape
    Kf = dequant_cache(k_cache, k_scale)
    Vf = dequant_cache(v_cache, v_scale)
    NB, BS, Hkv, _ = Kf.shape
    G = Hq // Hkv
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        K = gather_history(Kf, block_tables[b], L, BS)  # [L, Hkv, D]
        V = gather_history(Vf, block_tables[b], L, BS)
        Kq = np.repeat(K, G, axis=1)                     # head h reads kv head h // G
        Vq = np.repeat(V, G, axis=1)
        s = np.einsum("hd,thd->ht", q[b], Kq) * float(np.float32(scale))
        s -= s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[b] = np.einsum("ht,thd->hd", w, Vq)
    return out


def dense_attention_torch_sdpa(q_bits, k_cache, v_cache, block_tables, context_lens, scale,
                               k_scale=None, v_scale=None) -> np.ndarray:
    """Same result through torch.nn.functional.scaled_dot_product_attention (CPU, fp64)."""
    q = torch.from_numpy(bf16_bits_to_f64(q_bits))
    B, Hq, D = q.shape
    Kf = dequant_cache(k_cache, k_scale)
    Vf = dequant_cache(v_cache, v_scale)
    BS, Hkv = Kf.shape[1], Kf.shape[2]
    out = torch.zeros((B, Hq, D), dtype=torch.float64)
    for b in range(B):
        L = int(context_lens[b])
        if L <= 0:
            continue
        K = torch.from_numpy(np.ascontiguousarray(gather_history(Kf, block_tables[b], L, BS)))
        V = torch.from_numpy(np.ascontiguousarray(gather_history(Vf, block_tables[b], L, BS)))
        o = torch.nn.functional.scaled_dot_product_attention(
            q[b][:, None, :],                     # [Hq, 1, D]
            K.permute(1, 0, 2).contiguous(),      # [Hkv, L, D]
            V.permute(1, 0, 2).contiguous(),
            scale=float(np.float32(scale)), enable_gqa=True)
        out[b] = o[:, 0, :]
    return out.numpy()


def zero_padded_attention_numpy(q_bits, k_cache, v_cache, block_tables, context_lens, scale) -> np.ndarray:
    """The simplified route the first page warns about: every sequence is padded
    with zero K/V rows up to the batch's longest length and the pads are NOT
    masked, so they take softmax weight.  Used only as a negative reference."""
    q = bf16_bits_to_f64(q_bits)
    B, Hq, D = q.shape
    Kf = dequant_cache(k_cache, None)
    Vf = dequant_cache(v_cache, None)
    BS, Hkv = Kf.shape[1], Kf.shape[2]
    G = Hq // Hkv
    Lmax = int(max(context_lens))
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(context_lens[b])
        K = np.zeros((Lmax, Hkv, D))
        V = np.zeros((Lmax, Hkv, D))
        K[:L] = gather_history(Kf, block_tables[b], L, BS)
        V[:L] = gather_history(Vf, block_tables[b], L, BS)
        Kq = np.repeat(K, G, axis=1)
        Vq = np.repeat(V, G, axis=1)
        s = np.einsum("hd,thd->ht", q[b], Kq) * float(np.float32(scale))
        s -= s.max(axis=1, keepdims=True)
        w = np.exp(s)
        w /= w.sum(axis=1, keepdims=True)
        out[b] = np.einsum("ht,thd->hd", w, Vq)
    return out
