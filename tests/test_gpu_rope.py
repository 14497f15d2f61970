"""GPU checks of the RoPE-fused append (pkv_rope_kv_append) against the
oracle's RoPE ("tiny-vllm part 5", the RoPE section; Llama 3 scaled
frequencies) and its kv_append.

Rotated elements are floating point: each must be within one bf16 step of
the oracle's (both round the fp64 rotation to nearest even, and only the
libraries' pow / sin / cos can differ, in the last fp64 bit), and equal in
all but a vanishing fraction.  The append of the rotated keys is then
checked bit for bit against the oracle's kv_append of the same bf16 keys.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import brute
from tests.test_gpu_parity import DEV, say

pytestmark = pytest.mark.gpu

LLAMA3 = dict(theta=500000.0, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
              original_max=8192.0)


def freqs(D, **kw):
    p = dict(LLAMA3, **kw)
    return oracle.rope_freqs(D, p["theta"], p["factor"], p["low_freq_factor"],
                             p["high_freq_factor"], p["original_max"])


def assert_within_one_step(gpu_bits: np.ndarray, ref_bits: np.ndarray, what: str):
    """|gpu - ref| <= one bf16 step of ref, and (almost) always equal."""
    g = brute.bf16_bits_to_f64(gpu_bits)
    r = brute.bf16_bits_to_f64(ref_bits)
    step = np.abs(brute.bf16_bits_to_f64((ref_bits.astype(np.int64) + 1).astype(np.uint16)) - r)
    assert (np.abs(g - r) <= step).all(), f"{what}: off by more than one bf16 step"
    diff = int((gpu_bits != ref_bits).sum())
    assert diff <= max(1, gpu_bits.size // 100000), f"{what}: {diff} of {gpu_bits.size} differ"


def build(B, Hq, Hkv, D, BS, lengths, kv="bf16", seed=0):
    say(f"case B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} kv={kv} L={list(lengths)[:6]} seed={seed}")
    return W.build_workload("t", B, Hq, Hkv, D, BS, list(lengths), kv_dtype=kv, seed=seed,
                            device=DEV, poison=True)


def positions_of(wl):
    return torch.from_numpy((wl.lengths - 1).astype(np.int32)).to(DEV)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 8, 2), (128, 16, 1)])
def test_rope_bf16_matches_oracle(D, Hq, Hkv):
    L = [1, 2, 78, 4096, 8193, 40000, 131072][: 7]
    wl = build(len(L), Hq, Hkv, D, 16, L, seed=D + Hq)
    pos = positions_of(wl)
    q0, k0 = W.bf16_bits(wl.q), W.bf16_bits(wl.k_new)
    q_out = torch.empty_like(wl.q)
    ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, wl.k_cache, wl.v_cache,
                       q_out=q_out)
    torch.cuda.synchronize()
    f = freqs(D)
    pos_np = (wl.lengths - 1).astype(np.int32)
    q_ref, _ = oracle.rope_apply(q0, pos_np, f)
    k_ref, _ = oracle.rope_apply(k0, pos_np, f)
    assert_within_one_step(W.bf16_bits(q_out), q_ref, "q")
    kc = W.cache_host(wl.k_cache).reshape(-1, Hkv, D)
    vc = W.cache_host(wl.v_cache).reshape(-1, Hkv, D)
    assert_within_one_step(kc[wl.slot_mapping_np], k_ref, "k")
    assert np.array_equal(vc[wl.slot_mapping_np], W.bf16_bits(wl.v_new))
    # position 0 (the first sequence) is the identity
    assert np.array_equal(W.bf16_bits(q_out)[0], q0[0])


def test_plain_rope_and_in_place():
    wl = build(4, 32, 8, 128, 16, [5, 300, 9000, 70000], seed=3)
    pos = positions_of(wl)
    q0 = W.bf16_bits(wl.q)
    q = wl.q.clone()
    ops.rope_kv_append(q, wl.k_new, wl.v_new, pos, wl.slot_mapping, wl.k_cache, wl.v_cache,
                       factor=1.0)              # in place, no Llama 3 scaling
    torch.cuda.synchronize()
    q_ref, _ = oracle.rope_apply(q0, (wl.lengths - 1).astype(np.int32), freqs(128, factor=1.0))
    assert_within_one_step(W.bf16_bits(q), q_ref, "q plain")


@pytest.mark.parametrize("kv", ["fp8", "int8"])
def test_quantised_append_of_the_rotated_keys_is_bit_exact(kv):
    """Blocks opened by the new token and blocks already open: the codes and
    scales equal the oracle's kv_append of the oracle's own rotation of the
    keys.  (The rotated bf16 keys of the two sides agree bit for bit on these
    inputs, checked on a bf16 twin cache: the encoding is then compared on
    identical values.)"""
    L = [1, 33, 64, 65, 1000, 4097]
    wl = build(len(L), 32, 8, 128, 32, L, kv=kv, seed=7)
    twin = build(len(L), 32, 8, 128, 32, L, kv="bf16", seed=7)
    pos = positions_of(wl)
    pos_np = (wl.lengths - 1).astype(np.int32)
    host_k, host_v = W.cache_host(wl.k_cache).copy(), W.cache_host(wl.v_cache).copy()
    ks, vs = wl.k_scale.cpu().numpy().copy(), wl.v_scale.cpu().numpy().copy()
    k0, v0 = W.bf16_bits(wl.k_new), W.bf16_bits(wl.v_new)
    qa, qb = torch.empty_like(wl.q), torch.empty_like(wl.q)
    ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, wl.k_cache, wl.v_cache,
                       wl.k_scale, wl.v_scale, q_out=qa)
    ops.rope_kv_append(twin.q, twin.k_new, twin.v_new, pos, twin.slot_mapping, twin.k_cache,
                       twin.v_cache, q_out=qb)
    torch.cuda.synchronize()
    assert torch.equal(qa.view(torch.int16), qb.view(torch.int16))
    k_rot, _ = oracle.rope_apply(k0, pos_np, freqs(128))
    gpu_rot = W.cache_host(twin.k_cache).reshape(-1, 8, 128)[twin.slot_mapping_np]
    assert np.array_equal(gpu_rot, k_rot), "rotated keys differ: the encodings are not comparable"
    oracle.kv_append(k_rot, v0, wl.slot_mapping_np, host_k, host_v, ks, vs)
    assert np.array_equal(W.cache_host(wl.k_cache), host_k)
    assert np.array_equal(W.cache_host(wl.v_cache), host_v)
    assert np.array_equal(wl.k_scale.cpu().numpy().view(np.uint32), ks.view(np.uint32))
    assert np.array_equal(wl.v_scale.cpu().numpy().view(np.uint32), vs.view(np.uint32))


def test_skipped_slot_still_rotates_q():
    wl = build(3, 16, 4, 64, 16, [10, 20, 30], seed=9)
    pos = positions_of(wl)
    k0 = wl.k_cache.clone()
    skip = torch.full_like(wl.slot_mapping, -1)
    q_out = torch.empty_like(wl.q)
    ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, skip, wl.k_cache, wl.v_cache, q_out=q_out)
    torch.cuda.synchronize()
    assert torch.equal(k0.view(torch.int16), wl.k_cache.view(torch.int16))
    q_ref, _ = oracle.rope_apply(W.bf16_bits(wl.q), (wl.lengths - 1).astype(np.int32), freqs(64))
    assert_within_one_step(W.bf16_bits(q_out), q_ref, "q")


def test_rotated_step_attention_matches_oracle():
    """The decode step with RoPE: rotate and append, then attend with the
    rotated queries; against the oracle's rope, append and attention."""
    from tests import gpu_support as GS
    wl = build(4, 32, 8, 128, 16, [17, 500, 2049, 6000], seed=11)
    host = GS.HostProblem(wl)
    pos = positions_of(wl)
    q_rot = torch.empty_like(wl.q)
    ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, wl.k_cache, wl.v_cache,
                       q_out=q_rot)
    out = torch.empty_like(wl.q)
    ops.paged_decode_attention(q_rot, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                               wl.scale, out, workspace=GS.workspace_for(wl))
    torch.cuda.synchronize()
    f = freqs(128)
    p = (wl.lengths - 1).astype(np.int32)
    host.q, _ = oracle.rope_apply(host.q, p, f)
    host.k_new, _ = oracle.rope_apply(host.k_new, p, f)
    host.append()
    GS.assert_attention_close(GS.bf16_to_f64(out), host.attention(), "bf16", "rope step")
