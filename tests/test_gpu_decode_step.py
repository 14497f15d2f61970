"""The one-call decode step (pkv_decode_step) against the two calls it
replaces, kv_append with slot = position context_lens[b] - 1 followed by
paged_decode_attention: whole caches, scales and the output bit-identical,
for both partition-kernel variants.  With the MFMA variant the append runs
inside the partition kernel; with VALU the step launches the append kernel
(slots derived on the device) before it.  The tiny configuration is also
checked against the oracle directly.
"""
from __future__ import annotations

import dataclasses
import itertools

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_parity import DEV, KERNELS, SMALL, build, default_kernel, say, use_kernel

pytestmark = pytest.mark.gpu


@pytest.fixture(params=list(KERNELS))
def kernel(request):
    use_kernel(request.param)
    yield request.param
    default_kernel()


def derived_slots(wl: W.Workload) -> np.ndarray:
    """Position L - 1 of each sequence through its block table (-1: none)."""
    out = np.full(wl.B, -1, np.int64)
    for b in range(wl.B):
        L = int(wl.lengths[b])
        if 1 <= L <= wl.MBS * wl.BS:
            blk = int(wl.block_tables_np[b, (L - 1) // wl.BS])
            if 0 <= blk < wl.NB:
                out[b] = blk * wl.BS + (L - 1) % wl.BS
    return out


def twin(wl: W.Workload) -> W.Workload:
    """The same workload on cloned caches and scales."""
    c = lambda t: None if t is None else t.clone()  # noqa: E731
    return dataclasses.replace(wl, k_cache=c(wl.k_cache), v_cache=c(wl.v_cache),
                               k_scale=c(wl.k_scale), v_scale=c(wl.v_scale))


def step(wl: W.Workload, ws=None) -> torch.Tensor:
    out = torch.empty_like(wl.q)
    ws = GS.workspace_for(wl) if ws is None else ws
    ops.decode_step(wl.q, wl.k_new, wl.v_new, wl.k_cache, wl.v_cache, wl.block_tables,
                    wl.context_lens, wl.scale, out, wl.k_scale, wl.v_scale, ws)
    return out


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.uint8)


def assert_same_as_two_calls(wl: W.Workload, what: str):
    assert np.array_equal(derived_slots(wl), wl.slot_mapping_np.astype(np.int64)), what
    fused = twin(wl)
    ref_out = GS.gpu_step(wl)                # kv_append + attention
    out = step(fused)
    torch.cuda.synchronize()
    assert torch.equal(bits(fused.k_cache), bits(wl.k_cache)), f"{what}: K cache"
    assert torch.equal(bits(fused.v_cache), bits(wl.v_cache)), f"{what}: V cache"
    if wl.k_scale is not None:
        assert torch.equal(fused.k_scale.view(torch.int32), wl.k_scale.view(torch.int32)), what
        assert torch.equal(fused.v_scale.view(torch.int32), wl.v_scale.view(torch.int32)), what
    assert torch.equal(bits(out), bits(ref_out)), f"{what}: output"
    return out


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: f"B{s[0]}Hq{s[1]}Hkv{s[2]}D{s[3]}BS{s[4]}{s[6]}")
def test_step_equals_two_calls_small(shape, kernel):
    B, Hq, Hkv, D, BS, lengths, kv = shape
    wl = build(B, Hq, Hkv, D, BS, lengths, kv=kv, seed=B * 10 + D + BS)
    assert_same_as_two_calls(wl, f"{shape}")


def test_step_equals_two_calls_every_variant(kernel):
    """Every (D, BS, G, dtype) instantiation; lengths 1 and BS + 1 put the new
    token at offset 0 (it opens a block and, for fp8, sets the scale), the
    others put it mid-block and on the last offset of a block."""
    for D, BS, G, kv in itertools.product((64, 128), (16, 32), (1, 2, 4, 8, 16),
                                          ("bf16", "fp8", "int8")):
        Hkv = 4
        wl = build(5, Hkv * G, Hkv, D, BS, (1, BS + 1, 2 * BS, 9 * BS + 5, 3 * BS - 1), kv=kv,
                   seed=D + BS + G + 7)
        assert_same_as_two_calls(wl, f"D{D} BS{BS} G{G} {kv}")


@pytest.mark.parametrize("name", ["llama3_8b", "long_context", "mixed_70b", "fp8", "int8"])
def test_step_equals_two_calls_full_configuration(name, kernel):
    say(f"config {name}")
    wl = W.make_config_workload(name, device=DEV, poison=True)
    assert_same_as_two_calls(wl, name)


def test_step_matches_oracle_tiny():
    """Independent of the two-call path: the step's cache bytes equal the
    oracle's append, its output is within tolerance of the oracle's attention,
    and L = 1 gives bf16(v_new) exactly."""
    wl = W.make_config_workload("tiny", device=DEV, poison=True)
    host = GS.HostProblem(wl)
    out = step(wl)
    torch.cuda.synchronize()
    host.append()
    assert np.array_equal(W.cache_host(wl.k_cache)[host.old_blocks], host.k)
    assert np.array_equal(W.cache_host(wl.v_cache)[host.old_blocks], host.v)
    GS.assert_attention_close(GS.bf16_to_f64(out), host.attention(), wl.kv_dtype, "tiny step")
    v_new = wl.v_new.float().cpu().numpy()
    o = out.float().cpu().numpy()
    for h in range(wl.Hq):
        assert np.array_equal(o[0, h], v_new[0, h // wl.G])


def test_step_fp8_matches_oracle():
    """fp8 cache: appends that open a block (new scale) and that land
    mid-block (kept scale), bytes and scales equal to the oracle's append."""
    wl = build(4, 16, 4, 128, 32, (1, 33, 50, 700), kv="fp8", seed=41)
    host = GS.HostProblem(wl)
    out = step(wl)
    torch.cuda.synchronize()
    host.append()
    assert np.array_equal(W.cache_host(wl.k_cache)[host.old_blocks], host.k)
    assert np.array_equal(W.cache_host(wl.v_cache)[host.old_blocks], host.v)
    ks = wl.k_scale.cpu().numpy()[host.old_blocks]
    assert np.array_equal(ks.view(np.uint32), host.ks.view(np.uint32))
    vs = wl.v_scale.cpu().numpy()[host.old_blocks]
    assert np.array_equal(vs.view(np.uint32), host.vs.view(np.uint32))
    GS.assert_attention_close(GS.bf16_to_f64(out), host.attention(), "fp8", "fp8 step")


def test_step_lengths_outside_the_contract(kernel):
    """L = 0 and L > MBS * BS append nothing; L = 0 gives out = 0."""
    wl = build(3, 8, 2, 64, 16, (5, 20, 40), seed=43, poison=False)
    wl.context_lens[0] = 0
    wl.context_lens[2] = wl.MBS * wl.BS + 1
    k0, v0 = wl.k_cache.clone(), wl.v_cache.clone()
    out = step(wl)
    torch.cuda.synchronize()
    assert (out[0] == 0).all()
    changed = (bits(wl.k_cache) != bits(k0)).view(wl.NB * wl.BS, -1).any(1)
    slot1 = int(wl.slot_mapping_np[1])
    rows = torch.nonzero(changed).flatten().tolist()
    assert rows == [slot1] or rows == [], rows      # only sequence 1's slot may change
    assert torch.equal(bits(wl.v_cache.view(wl.NB * wl.BS, -1)[slot1]),
                       bits(wl.v_new[1].reshape(-1)))


def test_repeated_steps_are_idempotent(kernel):
    wl = build(8, 32, 8, 128, 16, np.random.default_rng(5).integers(100, 2000, 8), seed=44)
    ws = GS.workspace_for(wl)
    first = step(wl, ws).clone()
    k1 = wl.k_cache.clone()
    for _ in range(2):
        again = step(wl, ws)
        torch.cuda.synchronize()
        assert torch.equal(bits(again), bits(first))
        assert torch.equal(bits(wl.k_cache), bits(k1))
