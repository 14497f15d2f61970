"""The decode step with RoPE inside the partition kernel
(pkv_decode_step_rope) against the calls it fuses: pkv_rope_kv_append of q
and the new keys at position context_lens[b] - 1 into the derived slot, then
pkv_paged_decode_attention on the rotated q.  Caches, scales and the output
must be bit-identical (the kernel rotates with the append kernel's fp64
arithmetic and the attention runs the same MFMA kernel and split), with
several kv heads per wave and with one.  Independently, the output is
compared with the oracle: its RoPE ("tiny-vllm part 5", the RoPE section)
of q and the new keys, its append and its attention.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_decode_step import bits, twin
from tests.test_gpu_parity import DEV, build, default_kernel, say, use_kernel

pytestmark = pytest.mark.gpu

LLAMA3 = dict(theta=500000.0, factor=32.0, low_freq_factor=1.0, high_freq_factor=4.0,
              original_max_len=8192.0)


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


def workspace(wl, q_room=True):
    """The RoPE step's workspace; without the room for a rotated q (the
    attention call's size) a one-head call keeps the fused kernel."""
    kvd = GS.KV_KIND[wl.kv_dtype]
    n = max(ops.workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd),
            ops.attention_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd, 1))
    if q_room:
        n = ops.decode_step_rope_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd)
    return torch.zeros(n, dtype=torch.uint8, device=DEV)


def fused(wl, rope=None, q_room=True):
    out = torch.empty_like(wl.q)
    ops.decode_step_rope(wl.q, wl.k_new, wl.v_new, wl.k_cache, wl.v_cache, wl.block_tables,
                         wl.context_lens, wl.scale, out, wl.k_scale, wl.v_scale,
                         workspace(wl, q_room), rope=rope)
    return out


def two_calls(wl, rope=None):
    r = dict(LLAMA3, **(rope or {}))
    pos = torch.from_numpy((wl.lengths - 1).astype(np.int32)).to(DEV)
    q_rot = torch.empty_like(wl.q)
    ops.rope_kv_append(wl.q, wl.k_new, wl.v_new, pos, wl.slot_mapping, wl.k_cache, wl.v_cache,
                       wl.k_scale, wl.v_scale, q_out=q_rot, theta=r["theta"], factor=r["factor"],
                       low_freq_factor=r["low_freq_factor"],
                       high_freq_factor=r["high_freq_factor"],
                       original_max_len=r["original_max_len"])
    out = torch.empty_like(wl.q)
    ops.paged_decode_attention(q_rot, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                               wl.scale, out, wl.k_scale, wl.v_scale, workspace(wl))
    return out


def assert_fused_equals_two_calls(wl, what, rope=None, q_room=True):
    other = twin(wl)
    q0 = wl.q.clone()
    a = fused(wl, rope, q_room)
    b = two_calls(other, rope)
    torch.cuda.synchronize()
    assert torch.equal(wl.q, q0), f"{what}: q changed"
    assert torch.equal(bits(wl.k_cache), bits(other.k_cache)), f"{what}: K cache"
    assert torch.equal(bits(wl.v_cache), bits(other.v_cache)), f"{what}: V cache"
    if wl.k_scale is not None:
        assert torch.equal(wl.k_scale.view(torch.int32), other.k_scale.view(torch.int32)), what
        assert torch.equal(wl.v_scale.view(torch.int32), other.v_scale.view(torch.int32)), what
    assert torch.equal(bits(a), bits(b)), f"{what}: output"
    return a


CASES = [
    # (B, Hq, Hkv, D, BS, lengths, kv)
    (4, 32, 8, 128, 16, (1, 17, 900, 5000), "bf16"),
    (3, 16, 8, 64, 32, (32, 33, 2000), "bf16"),
    (3, 64, 8, 128, 16, (2, 700, 3000), "bf16"),
    (4, 32, 8, 128, 32, (1, 33, 1000, 4097), "fp8"),
    (3, 8, 2, 64, 16, (16, 17, 600), "fp8"),
    (4, 32, 8, 128, 32, (1, 33, 1000, 4097), "int8"),
    (3, 20, 5, 128, 16, (9, 300, 2500), "bf16"),      # odd Hkv: one kv head per wave
]


@pytest.mark.parametrize("q_room", [True, False], ids=["room", "noroom"])
@pytest.mark.parametrize("units", ["mfma", "mfma1"])
@pytest.mark.parametrize("case", CASES, ids=lambda s: f"Hq{s[1]}Hkv{s[2]}D{s[3]}BS{s[4]}{s[6]}")
def test_fused_rope_step_equals_the_two_calls(case, units, q_room):
    """With one kv head per wave (mfma1, or the odd Hkv) the step runs the two
    calls themselves when the workspace has room for the rotated q, and the
    fused one-head kernel otherwise; both must give the two calls' bits."""
    B, Hq, Hkv, D, BS, lengths, kv = case
    use_kernel(units)
    wl = build(B, Hq, Hkv, D, BS, lengths, kv=kv, seed=B + Hq + D + BS)
    assert_fused_equals_two_calls(wl, f"{case} {units} q_room={q_room}", q_room=q_room)


def test_rope_step_workspace_query():
    """The RoPE step's workspace is the attention call's plus a rotated q."""
    for B, Hq, Hkv, D, BS, MBS, kvd in [(4, 32, 8, 128, 16, 64, ops.KV_BF16),
                                        (3, 20, 5, 64, 32, 40, ops.KV_FP8),
                                        (64, 32, 8, 128, 16, 256, ops.KV_INT8)]:
        room = (B * Hq * D * 2 + 255) // 256 * 256
        assert ops.decode_step_rope_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kvd) == \
            ops.attention_workspace_bytes(B, Hq, Hkv, D, BS, MBS, kvd, 1) + room
    assert ops.decode_step_rope_workspace_bytes(4, 32, 8, 96, 16, 64, ops.KV_BF16) == 0


def test_fused_rope_step_plain_rope_parameters():
    """factor 1 (plain RoPE) and another theta."""
    wl = build(3, 32, 8, 128, 16, (5, 3000, 9000), seed=77)
    assert_fused_equals_two_calls(wl, "plain", rope=dict(theta=10000.0, factor=1.0))


def test_fused_rope_step_matches_oracle():
    """The oracle's RoPE of q and the new keys at L - 1, its append and its
    attention; q is compared through the attention output (bars of the
    decode step) since the rotated q never leaves the kernel."""
    for kv in ("bf16", "fp8"):
        wl = build(4, 32, 8, 128, 16, (1, 17, 900, 5000), kv=kv, seed=91)
        f = oracle.rope_freqs(128, 500000.0, 32.0, 1.0, 4.0, 8192.0)
        pos = (wl.lengths - 1).astype(np.int32)
        q_ref, _ = oracle.rope_apply(W.bf16_bits(wl.q), pos, f)
        k_ref, _ = oracle.rope_apply(W.bf16_bits(wl.k_new), pos, f)
        rot = dataclasses.replace(
            wl, q=torch.from_numpy(q_ref.view(np.int16)).to(DEV).view(torch.bfloat16),
            k_new=torch.from_numpy(k_ref.view(np.int16)).to(DEV).view(torch.bfloat16))
        host = GS.HostProblem(rot)              # the oracle's view, taken before the GPU runs
        out = fused(wl)
        torch.cuda.synchronize()
        host.append()
        GS.assert_attention_close(GS.bf16_to_f64(out), host.attention(), kv, f"rope step {kv}")
        if kv == "bf16":   # position 0 (the first sequence, L = 1) sees its own value only
            assert np.array_equal(out[0].float().cpu().numpy(),
                                  np.repeat(wl.v_new[0].float().cpu().numpy(), wl.G, axis=0))


def test_fused_rope_step_rejects_bad_parameters():
    wl = build(2, 8, 2, 64, 16, (5, 40), seed=2)
    with pytest.raises(ops.PkvError):
        fused(wl, rope=dict(theta=1.0))
    with pytest.raises(ops.PkvError):
        fused(wl, rope=dict(low_freq_factor=4.0, high_freq_factor=1.0))
