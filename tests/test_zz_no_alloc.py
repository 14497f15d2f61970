"""The allocation-free attention entry point (pkv_paged_decode_attention_noalloc)
against the workspace one it mirrors, through the C ABI (GPU).

Both run the same kernels with the same grid, so their outputs must be equal
bit for bit.  Two calls in a row, the second on a smaller input: the static
scratch keeps the first call's partial results, and the second must not
depend on them.
"""
from __future__ import annotations

import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as S

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def default_kernels():
    # (other tests may have switched the process-wide selections)
    ops.select_partition_kernel(ops.PARTITION_MFMA)
    ops.select_unit_heads(ops.UNITS_AUTO)
    yield


def with_workspace(wl) -> torch.Tensor:
    out = torch.empty_like(wl.q)
    ops.paged_decode_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                               wl.scale, out, wl.k_scale, wl.v_scale, S.workspace_for(wl))
    return out


def without_workspace(wl) -> torch.Tensor:
    out = torch.full_like(wl.q, float("nan"))
    ops.paged_decode_attention_noalloc(wl.q, wl.k_cache, wl.v_cache, wl.block_tables,
                                       wl.context_lens, wl.scale, out, wl.k_scale, wl.v_scale)
    return out


def _announce(what: str):
    print(f"\n[no_alloc] {what}", flush=True)


@pytest.mark.parametrize("first,second", [("llama3_8b", "tiny"), ("fp8", "tiny")])
def test_two_calls_in_a_row_match_the_workspace_call(first, second):
    dev = "cuda:0"
    big = W.make_config_workload(first, device=dev)
    small = W.make_config_workload(second, device=dev, poison=True)
    assert S.workspace_for(big).numel() <= ops.STATIC_SCRATCH_BYTES
    for wl in (big, small):
        _announce(f"{wl.name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} D={wl.D} BS={wl.BS} {wl.kv_dtype}")
        got = without_workspace(wl)
        ref = with_workspace(wl)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), wl.name
    # the small call also against the oracle (its history is NaN-poisoned
    # outside the pre-filled tokens; position L - 1 is filled by the append)
    small2 = W.make_config_workload(second, device=dev, poison=True)
    host = S.HostProblem(small2)
    ops.kv_append(small2.k_new, small2.v_new, small2.slot_mapping, small2.k_cache,
                  small2.v_cache, small2.k_scale, small2.v_scale)
    got = without_workspace(small2)
    torch.cuda.synchronize()
    host.append()
    S.assert_attention_close(S.bf16_to_f64(got), host.attention(), small2.kv_dtype, "noalloc tiny")


def test_sizes_beyond_the_scratch_are_rejected_before_any_launch():
    dev = "cuda:0"
    B, Hq, Hkv, D, BS, NB, MBS = 8192, 32, 8, 128, 16, 4, 1
    _announce(f"rejection: B={B}")
    need = ops.workspace_bytes(B, Hq, Hkv, D, BS, MBS)
    assert need > ops.STATIC_SCRATCH_BYTES
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev)
    out = torch.full_like(q, 7.0)
    kc = torch.zeros((NB, BS, Hkv, D), dtype=torch.bfloat16, device=dev)
    bt = torch.zeros((B, MBS), dtype=torch.int32, device=dev)
    cl = torch.ones(B, dtype=torch.int32, device=dev)
    with pytest.raises(ops.PkvError) as ei:
        ops.paged_decode_attention_noalloc(q, kc, kc.clone(), bt, cl, 0.1, out)
    assert ei.value.status == -4
    assert "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())          # nothing ran
    # a call that fits still works afterwards
    wl = W.make_config_workload("tiny", device=dev)
    got = without_workspace(wl)
    ref = with_workspace(wl)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))


def test_empty_batch_is_a_no_op():
    ops.lib()
    st = ops.lib().pkv_paged_decode_attention_noalloc(None, None, None, None, None, None, None,
                                                      0.1, None, 0, 8, 2, 64, 16, 4, 1, 0, None)
    assert st == 0
