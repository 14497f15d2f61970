"""The run cost of the MFMA work split (GPU).

The split counts `run_cost` positions of no pages ahead of each non-empty
(sequence, unit) run, so that waves whose pieces start several runs get fewer
pages; the merge kernel finds a run's share rows from its first and last page
positions.  Checked through the C ABI at costs 0, 2 (the default) and 8 (many
pieces then hold only such positions, or a run's first page only): the
two-call step against the fp64 oracle, the fused step bit for bit the
two-call one, and the generalised call against the oracle, on batches of
short and long sequences.  (Empty sequences, which take no positions at
all, are covered at the default cost by the parity tests' emptied batches.)
"""
from __future__ import annotations

import numpy as np
import pytest

from paged_kv_decode_06_amd import ops
from tests import gpu_support as GS
from tests.test_gpu_decode_step import assert_same_as_two_calls
from tests.test_gpu_general import build as build_general
from tests.test_gpu_general import check as check_general
from tests.test_gpu_parity import build, check_step, default_kernel, use_kernel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


def mix(seed, n_short, n_long, hi=4000):
    rng = np.random.default_rng(seed)
    L = np.concatenate([rng.integers(1, 40, n_short), rng.integers(500, hi, n_long)])
    rng.shuffle(L)
    return [int(x) for x in L]


@pytest.mark.parametrize("cost", [0, 2, 8])
@pytest.mark.parametrize("mode,kv", [("mfma", "bf16"), ("mfma1", "bf16"), ("mfma", "fp8"),
                                     ("mfma", "int8")])
def test_decode_with_run_cost(cost, mode, kv):
    use_kernel(mode)
    ops.select_run_cost(cost)
    L = mix(cost + 3, 150, 12)
    BS = 16 if kv == "bf16" else 32
    wl = build(len(L), 32, 8, 128, BS, L, kv=kv, seed=cost + 5)
    check_step(wl, f"run cost {cost} {mode} {kv}")
    wl2 = build(len(L), 32, 8, 128, BS, L, kv=kv, seed=cost + 6)
    assert_same_as_two_calls(wl2, f"run cost {cost} {mode} {kv} fused")


@pytest.mark.parametrize("cost", [0, 8])
def test_sixteen_heads_with_run_cost(cost):
    """G = 16 (one kv head, 16 columns): stored shares and outputs."""
    ops.select_run_cost(cost)
    L = mix(11, 80, 6)
    wl = build(len(L), 128, 8, 128, 16, L, seed=12)
    check_step(wl, f"G16 run cost {cost}")


@pytest.mark.parametrize("cost", [0, 2, 8])
@pytest.mark.parametrize("q_len,Hq,window", [(4, 32, 0), (4, 64, 0), (1, 32, 300)])
def test_generalised_with_run_cost(cost, q_len, Hq, window):
    ops.select_run_cost(cost)
    L = mix(cost + 20, 60, 8)
    wl = build_general(len(L), Hq, 8, 128, 16, L, [min(q_len, x) for x in L], seed=cost + 21,
                       sinks=4 if window else 0, window=window)
    check_general(wl, f"run cost {cost} q{q_len} Hq{Hq} W{window}")


def test_run_cost_range():
    with pytest.raises(ops.PkvError):
        ops.select_run_cost(9)
    with pytest.raises(ops.PkvError):
        ops.select_run_cost(-1)


def test_emptied_sequences_with_run_cost():
    """Every 5th sequence emptied (L = 0: no positions at all, output 0) at
    cost 8; the rest still within the bar of the oracle."""
    import torch
    ops.select_run_cost(8)
    L = mix(31, 100, 8)
    wl = build(len(L), 32, 8, 128, 16, L, seed=31)
    _, ref = check_step(wl, "run cost 8 before emptying")
    wl.context_lens[::5] = 0
    out0 = GS.gpu_step(wl, append=False)
    torch.cuda.synchronize()
    assert (out0[::5] == 0).all()
    keep = np.ones(len(L), dtype=bool)
    keep[::5] = False
    GS.assert_attention_close(GS.bf16_to_f64(out0)[keep], ref[keep], wl.kv_dtype, "emptied")
