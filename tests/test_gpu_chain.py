"""The chain combine of parked shares in the generalised partition kernel (GPU).

Generalised calls whose waves serve one kv head and 9 to 32 columns (e.g. 4
draft tokens at G = 4 or G = 8) park mid-piece results in LDS.  With the
share combine on (the default), a run that crosses the edge between
consecutive waves of a workgroup is combined after the workgroup's barrier
by the first of those waves: the later ones leave their shares in their
parking slots (with two column tiles, tile 0 from the tile buffer on), and
the run leaves one share row per workgroup, or its bf16 output when the
workgroup saw all of it.  Checked through the C ABI: against the fp64
oracle with the chain on and off, outputs within two bf16 steps of each
other (only the summation order differs) and not all equal (the chain was
taken), repeated calls bit for bit, the workspace the same either way, on
runs that end inside a workgroup, pass through all four of its waves or
cross workgroup edges; with windows and sinks, fp8 and int8 caches, D = 64,
G = 2, run costs 0 and 8, and batches whose lengths and query offsets do
not fit in LDS.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_general import build, check
from tests.test_gpu_parity import DEV, default_kernel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def lengths(seed, n_short, n_long, long_hi=5000):
    rng = np.random.default_rng(seed)
    L = np.concatenate([rng.integers(1, 60, n_short), rng.integers(600, long_hi, n_long)])
    rng.shuffle(L)
    return [int(x) for x in L]


def assert_order_only(on: torch.Tensor, off: torch.Tensor, what: str):
    """Outputs that differ only by summation order: within two bf16 steps of
    each other; and not bit for bit the same, so the chain was taken.  (A
    run whose two shares the chain joins gets the merge kernel's bits: both
    scale the first share by the same weight and add the second with one
    fused multiply-add.  The batches here hold runs over many pieces, whose
    workgroup rows the merge then groups otherwise.)"""
    a, b = GS.bf16_to_f64(on), GS.bf16_to_f64(off)
    assert np.all(np.abs(a - b) <= 2 * 2.0 ** -8 * np.maximum(np.abs(a), np.abs(b)) + 1e-6), what
    assert not torch.equal(bits(on), bits(off)), f"{what}: chain not taken"


CASES = [
    # (B-mix seed, n_short, n_long, Hq, Hkv, D, BS, q_len, kv, sinks, window)
    (1, 40, 24, 32, 8, 128, 16, 4, "bf16", 0, 0),     # G = 4, 4 queries: 16 columns
    (2, 60, 8, 16, 8, 128, 32, 8, "bf16", 0, 0),      # G = 2, 8 queries
    (3, 30, 20, 32, 8, 64, 16, 4, "bf16", 0, 0),      # D = 64
    (4, 40, 16, 32, 8, 128, 32, 4, "fp8", 0, 0),
    (5, 40, 16, 32, 8, 128, 32, 3, "int8", 2, 300),   # 12 columns, window with sinks
    (6, 20, 12, 32, 8, 128, 16, 4, "bf16", 16, 1000),
    # two 16-column tiles
    (7, 10, 30, 16, 4, 128, 16, 5, "bf16", 0, 0),     # G = 4, 5 queries: 20 columns
    (8, 60, 10, 64, 8, 128, 16, 4, "bf16", 0, 0),     # G = 8, 4 queries: 32 columns
    (9, 40, 10, 32, 8, 128, 16, 6, "bf16", 2, 300),   # 24 columns, window with sinks
    (10, 40, 12, 64, 8, 128, 32, 4, "fp8", 0, 0),
    (11, 30, 10, 64, 8, 64, 16, 3, "int8", 0, 0),     # D = 64, 24 columns
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[8]}-D{c[5]}G{c[3]//c[4]}-q{c[7]}-W{c[10]}")
def test_chain_on_and_off_meet_the_oracle_and_agree(case):
    seed, ns, nl, Hq, Hkv, D, BS, ql, kv, S, Wn = case
    L = lengths(seed, ns, nl)
    q_lens = [min(ql, x) for x in L]
    wl = build(len(L), Hq, Hkv, D, BS, L, q_lens, kv=kv, seed=seed, poison=False, sinks=S,
               window=Wn)
    on, _ = check(wl, f"{case} chain on")
    again = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(on), bits(again)), "repeated call"
    ops.select_share_combine(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert_order_only(on, off, str(case))


@pytest.mark.parametrize("cost", [0, 8])
def test_chain_with_run_cost(cost):
    """Run costs 0 and 8 move the piece edges against the runs' pages (at 8
    many pieces begin with positions of no pages)."""
    ops.select_run_cost(cost)
    L = lengths(20 + cost, 80, 10)
    wl = build(len(L), 32, 8, 128, 16, L, [min(4, x) for x in L], seed=20 + cost, poison=False)
    on, _ = check(wl, f"chain run cost {cost}")
    ops.select_share_combine(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert_order_only(on, off, f"run cost {cost}")


@pytest.mark.parametrize("B", [700, 2500])
def test_chain_in_large_batches(B):
    """Above 512 sequences the query-row offsets, and above 2048 the
    lengths, come from memory rather than LDS; short sequences put several
    runs in a piece, and the first run of a piece after the first wave of a
    workgroup is often a walker's."""
    rng = np.random.default_rng(B)
    L = [int(x) for x in rng.integers(1, 200, B)]
    for i in rng.choice(B, 8, replace=False):   # runs over many pieces (see assert_order_only)
        L[i] = int(rng.integers(2000, 6000))
    wl = build(B, 32, 8, 64, 16, L, [min(4, x) for x in L], seed=B, poison=False)
    on, _ = check(wl, f"B{B} chain on")
    ops.select_share_combine(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert_order_only(on, off, f"B{B}")


def test_long_runs_through_every_wave():
    """Two sequences of 60000 tokens and 4 queries at G = 4: each run spans
    hundreds of pieces, so every wave of most workgroups carries the run on
    and each workgroup leaves one share row."""
    L = [60000, 45000]
    wl = build(2, 32, 8, 128, 16, L, [4, 4], seed=3, poison=False)
    on, _ = check(wl, "long runs chain on")
    ops.select_share_combine(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert_order_only(on, off, "long runs")


def test_chain_keeps_the_workspace():
    """The chain needs one share row per workgroup and run, fewer than the
    per-piece rows the workspace holds: the query is the same either way."""
    kv = ops.KV_BF16
    on = ops.attention_workspace_bytes(64, 32, 8, 128, 16, 256, kv, 4)
    on2 = ops.attention_workspace_bytes(256, 64, 8, 128, 16, 1024, kv, 4)   # two tiles
    ops.select_share_combine(0)
    off = ops.attention_workspace_bytes(64, 32, 8, 128, 16, 256, kv, 4)
    off2 = ops.attention_workspace_bytes(256, 64, 8, 128, 16, 1024, kv, 4)
    assert on == off and on2 == off2


@pytest.mark.parametrize("name", ["llama3_8b_verify4", "mixed_70b_verify4"])
def test_verify_workload_chain_on_and_off(name):
    """The verify workloads (4 draft tokens; the Llama shape at G = 4, one
    column tile; the 70B-shaped mix at G = 8, two): every output within the
    oracle's bar (covered by the full-configuration test) and within two
    bf16 steps of the unchained outputs; repeated calls bit for bit."""
    wl = W.make_config_workload(name, device=DEV)
    first = GS.general_step(wl, append=False).clone()
    again = GS.general_step(wl, append=False).clone()
    ops.select_share_combine(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(first), bits(again))
    assert_order_only(first, off, name)
    say(f"{name}: outputs that differ from the unchained call",
        int((bits(first) != bits(off)).sum()), "of", first.numel())


def test_two_tile_chain_in_large_batches():
    """Two column tiles (G = 8, 4 queries) at B = 700 and D = 64, where park
    mode 2 still leaves two workgroups per CU: query-row offsets from
    memory, many runs per piece, a few runs over many pieces."""
    rng = np.random.default_rng(70)
    B = 700
    L = [int(x) for x in rng.integers(1, 120, B)]
    for i in rng.choice(B, 6, replace=False):
        L[i] = int(rng.integers(3000, 8000))
    wl = build(B, 64, 8, 64, 16, L, [min(4, x) for x in L], seed=70, poison=False)
    on, _ = check(wl, "B700 two tiles chain on")
    ops.select_share_combine(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert_order_only(on, off, "B700 two tiles")
