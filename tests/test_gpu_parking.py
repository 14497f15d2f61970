"""Parking of mid-piece results in the generalised partition kernel (GPU).

Calls whose partition waves serve one kv head, without the workgroup combine
(e.g. 4 draft tokens at G = 4 or G = 8), keep the result of a run that a wave
finishes before its last one in LDS (with two 16-column tiles, a share's
first tile in registers) and store it after the wave's last tile.  Checked
through the C ABI: against the fp64 oracle, and, with the share combine off
(so that no shares are chained through the slots: see test_gpu_chain), bit
for bit the same output as storing every result when its run ends
(pkv_select_result_parking(0)), on batches whose pieces hold complete short
runs (parked bf16 outputs), runs split across pieces (parked shares) and
several runs per piece (the slot is taken; later results are stored at
once).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_general import build, check
from tests.test_gpu_parity import DEV, default_kernel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore():
    yield
    ops.select_result_parking(1)
    default_kernel()


def rng_lengths(seed, n_short, n_long, long_hi=5000):
    rng = np.random.default_rng(seed)
    L = np.concatenate([rng.integers(1, 60, n_short), rng.integers(600, long_hi, n_long)])
    rng.shuffle(L)
    return [int(x) for x in L]


CASES = [
    # (B-mix seed, n_short, n_long, Hq, Hkv, D, BS, q_len, kv, sinks, window)
    (1, 40, 24, 32, 8, 128, 16, 4, "bf16", 0, 0),     # G = 4, 4 queries: 16 columns
    (2, 60, 8, 16, 8, 128, 32, 8, "bf16", 0, 0),      # G = 2, 8 queries
    (3, 30, 20, 32, 8, 64, 16, 4, "bf16", 0, 0),      # D = 64
    (4, 40, 16, 32, 8, 128, 32, 4, "fp8", 0, 0),
    (5, 40, 16, 32, 8, 128, 32, 3, "int8", 2, 300),   # window with sinks
    (6, 20, 12, 128, 8, 128, 16, 1, "bf16", 4, 256),  # G = 16, one query, window
    # two 16-column tiles: the share's first tile waits in registers
    (7, 60, 10, 64, 8, 128, 16, 4, "bf16", 0, 0),     # G = 8, 4 queries: 32 columns
    (8, 40, 10, 32, 8, 128, 16, 6, "bf16", 2, 300),   # G = 4, 6 queries: 24 columns, window
    (9, 40, 12, 64, 8, 128, 32, 4, "fp8", 0, 0),
    (10, 30, 10, 64, 8, 64, 16, 3, "int8", 0, 0),     # D = 64, 24 columns
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[8]}-D{c[5]}G{c[3]//c[4]}-q{c[7]}-W{c[10]}")
def test_parking_meets_the_oracle_and_changes_no_bit(case):
    seed, ns, nl, Hq, Hkv, D, BS, ql, kv, S, Wn = case
    L = rng_lengths(seed, ns, nl)
    q_lens = [min(ql, x) for x in L]
    wl = build(len(L), Hq, Hkv, D, BS, L, q_lens, kv=kv, seed=seed, poison=False, sinks=S,
               window=Wn)
    ops.select_share_combine(0)
    ops.select_result_parking(1)
    on, _ = check(wl, f"{case} parking on")
    ops.select_result_parking(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))


@pytest.mark.parametrize("name", ["llama3_8b_verify4", "mixed_70b_verify4"])
def test_full_verify_workload_bit_for_bit(name):
    """The verify workloads (4 draft tokens; G = 4: one tile, G = 8: two),
    share combine off: parking on and off give the same bits, and repeated
    calls too."""
    wl = W.make_config_workload(name, device=DEV)
    ops.select_share_combine(0)
    ops.select_result_parking(1)
    first = GS.general_step(wl, append=False).clone()
    again = GS.general_step(wl, append=False).clone()
    ops.select_result_parking(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), again.view(torch.int16))
    assert torch.equal(first.view(torch.int16), off.view(torch.int16))


def test_parking_keeps_the_workspace():
    """Parking never changes the grid, so the workspace queries do not
    depend on it."""
    kv = ops.KV_BF16
    on = ops.attention_workspace_bytes(64, 32, 8, 128, 16, 256, kv, 4)
    ops.select_result_parking(0)
    off = ops.attention_workspace_bytes(64, 32, 8, 128, 16, 256, kv, 4)
    assert on == off


@pytest.mark.parametrize("window", [0, 300])
def test_parking_with_duplicated_columns(window):
    """At most 8 columns (one query at G = 4, one kv head per wave) normally
    take the workgroup combine; with it off the results are parked, in the
    layout where columns 8..15 repeat columns 0..7: bit for bit the stored
    results, and within the oracle's bar."""
    L = rng_lengths(41, 50, 12)
    wl = build(len(L), 32, 8, 128, 16, L, [1] * len(L), seed=41, poison=False,
               sinks=4 if window else 0, window=window)
    ops.select_unit_heads(1)
    ops.select_share_combine(0)
    ops.select_result_parking(1)
    on, _ = check(wl, f"dup parking window {window}")
    ops.select_result_parking(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))


@pytest.mark.parametrize("B", [700, 2500])
def test_parking_with_two_tiles_in_large_batches(B):
    """Two column tiles park at any batch size: above 512 sequences the
    query-row offsets, and above 2048 the lengths, come from memory rather
    than LDS.  Short sequences (many runs per piece), 4 draft tokens at
    G = 8: within the oracle's bar and bit for bit the stored results."""
    rng = np.random.default_rng(B)
    L = [int(x) for x in rng.integers(1, 60, B)]
    wl = build(B, 64, 8, 64, 16, L, [min(4, x) for x in L], seed=B, poison=False)
    ops.select_share_combine(0)
    ops.select_result_parking(1)
    on, _ = check(wl, f"B{B} two tiles parking on")
    ops.select_result_parking(0)
    off = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(on.view(torch.int16), off.view(torch.int16))
