"""Seeded random sweep of valid inputs against the oracle.

The hand-picked cases cover each shape variant and edge case once; this
sweep draws combinations of them (batch, query group, kv heads, head dim,
block size, cache kind, lengths with page-boundary and length-1 cases mixed
in, and for the generalised call query counts, windows and sinks) so that
interactions none of them picks are checked too.  Every case is a fixed
seed: a failure names its case and reproduces.  The last two sweeps also set
the process-wide switches (run cost, parking, combine, unit size) at random.
"""
from __future__ import annotations

import numpy as np
import pytest

from tests.test_gpu_decode_step import assert_same_as_two_calls
from tests.test_gpu_general import build as build_general
from tests.test_gpu_general import check as check_general
from tests.test_gpu_parity import build, check_step, say

pytestmark = pytest.mark.gpu


def draw_lengths(rng, B, BS, lo=1, hi=3000):
    L = rng.integers(lo, hi, B)
    for i in range(B):              # page boundaries and single tokens now and then
        r = rng.random()
        if r < 0.15:
            L[i] = BS * int(rng.integers(1, 40)) + 1      # the new token opens a block
        elif r < 0.25:
            L[i] = BS * int(rng.integers(1, 40))          # the new token fills one
        elif r < 0.3:
            L[i] = 1
    return [int(x) for x in L]


def draw_shape(rng):
    G = int(rng.choice([1, 2, 4, 8, 16]))
    Hkv = int(rng.choice([1, 2, 3, 4, 8] if G < 16 else [1, 2, 4, 8]))
    D = int(rng.choice([64, 128]))
    BS = int(rng.choice([16, 32]))
    kv = str(rng.choice(["bf16", "fp8", "int8"]))
    B = int(rng.integers(1, 13))
    return B, G * Hkv, Hkv, D, BS, kv


@pytest.mark.parametrize("seed", range(40))
def test_random_decode_step(seed):
    """kv_append + attention against the oracle, and the one-call step
    bit-identical to them."""
    rng = np.random.default_rng(5000 + seed)
    B, Hq, Hkv, D, BS, kv = draw_shape(rng)
    L = draw_lengths(rng, B, BS)
    say(f"seed {seed}: B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} {kv} L={L}")
    wl = build(B, Hq, Hkv, D, BS, L, kv=kv, seed=seed)
    check_step(wl, f"seed {seed}")
    wl = build(B, Hq, Hkv, D, BS, L, kv=kv, seed=seed)
    assert_same_as_two_calls(wl, f"seed {seed}")


@pytest.mark.parametrize("seed", range(30))
def test_random_general_attention(seed):
    rng = np.random.default_rng(7000 + seed)
    B, Hq, Hkv, D, BS, kv = draw_shape(rng)
    G = Hq // Hkv
    qmax = 16 // G
    q = [int(rng.integers(1, qmax + 1)) for _ in range(B)]
    L = [max(l, qq) for l, qq in zip(draw_lengths(rng, B, BS), q)]
    window = int(rng.choice([0, 0, int(rng.integers(1, 600))]))
    sinks = int(rng.integers(0, 40)) if window > 0 and rng.random() < 0.6 else 0
    say(f"seed {seed}: B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} {kv} L={L} q={q} "
        f"window={window} sinks={sinks}")
    wl = build_general(B, Hq, Hkv, D, BS, L, q, kv=kv, seed=seed, sinks=sinks, window=window)
    check_general(wl, f"seed {seed}")


@pytest.mark.parametrize("seed", range(20))
def test_random_general_attention_two_tiles(seed):
    """Query counts past one 16-column tile (16 < G * max_q <= 32); one
    sequence always takes the most, the others are ragged."""
    rng = np.random.default_rng(9000 + seed)
    B, Hq, Hkv, D, BS, kv = draw_shape(rng)
    G = Hq // Hkv
    qmax = 32 // G
    q = [int(rng.integers(1, qmax + 1)) for _ in range(B)]
    q[int(rng.integers(0, B))] = qmax
    L = [max(l, qq) for l, qq in zip(draw_lengths(rng, B, BS), q)]
    window = int(rng.choice([0, 0, int(rng.integers(1, 600))]))
    sinks = int(rng.integers(0, 40)) if window > 0 and rng.random() < 0.6 else 0
    say(f"seed {seed}: B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} {kv} L={L} q={q} "
        f"window={window} sinks={sinks}")
    wl = build_general(B, Hq, Hkv, D, BS, L, q, kv=kv, seed=seed, sinks=sinks, window=window)
    check_general(wl, f"seed {seed}")


def draw_switches(rng) -> str:
    """The process-wide switches at random: the split's run cost, parking of
    mid-piece results, the workgroup combine and one kv head per wave."""
    from paged_kv_decode_06_amd import ops
    rc = int(rng.choice([0, 2, 5, 8]))
    park, wgc = int(rng.integers(0, 2)), int(rng.integers(0, 2))
    one = int(rng.random() < 0.3)
    ops.select_run_cost(rc)
    ops.select_result_parking(park)
    ops.select_share_combine(wgc)
    ops.select_unit_heads(one)
    return f"run cost {rc}, parking {park}, combine {wgc}, one head {one}"


def draw_batch(rng, B, BS):
    """Now and then a batch of 60..400 short sequences (many runs a piece)."""
    if rng.random() < 0.3:
        B = int(rng.integers(60, 400))
        return B, [int(x) for x in rng.integers(1, 80, B)]
    return B, draw_lengths(rng, B, BS)


@pytest.fixture
def switches_restored():
    from tests.test_gpu_parity import default_kernel
    yield
    default_kernel()


@pytest.mark.parametrize("seed", range(60))
def test_random_decode_step_with_switches(seed, switches_restored):
    rng = np.random.default_rng(11000 + seed)
    B, Hq, Hkv, D, BS, kv = draw_shape(rng)
    B, L = draw_batch(rng, B, BS)
    sw = draw_switches(rng)
    say(f"seed {seed}: B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} {kv}; {sw}")
    wl = build(B, Hq, Hkv, D, BS, L, kv=kv, seed=seed)
    check_step(wl, f"seed {seed}; {sw}")
    wl = build(B, Hq, Hkv, D, BS, L, kv=kv, seed=seed)
    assert_same_as_two_calls(wl, f"seed {seed}; {sw}")


@pytest.mark.parametrize("seed", range(80))
def test_random_general_attention_with_switches(seed, switches_restored):
    rng = np.random.default_rng(13000 + seed)
    B, Hq, Hkv, D, BS, kv = draw_shape(rng)
    G = Hq // Hkv
    qmax = (32 if rng.random() < 0.4 else 16) // G
    B, L0 = draw_batch(rng, B, BS)
    q = [int(rng.integers(1, qmax + 1)) for _ in range(B)]
    L = [max(l, qq) for l, qq in zip(L0, q)]
    window = int(rng.choice([0, 0, int(rng.integers(1, 600))]))
    sinks = int(rng.integers(0, 40)) if window > 0 and rng.random() < 0.6 else 0
    sw = draw_switches(rng)
    say(f"seed {seed}: B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} {kv} q<={qmax} "
        f"window={window} sinks={sinks}; {sw}")
    wl = build_general(B, Hq, Hkv, D, BS, L, q, kv=kv, seed=seed, sinks=sinks, window=window)
    check_general(wl, f"seed {seed}; {sw}")
