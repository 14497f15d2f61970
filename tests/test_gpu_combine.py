"""The workgroup combine of the partition kernel's shares (GPU).

The four waves of a partition workgroup stream consecutive pieces of the
work axis; with the combine on (the default, for calls whose share rows have
at most 8 columns, or 16 with two kv heads per wave, and B <= 1024) they
merge their shares of a run in LDS, so
a run inside a workgroup's range is finished by the workgroup and a run
crossing its edge leaves one share row per workgroup.  Checked: the same
oracle bar with the combine on and off, results that differ only by
summation order, repeated calls bit for bit, runs inside and across
workgroup ranges, the generalised call, the workspace each mode needs, and
the floor/ceil split of small workloads.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_parity import (DEFAULT_RUN_COST, DEV, build, check_step, default_kernel, say,
                                   use_kernel)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


def bits(t: torch.Tensor) -> torch.Tensor:
    return t.view(torch.int16)


def twin(wl: W.Workload) -> W.Workload:
    """A second copy of a workload's tensors (same values, other memory)."""
    import copy
    o = copy.copy(wl)
    for name in ("q", "k_new", "v_new", "k_cache", "v_cache", "k_scale", "v_scale",
                 "context_lens", "block_tables", "slot_mapping", "q_start"):
        t = getattr(wl, name)
        setattr(o, name, None if t is None else t.clone())
    return o


CASES = [
    # (B, Hq, Hkv, D, BS, lengths, kv, kernel mode)
    (6, 32, 8, 128, 16, (40, 700, 1500, 3, 2600, 17), "bf16", "mfma"),   # two heads, G = 4
    (5, 16, 8, 128, 32, (33, 1, 900, 64, 2049), "fp8", "mfma"),          # two heads, G = 2
    (5, 16, 8, 64, 16, (500, 2, 1200, 77, 300), "int8", "mfma"),
    (4, 64, 8, 128, 16, (20, 1000, 2000, 5), "bf16", "mfma1"),           # one head, G = 8
    (6, 64, 8, 128, 16, (40, 700, 1500, 3, 2600, 17), "bf16", "mfma"),   # two heads, G = 8: 16 columns
    (5, 32, 4, 64, 32, (33, 1, 900, 64, 2049), "fp8", "mfma"),           # two heads, G = 8, D = 64
    (4, 32, 8, 128, 16, (20, 1000, 2000, 5), "bf16", "mfma1"),           # one head, G = 4
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"Hq{c[1]}Hkv{c[2]}D{c[3]}{c[6]}{c[7]}")
def test_combine_on_and_off_meet_the_oracle_and_agree(case):
    B, Hq, Hkv, D, BS, lengths, kv, mode = case
    use_kernel(mode)
    wl = build(B, Hq, Hkv, D, BS, lengths, kv=kv, seed=B + Hq + D)
    other = twin(wl)
    on, _ = check_step(wl, f"{case} combine on")
    ops.select_share_combine(0)
    off, _ = check_step(other, f"{case} combine off")
    # only the summation order differs: within two bf16 steps of each other
    a, b = GS.bf16_to_f64(on), GS.bf16_to_f64(off)
    assert np.all(np.abs(a - b) <= 2 * 2.0 ** -8 * np.maximum(np.abs(a), np.abs(b)) + 1e-6)


def test_repeated_calls_are_bit_identical():
    wl = build(16, 32, 8, 128, 16, np.random.default_rng(5).integers(100, 3000, 16), seed=5,
               poison=False)
    GS.append_in_order(wl)
    ws = GS.workspace_for(wl)
    first = GS.gpu_step(wl, workspace=ws, append=False).clone()
    for _ in range(3):
        again = GS.gpu_step(wl, workspace=ws, append=False)
        assert torch.equal(bits(again), bits(first))


def test_runs_inside_and_across_workgroup_ranges():
    """Many short sequences (runs inside one workgroup's range, finished in
    the workgroup, some by several waves) and a few long ones (runs across
    many ranges, left to the merge), lengths 1 .. 9000."""
    rng = np.random.default_rng(31)
    L = np.concatenate([rng.integers(1, 80, 200), rng.integers(3000, 9000, 6)])
    rng.shuffle(L)
    wl = build(len(L), 32, 8, 128, 16, L, seed=31)
    check_step(wl, "short and long runs")


@pytest.mark.parametrize("window", [0, 300])
def test_generalised_call_with_one_query(window):
    """The generalised instantiation takes the combine when its columns fit
    (one query per sequence at G <= 4): against the oracle, and without a
    window bit for bit the decode call (same split, same grouping)."""
    wl = build(5, 32, 8, 128, 16, (1, 400, 1800, 3100, 66), seed=9, poison=True)
    wl_q = W.build_workload("t", 5, 32, 8, 128, 16, list(wl.lengths), seed=9, device=DEV,
                            poison=True, q_lens=[1] * 5, window=window, sinks=4 if window else 0)
    host = GS.GeneralHost(wl_q)
    out = GS.general_step(wl_q)
    torch.cuda.synchronize()
    host.append()
    GS.assert_attention_close(GS.bf16_to_f64(out)[host.rows], host.attention(), "bf16",
                              f"window {window}")
    if window == 0:
        dec = GS.gpu_step(wl)
        torch.cuda.synchronize()
        assert torch.equal(bits(dec), bits(out))


def test_workspace_follows_the_mode():
    """Share rows are per workgroup with the combine (a quarter as many
    wave rows) and per wave without it: 8-column rows (G = 4, two heads)
    and 16-column rows with two heads (G = 8) combine; one head with 16
    columns (G = 16: its tile buffer cannot hold such a share) and more than
    1024 sequences never do."""
    kv = ops.KV_BF16
    on = ops.workspace_bytes(64, 32, 8, 128, 16, 256, kv)
    on16 = ops.workspace_bytes(256, 64, 8, 128, 16, 1024, kv)             # G = 8: 16 columns
    ops.select_share_combine(0)
    off = ops.workspace_bytes(64, 32, 8, 128, 16, 256, kv)
    off16 = ops.workspace_bytes(256, 64, 8, 128, 16, 1024, kv)
    g16_off = ops.workspace_bytes(64, 128, 8, 128, 16, 256, kv)           # G = 16, one head
    big_off = ops.workspace_bytes(2000, 32, 8, 128, 16, 64, kv)
    ops.select_share_combine(1)
    assert on < off and on16 < off16
    assert ops.workspace_bytes(64, 128, 8, 128, 16, 256, kv) == g16_off
    assert ops.workspace_bytes(2000, 32, 8, 128, 16, 64, kv) == big_off
    say("workspace bytes, Llama shape: combine", on, "per wave", off)


def balanced_split(total: int, pieces: int) -> bool:
    """Whether the partition kernels cut a work axis of `total` pages into
    `pieces` pieces of floor/ceil(total / pieces) pages (else every piece
    has ceil(total / pieces) pages and the last ones are empty)."""
    qp = -(-total // pieces)
    used = -(-total // qp)
    return total >= pieces and 16 * (pieces - used) > pieces


@pytest.mark.parametrize("mode", ["mfma", "mfma1"])
@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_balanced_split(mode, kv):
    """A batch of about 700 pages per kv head: the rounded-up split would
    leave a third of the waves idle, so the pieces are floor/ceil sized and
    every wave streams one or two pages; runs of one to 250 pages cross many
    piece (and workgroup) edges.  Against the oracle, combine on and off."""
    use_kernel(mode)
    lengths = (40, 3000, 1, 2500, 700, 4000, 17, 900)
    wl = build(len(lengths), 32, 8, 128, 16, lengths, kv=kv, seed=77)
    kvd = GS.KV_KIND[kv]
    waves = ops.attention_waves(wl.B, 32, 8, 128, 16, kvd)
    U = 8 // ops.decode_unit_heads(wl.B, 32, 8, 128, 16, kvd)
    # (the split counts each run's pages plus the run cost's positions)
    total = U * sum(-(-L // 16) + DEFAULT_RUN_COST for L in lengths if L > 0)
    assert balanced_split(total, waves), (total, waves)
    other = twin(wl)
    check_step(wl, f"balanced split {mode} {kv} combine on")
    ops.select_share_combine(0)
    check_step(other, f"balanced split {mode} {kv} combine off")


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_sixteen_column_combine_at_the_batch_limit(kv):
    """B = 1024 sequences at G = 8 with two kv heads per wave: 16-column
    share slots, the largest batch that combines, whose LDS (prefix sums,
    lengths, four waves' tiles and slots) still leaves two workgroups per
    CU.  Lengths 1 .. 300 (runs inside and across workgroup ranges)."""
    B = 1024
    L = np.random.default_rng(41).integers(1, 300, B)
    kvd = GS.KV_KIND[kv]
    BS = 16 if kv == "bf16" else 32
    assert ops.decode_unit_heads(B, 64, 8, 128, BS, kvd) == 2
    on = ops.workspace_bytes(B, 64, 8, 128, BS, 32, kvd)
    ops.select_share_combine(0)
    off = ops.workspace_bytes(B, 64, 8, 128, BS, 32, kvd)
    ops.select_share_combine(1)
    assert on < off                                   # the combine is taken
    wl = build(B, 64, 8, 128, BS, L, kv=kv, seed=41)
    check_step(wl, f"B{B} G8 {kv} 16-column combine")
