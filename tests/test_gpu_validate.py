"""pkv_validate_inputs: the debug check of the device-resident contract of
the attention call (lengths in [1, MBS * BS], block ids of the used pages in
[0, NB), positive finite scales of those blocks for one-byte caches).  It
checks the attention's inputs, so each workload first gets its step's
append (a token that opens a block sets that block's scale).  A clean
workload and the test generator's poison (NaN in free blocks, -1 in unused
table entries, NaN scales of unused blocks) pass; each planted violation is
reported with the first offending sequence and page."""
from __future__ import annotations

import math

import pytest
import torch

from paged_kv_decode_06_amd import ops
from tests import gpu_support as GS
from tests.test_gpu_parity import build

pytestmark = pytest.mark.gpu

PKV_ERR_INPUT = -7


def appended(wl):
    ops.kv_append(wl.k_new, wl.v_new, wl.slot_mapping, wl.k_cache, wl.v_cache, wl.k_scale,
                  wl.v_scale)
    return wl


def validate(wl):
    ops.validate_inputs(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                        wl.scale, torch.empty_like(wl.q), wl.k_scale, wl.v_scale,
                        GS.workspace_for(wl))


def rejects(wl, *fragments):
    with pytest.raises(ops.PkvError) as e:
        validate(wl)
    assert e.value.status == PKV_ERR_INPUT
    for f in fragments:
        assert f in str(e.value), str(e.value)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
def test_clean_and_poisoned_workloads_pass(kv):
    wl = appended(build(5, 16, 4, 128, 16, (1, 16, 17, 300, 2000), kv=kv, seed=3, poison=True))
    validate(wl)


def test_length_outside_the_table():
    wl = appended(build(4, 8, 2, 64, 16, (5, 40, 70, 9), seed=4))
    wl.context_lens[2] = wl.MBS * wl.BS + 1
    wl.context_lens[3] = 0
    rejects(wl, "sequence 2", "context length")


def test_zero_length_is_reported():
    wl = appended(build(3, 8, 2, 64, 16, (5, 40, 70), seed=5))
    wl.context_lens[1] = 0
    rejects(wl, "sequence 1", "context length 0")


def test_block_id_out_of_range():
    wl = appended(build(3, 8, 2, 64, 16, (5, 40, 70), seed=6))
    wl.block_tables[2, 3] = wl.NB          # page 3 of 5 used pages
    wl.block_tables[1, 0] = -1
    rejects(wl, "sequence 1, page 0", "block id -1")


def test_unused_table_entries_are_not_checked():
    wl = appended(build(2, 8, 2, 64, 16, (5, 17), seed=7))
    wl.block_tables[0, 1:] = 1 << 30        # past ceil(5 / 16) = 1 page
    validate(wl)


@pytest.mark.parametrize("kv,which,value", [("fp8", "K", math.nan), ("int8", "V", 0.0),
                                            ("fp8", "V", -1.0), ("int8", "K", math.inf)])
def test_bad_scale_of_a_used_block(kv, which, value):
    wl = appended(build(3, 16, 4, 128, 32, (40, 100, 33), kv=kv, seed=8))
    blk = int(wl.block_tables_np[1, 2])    # sequence 1, page 2 (of 4)
    (wl.k_scale if which == "K" else wl.v_scale)[blk, 3] = value
    rejects(wl, "sequence 1, page 2", f"a {which} scale")
