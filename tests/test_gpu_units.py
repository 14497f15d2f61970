"""Several kv heads per partition wave (the MFMA kernel's decode
instantiations): the unit size each configuration gets, bit-for-bit
agreement with one kv head per wave, per-head fp8 / int8 scales inside a
unit in the fused append, and the fallback when the unit does not divide
Hkv.

Bit-for-bit: a unit's scores for column n come from the MFMA chain of that
column's own kv head (the same chain one head per wave runs), and the output
adds the other heads' products with P = 0 (exact zeros).  So every share is
the same bits as with one head per wave whenever both split the work into
the same page ranges, which holds when every piece is one page (the total
page count does not exceed either grid's waves); the test checks that
precondition before comparing (with no run cost in the split, whose
extra positions would depend on the unit size).  These comparisons run with
the workgroup combine of the shares switched off: it groups the pieces of four waves, and
the two unit sizes lay out the work axis differently, so they would group
different pages (tests/test_gpu_combine.py covers the combine).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_decode_step import assert_same_as_two_calls, bits, step, twin
from tests.test_gpu_parity import DEV, build, default_kernel, say, use_kernel

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


@pytest.fixture
def no_combine():
    """Combine off, and no run cost in the split: every page its own piece."""
    ops.select_share_combine(0)
    ops.select_run_cost(0)
    yield
    ops.select_share_combine(1)
    default_kernel()


def unit_heads(wl: W.Workload) -> int:
    return ops.decode_unit_heads(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, GS.KV_KIND[wl.kv_dtype])


def waves(wl: W.Workload) -> int:
    return ops.attention_waves(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, GS.KV_KIND[wl.kv_dtype])


@pytest.mark.parametrize("name,hg", [("llama3_8b", 2), ("long_context", 2), ("mixed_70b", 2),
                                     ("fp8", 2), ("int8", 2), ("tiny", 2)])
def test_unit_heads_of_the_configurations(name, hg):
    c = W.CONFIGS[name]
    kvd = GS.KV_KIND[c.kv_dtype]
    B = c.B
    assert ops.decode_unit_heads(B, c.Hq, c.Hkv, c.D, c.BS, kvd) == hg
    use_kernel("mfma1")
    assert ops.decode_unit_heads(B, c.Hq, c.Hkv, c.D, c.BS, kvd) == 1
    use_kernel("valu")
    assert ops.decode_unit_heads(B, c.Hq, c.Hkv, c.D, c.BS, kvd) == 1


@pytest.mark.parametrize("name", ["llama3_8b", "fp8", "int8", "mixed_70b"])
def test_grid_is_the_compiled_waves_per_simd(name):
    """The persistent grid is 2 waves per SIMD with two-head units and 3
    with one head, on every CU (4 SIMDs a CU), whatever registers the
    kernels end up with: the occupancy query alone once gave one-head calls
    4 per SIMD, which ran 13-15% slower."""
    c = W.CONFIGS[name]
    kvd = GS.KV_KIND[c.kv_dtype]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert ops.attention_waves(c.B, c.Hq, c.Hkv, c.D, c.BS, kvd) == cus * 4 * 2
    use_kernel("mfma1")
    try:
        assert ops.attention_waves(c.B, c.Hq, c.Hkv, c.D, c.BS, kvd) == cus * 4 * 3
    finally:
        default_kernel()


def one_page_pieces(wl: W.Workload) -> bool:
    pages = int(sum((int(L) + wl.BS - 1) // wl.BS for L in wl.lengths))
    return pages * wl.Hkv <= waves(wl) and pages * wl.Hkv // max(unit_heads(wl), 1) <= waves(wl)


CASES = [
    # (B, Hq, Hkv, D, BS, lengths, kv)
    (3, 32, 8, 128, 16, (100, 700, 1500), "bf16"),
    (4, 16, 8, 128, 32, (1, 33, 640, 2000), "bf16"),
    (3, 64, 8, 128, 16, (17, 300, 1100), "bf16"),     # G = 8
    (3, 8, 8, 64, 16, (5, 260, 900), "bf16"),         # G = 1
    (3, 32, 8, 128, 32, (31, 500, 2100), "fp8"),
    (3, 16, 4, 64, 16, (64, 129, 1000), "fp8"),
    (3, 32, 8, 128, 32, (31, 500, 2100), "int8"),
    (3, 64, 8, 128, 16, (2, 96, 1500), "int8"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda s: f"Hq{s[1]}Hkv{s[2]}D{s[3]}BS{s[4]}{s[6]}")
def test_units_equal_one_head_bit_for_bit(case, no_combine):
    B, Hq, Hkv, D, BS, lengths, kv = case
    wl = build(B, Hq, Hkv, D, BS, lengths, kv=kv, seed=Hq + Hkv + D + BS)
    assert unit_heads(wl) > 1
    assert one_page_pieces(wl)
    GS.append_in_order(wl)
    a = GS.gpu_step(wl, append=False).clone()
    use_kernel("mfma1")
    assert one_page_pieces(wl)
    b = GS.gpu_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))
    # and against the oracle
    host = GS.HostProblem(wl)
    GS.assert_attention_close(GS.bf16_to_f64(a), host.attention(), wl.kv_dtype, f"{case}")


@pytest.mark.parametrize("case", CASES[:2] + CASES[4:6], ids=lambda s: f"Hq{s[1]}Hkv{s[2]}{s[6]}")
def test_fused_step_units_equal_one_head_bit_for_bit(case, no_combine):
    B, Hq, Hkv, D, BS, lengths, kv = case
    wl = build(B, Hq, Hkv, D, BS, lengths, kv=kv, seed=Hq + Hkv + D + BS + 1)
    assert unit_heads(wl) > 1 and one_page_pieces(wl)
    other = twin(wl)
    a = step(wl).clone()
    use_kernel("mfma1")
    assert one_page_pieces(wl)
    b = step(other)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))
    assert torch.equal(bits(wl.k_cache), bits(other.k_cache))
    assert torch.equal(bits(wl.v_cache), bits(other.v_cache))
    if wl.k_scale is not None:
        assert torch.equal(wl.k_scale.view(torch.int32), other.k_scale.view(torch.int32))
        assert torch.equal(wl.v_scale.view(torch.int32), other.v_scale.view(torch.int32))


@pytest.mark.parametrize("kv", ["fp8", "int8"])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_unit_scales_per_head(kv, G):
    """New tokens whose kv heads differ by powers of two in magnitude: each
    head of a unit opens (or joins) its block with its own scale; the fused
    step equals the stand-alone append plus attention bit for bit, and the
    oracle.  The outputs of a head whose new values were scaled up by 2^k
    are compared divided by 2^k (exact), so the bars, set for values of unit
    size, keep their meaning: a block opened by the scaled token holds the
    same codes with a scale 2^k times larger, and its output is an average
    of values at most 2^k times the unit size."""
    Hkv, BS = 8, 16
    wl = build(4, Hkv * G, Hkv, 128, BS, (1, BS + 1, 7 * BS + 9, 40 * BS), kv=kv, seed=60 + G)
    fk = torch.tensor([1.0, 8.0, 0.125, 64.0, 0.5, 16.0, 0.25, 2.0], device=DEV)[:Hkv]
    fv = fk.flip(0)
    wl.k_new.mul_(fk.view(1, Hkv, 1).to(wl.k_new.dtype))
    wl.v_new.mul_(fv.view(1, Hkv, 1).to(wl.v_new.dtype))
    assert unit_heads(wl) == 2
    host = GS.HostProblem(wl)
    out = assert_same_as_two_calls(wl, f"G{G} {kv}")
    host.append()
    ks = wl.k_scale.cpu().numpy()[host.old_blocks]
    assert np.array_equal(ks.view(np.uint32), host.ks.view(np.uint32))
    per_head = np.repeat(np.maximum(fv.cpu().numpy().astype(np.float64), 1.0), G)[None, :, None]
    GS.assert_attention_close(GS.bf16_to_f64(out) / per_head, host.attention() / per_head, kv,
                              f"G{G} {kv}")


@pytest.mark.parametrize("Hq,Hkv,hg", [(20, 5, 1), (72, 9, 1), (24, 12, 2), (48, 6, 2)])
def test_units_that_do_not_divide_fall_back(Hq, Hkv, hg):
    """An odd Hkv: one kv head per wave; Hkv = 12 or 6: units of 2."""
    wl = build(3, Hq, Hkv, 128, 16, (40, 333, 1200), seed=Hq + Hkv)
    assert unit_heads(wl) == hg
    say(f"unit heads {hg}")
    host = GS.HostProblem(wl)
    out = GS.gpu_step(wl)
    torch.cuda.synchronize()
    host.append()
    GS.assert_attention_close(GS.bf16_to_f64(out), host.attention(), wl.kv_dtype, f"Hkv{Hkv}")


# ------------------------------------------------ the generalised call --
# Two-head units serve the generalised call too when 2 G max_q <= 16.
GEN_CASES = [
    # (B, Hq, Hkv, D, BS, lengths, q_lens, kv, sinks, window)
    (3, 16, 4, 128, 16, (50, 333, 1200), (2, 1, 2), "bf16", 0, 0),        # G 4, 2 queries
    (4, 32, 8, 128, 16, (100, 700, 1500, 9), (1, 1, 1, 1), "bf16", 16, 256),  # window decode
    (3, 16, 8, 64, 32, (40, 500, 2000), (4, 4, 3), "fp8", 0, 0),         # G 2, 4 queries
    (3, 8, 8, 128, 16, (17, 300, 1100), (8, 5, 8), "int8", 16, 128),     # G 1, 8, window
]


def general_pages(wl: W.Workload) -> int:
    """Pages on the work axis: each sequence's sink and window pages."""
    n = 0
    for L, ql in zip(wl.lengths, wl.q_lens):
        L, ql = int(L), int(ql)
        pe = (L + wl.BS - 1) // wl.BS
        if wl.window <= 0:
            n += pe
            continue
        lo = max(L - ql - wl.window + 1, 0)
        pw, ps = lo // wl.BS, min((wl.sinks + wl.BS - 1) // wl.BS, pe)
        n += pe if pw <= ps else ps + (pe - pw)
    return n


@pytest.mark.parametrize("case", GEN_CASES, ids=lambda s: f"G{s[1] // s[2]}q{max(s[6])}{s[7]}w{s[9]}")
def test_general_units_equal_one_head_bit_for_bit(case, no_combine):
    """Same precondition as the decode test: every piece one page in both
    grids, so both split the work alike."""
    B, Hq, Hkv, D, BS, lengths, q_lens, kv, sinks, window = case
    from tests.test_gpu_general import build as build_general
    wl = build_general(B, Hq, Hkv, D, BS, lengths, q_lens, kv=kv, seed=B + Hq + D,
                       sinks=sinks, window=window)
    assert 2 * (Hq // Hkv) * max(q_lens) <= 16
    pages = general_pages(wl)
    assert pages * Hkv <= waves(wl) and pages * Hkv // 2 <= waves(wl)
    host = GS.GeneralHost(wl)                 # the oracle's view, before the GPU appends
    GS.append_in_order(wl)
    a = GS.general_step(wl, append=False).clone()
    use_kernel("mfma1")
    assert pages * Hkv <= waves(wl)
    b = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))
    host.append()
    GS.assert_attention_close(GS.bf16_to_f64(a)[host.rows], host.attention(), kv, f"{case}")


def test_general_one_query_equals_decode_with_units():
    """One query, no window: the generalised call is the decode call bit for
    bit with two-head units in both (same grid, same split)."""
    from tests.test_gpu_general import build as build_general
    wl = build_general(5, 32, 8, 128, 16, (1, 17, 300, 2000, 4096), (1,) * 5, seed=3)
    assert unit_heads(wl) == 2
    GS.append_in_order(wl)
    a = GS.gpu_step(wl, append=False)
    b = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))


def test_small_windowed_call_takes_one_head():
    """A windowed call whose window bounds its work to a few pages per wave
    (here at most 130 per sequence and kv head: 4 x 8 x 130 pages for 3072
    one-head waves) runs one kv head per wave: the same bits as with one head
    forced; its workspace query covers that unit size."""
    from tests.test_gpu_general import build as build_general
    wl = build_general(4, 32, 8, 128, 16, (20000, 30000, 5000, 9000), (1, 1, 1, 1), seed=3,
                       sinks=16, window=2048, poison=False)
    GS.append_in_order(wl)
    a = GS.general_step(wl, append=False).clone()
    use_kernel("mfma1")
    b = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.equal(bits(a), bits(b))
