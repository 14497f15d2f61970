"""GPU parity of the generalised attention (pkv_paged_attention): several
query tokens per sequence with the bottom-right causal mask, and a sliding
window with attention sinks, against the fp64 oracle on the same seeded
inputs, through the C ABI.  Same bars as the decode call (bf16 cache:
|gpu - ref| <= 4e-3 + 8e-3 |ref|; fp8: <= 3e-2 absolute); appends bit-exact.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from paged_kv_decode_06_amd import workloads as W
from tests import gpu_support as GS
from tests.test_gpu_parity import DEV, default_kernel, say, use_kernel

pytestmark = pytest.mark.gpu


def build(B, Hq, Hkv, D, BS, lengths, q_lens, kv="bf16", seed=0, poison=True, sinks=0,
          window=0, scale=None):
    say(f"case B={B} Hq={Hq} Hkv={Hkv} D={D} BS={BS} kv={kv} L={list(lengths)[:6]} "
        f"q_lens={list(q_lens)[:6]} sinks={sinks} window={window} seed={seed}")
    return W.build_workload("t", B, Hq, Hkv, D, BS, list(lengths), kv_dtype=kv, seed=seed,
                            device=DEV, poison=poison, q_lens=list(q_lens), window=window,
                            sinks=sinks, scale=scale)


def check(wl, what=""):
    host = GS.GeneralHost(wl)
    out = GS.general_step(wl)
    torch.cuda.synchronize()
    host.append()
    assert np.array_equal(W.cache_host(wl.k_cache)[host.old_blocks], host.k), f"{what}: K append"
    assert np.array_equal(W.cache_host(wl.v_cache)[host.old_blocks], host.v), f"{what}: V append"
    ref = host.attention()
    GS.assert_attention_close(GS.bf16_to_f64(out), ref, wl.kv_dtype, what)
    return out, ref


CASES = [
    # (B, Hq, Hkv, D, BS, lengths, q_lens, kv, sinks, window)
    (3, 8, 2, 64, 16, (7, 20, 45), (1, 3, 4), "bf16", 0, 0),
    (4, 32, 8, 128, 16, (40, 513, 1000, 2047), (4, 4, 4, 4), "bf16", 0, 0),
    (3, 16, 8, 128, 16, (9, 300, 777), (8, 5, 2), "bf16", 0, 0),           # G = 2
    (2, 16, 16, 64, 32, (100, 900), (16, 9), "bf16", 0, 0),                # G = 1, 16 queries
    (3, 16, 2, 128, 32, (2, 70, 1500), (2, 1, 2), "bf16", 0, 0),            # G = 8
    (3, 8, 2, 64, 16, (7, 20, 45), (1, 3, 4), "bf16", 2, 9),
    (3, 32, 8, 128, 16, (700, 1500, 3000), (1, 1, 1), "bf16", 4, 256),      # decode + window
    (2, 32, 8, 128, 16, (4000, 9000), (4, 2), "bf16", 16, 1000),            # window off a page edge
    (2, 32, 8, 128, 16, (4000, 9000), (1, 1), "bf16", 0, 1024),             # window on page edges
    (3, 16, 4, 128, 32, (40, 700, 2000), (2, 4, 3), "fp8", 0, 0),
    (3, 16, 4, 128, 32, (40, 700, 2000), (2, 4, 3), "fp8", 3, 100),
    (2, 8, 2, 64, 16, (50, 400), (4, 2), "fp8", 1, 33),
    (3, 16, 4, 128, 32, (40, 700, 2000), (2, 4, 3), "int8", 0, 0),
    (2, 32, 8, 128, 16, (600, 3000), (4, 1), "int8", 8, 300),
    (3, 128, 8, 128, 16, (700, 1500, 3000), (1, 1, 1), "bf16", 4, 256),    # G = 16, window
    (2, 64, 4, 64, 32, (500, 2000), (1, 1), "fp8", 0, 0),                  # G = 16
    # two 16-column tiles (G * max_q in 17..32, one kv head per wave)
    (3, 64, 8, 128, 16, (9, 700, 2500), (4, 3, 4), "bf16", 0, 0),           # G = 8, 4 queries
    (3, 32, 8, 128, 16, (40, 513, 3000), (8, 5, 1), "bf16", 2, 300),        # G = 4, 8 queries
    (2, 16, 1, 128, 32, (100, 4000), (2, 2), "bf16", 0, 0),                 # G = 16, 2 queries
    (2, 16, 8, 64, 16, (60, 900), (16, 11), "bf16", 0, 0),                  # G = 2, 16 queries
    (2, 4, 4, 64, 32, (50, 1000), (32, 17), "bf16", 4, 40),                 # G = 1, 32 queries
    (3, 32, 8, 128, 16, (5, 300, 1200), (5, 6, 6), "bf16", 0, 0),           # G = 4: 24 columns
    (3, 64, 8, 64, 16, (3, 77, 1200), (3, 3, 2), "bf16", 1, 64),            # G = 8: 24 columns
    (3, 64, 8, 128, 32, (40, 700, 2000), (4, 2, 4), "fp8", 0, 0),
    (3, 64, 8, 128, 32, (40, 700, 2000), (4, 4, 3), "int8", 3, 100),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[7]}-D{c[3]}G{c[1]//c[2]}-ql{max(c[6])}-S{c[8]}W{c[9]}")
def test_general_attention_matches_oracle(case):
    B, Hq, Hkv, D, BS, L, ql, kv, S, Wn = case
    wl = build(B, Hq, Hkv, D, BS, L, ql, kv=kv, seed=B + D + BS + S, sinks=S, window=Wn)
    check(wl, str(case))


@pytest.mark.parametrize("cols", [16, 32], ids=["one-tile", "two-tiles"])
def test_every_variant_with_queries_and_a_window(cols):
    """Every (D, BS, G, dtype) instantiation with the most queries it takes
    in one 16-column tile, then in two."""
    import itertools
    for D, BS, G, kv in itertools.product((64, 128), (16, 32), (1, 2, 4, 8, 16),
                                          ("bf16", "fp8", "int8")):
        Hkv = 2
        q = cols // G
        wl = build(3, Hkv * G, Hkv, D, BS, (q, BS + q + 3, 9 * BS + 5), (q, q, max(1, q // 2)),
                   kv=kv, seed=D + BS + G, sinks=2, window=BS + 5)
        check(wl, f"D{D} BS{BS} G{G} {kv} q{q}")


def test_one_query_no_window_is_the_decode_call_bit_for_bit():
    """(With one kv head per wave in both calls, so the two split the work
    alike; several heads per wave are checked against one in test_gpu_units.)"""
    wl = build(5, 32, 8, 128, 16, (1, 17, 300, 2000, 4096), (1,) * 5, seed=3)
    GS.append_in_order(wl)
    use_kernel("mfma1")
    try:
        a = GS.gpu_step(wl, append=False)
        b = GS.general_step(wl, append=False)
        torch.cuda.synchronize()
    finally:
        default_kernel()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_wide_window_and_all_sinks_equal_the_full_history_bit_for_bit():
    wl = build(3, 16, 4, 128, 16, (50, 333, 1200), (2, 3, 4), seed=4, poison=False)
    GS.append_in_order(wl)
    full = GS.general_step(wl, append=False).clone()
    wide = GS.general_step(wl, window=1200, sinks=0, append=False).clone()
    sinks = GS.general_step(wl, window=5, sinks=1200, append=False)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), wide.view(torch.int16))
    assert torch.equal(full.view(torch.int16), sinks.view(torch.int16))


def test_window_of_one_returns_the_value_at_the_limit():
    wl = build(3, 8, 2, 64, 16, (9, 30, 50), (2, 4, 3), seed=5, poison=True)
    out = GS.general_step(wl, window=1, sinks=0).float().cpu().numpy()
    v = wl.v_cache.float().cpu().numpy()
    for b in range(3):
        L, r0, ql = int(wl.lengths[b]), int(wl.q_start_np[b]), int(wl.q_lens[b])
        for i in range(ql):
            t = L - ql + i
            blk = wl.block_tables_np[b, t // 16]
            for h in range(8):
                assert np.array_equal(out[r0 + i, h], v[blk, t % 16, h // 4])


def test_pages_outside_the_window_are_never_read():
    """Block-table entries of pages no query sees are set to -1 and those
    blocks are filled with NaN: the output is unchanged and finite."""
    wl = build(2, 32, 8, 128, 16, (3000, 5000), (2, 3), seed=6, poison=False, sinks=16,
               window=700)
    GS.append_in_order(wl)
    a = GS.general_step(wl, append=False).clone()
    torch.cuda.synchronize()
    bt = wl.block_tables_np.copy()
    for b in range(2):
        L, ql = int(wl.lengths[b]), int(wl.q_lens[b])
        lo = L - ql - 700 + 1
        for j in range(1, lo // 16):                 # page 0 holds the sinks
            wl.k_cache[int(bt[b, j])] = float("nan")
            wl.v_cache[int(bt[b, j])] = float("nan")
            bt[b, j] = -1
    wl.block_tables = torch.from_numpy(bt).to(DEV)
    b_ = GS.general_step(wl, append=False)
    torch.cuda.synchronize()
    assert torch.isfinite(b_.float()).all()
    assert torch.equal(a.view(torch.int16), b_.view(torch.int16))


@pytest.mark.parametrize("Hq", [16, 32, 64], ids=["G2-units", "G4-one-tile", "G8-two-tiles"])
def test_a_sequence_without_queries(Hq):
    """q_start may give a sequence no queries: it takes no rows, and every
    other sequence's output is bit for bit that of the call where it has
    them (the work split depends on the lengths only)."""
    wl = build(3, Hq, 8, 128, 16, (300, 900, 2000), (2, 3, 4), seed=8)
    GS.append_in_order(wl)
    full = GS.general_step(wl, append=False).clone()
    keep = torch.from_numpy(np.r_[0:2, 5:9]).to(DEV)      # sequence 1's rows 2..4 dropped
    q = wl.q.index_select(0, keep).contiguous()
    q_start = torch.tensor([0, 2, 2, 6], dtype=torch.int32, device=DEV)
    out = torch.empty_like(q)
    n = ops.attention_workspace_bytes(3, Hq, 8, 128, 16, wl.MBS, ops.KV_BF16, 4)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ops.paged_attention(q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens, wl.scale,
                        out, q_start=q_start, max_q_len=4, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), full.index_select(0, keep).view(torch.int16))


@pytest.mark.parametrize("name", ["llama3_8b_verify4", "long_context_window", "mixed_70b_verify4"])
def test_full_configuration(name):
    """The full-size generalised workloads: every query row of every sequence
    against the oracle."""
    say(f"config {name}")
    wl = W.make_config_workload(name, device=DEV, poison=True)
    host = GS.GeneralHost(wl)
    out = GS.general_step(wl)
    torch.cuda.synchronize()
    host.append()
    idx = torch.from_numpy(host.old_blocks).to(DEV)
    assert np.array_equal(W.cache_host(wl.k_cache.index_select(0, idx)), host.k)
    assert np.array_equal(W.cache_host(wl.v_cache.index_select(0, idx)), host.v)
    ref = host.attention()
    gpu = GS.bf16_to_f64(out)[host.rows]
    GS.assert_attention_close(gpu, ref, wl.kv_dtype, name)
    say(name, GS.error_report(gpu, ref, wl.kv_dtype))


def test_unsupported_query_counts_are_rejected():
    wl = build(2, 16, 2, 64, 16, (10, 20), (2, 5), seed=7)
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(wl.q)
    with pytest.raises(ops.PkvError) as e:          # G = 8: at most 4 queries
        ops.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                            wl.scale, out, q_start=wl.q_start, max_q_len=5, workspace=ws)
    assert e.value.status == -3
    assert ops.attention_workspace_bytes(2, 16, 2, 64, 16, wl.MBS, 0, 5) == 0
    assert ops.attention_workspace_bytes(2, 16, 2, 64, 16, wl.MBS, 0, 4) > 0
