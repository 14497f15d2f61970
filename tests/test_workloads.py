"""The seeded input recipes (CPU only): lengths, pools, tables and slots."""
import math

import numpy as np
import pytest

from paged_kv_decode_06_amd import workloads as W


def lengths(name):
    cfg = W.CONFIGS[name]
    return W.draw_lengths(cfg, np.random.default_rng(cfg.seed))


def test_length_recipes():
    assert list(lengths("tiny")) == [1, 17, 33, 100]
    L1 = lengths("llama3_8b")
    assert L1.shape == (64,) and L1.min() >= 512 and L1.max() <= 4096
    assert (lengths("long_context") == 131072).all()
    L3 = lengths("mixed_70b")
    assert L3.shape == (256,) and L3.min() == 1 and L3.max() <= 16384
    assert (L3 == 1).sum() >= 13                        # 5% forced to length 1
    assert 1000 < np.median(L3) < 2200                  # lognormal median 1500
    L4 = lengths("fp8")
    assert L4.shape == (128,) and L4.max() <= 16384
    assert ((L4 - 1) % 32 == 0).sum() == 32             # exactly 25% open a block


def test_lengths_are_deterministic():
    for name in W.CONFIG_ORDER:
        assert np.array_equal(lengths(name), lengths(name))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_pool_tables_and_slots(kv):
    BS = 16 if kv == "bf16" else 32
    L = [1, 15, 16, 17, 100, 257]
    wl = W.build_workload("t", 6, 8, 2, 64, BS, L, kv_dtype=kv, seed=3, poison=True)
    pages = [math.ceil(x / BS) for x in L]
    assert wl.NB == math.ceil(1.1 * sum(pages))
    used = wl.block_tables_np[wl.block_tables_np >= 0]
    assert len(used) == sum(pages) and len(set(used.tolist())) == len(used)   # no block shared
    for b, n in enumerate(pages):
        assert (wl.block_tables_np[b, :n] >= 0).all() and (wl.block_tables_np[b, n:] == -1).all()
        pos = L[b] - 1
        assert wl.slot_mapping_np[b] == wl.block_tables_np[b, pos // BS] * BS + pos % BS
    # the slot about to be appended is poisoned, the pre-filled history is not
    k = W.cache_host(wl.k_cache)
    for b in range(6):
        blk, off = divmod(int(wl.slot_mapping_np[b]), BS)
        if kv == "bf16":
            assert (k[blk, off] == W.BF16_NAN_BITS).all()
        else:
            assert (k[blk, off] == W.E4M3FN_NAN_CODE).all()
        if L[b] > 1:
            blk0 = wl.block_tables_np[b, 0]
            assert (k[blk0, 0] != (W.BF16_NAN_BITS if kv == "bf16" else W.E4M3FN_NAN_CODE)).all()


def test_verify_recipes_query_counts():
    """Verify workloads take q_len tokens per sequence, fewer where the
    history is shorter (the 70B mix has sequences of length 1)."""
    for name, G, q in (("llama3_8b_verify4", 4, 4), ("mixed_70b_verify4", 8, 4)):
        cfg = W.CONFIGS[name]
        assert cfg.Hq // cfg.Hkv == G and cfg.q_len == q
        wl = W.make_config_workload(name)
        L = np.asarray(wl.lengths)
        assert np.array_equal(wl.q_lens, np.minimum(q, L))
        assert np.array_equal(L, lengths(name))
        assert wl.q_start_np[-1] == wl.q_lens.sum() == wl.q.shape[0]
    assert (wl.q_lens == 1).sum() >= 13
