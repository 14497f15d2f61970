"""Pins for the fp64 oracle, checked against things other than itself.

Each test names the fact it checks and where that fact comes from: the
pages ("Decode Phase Attention Forward Pass", the "Decode Phase" glossary,
"tiny-vllm part 5", "Prefill Forward Prefix Caching Explained"), a closed
form, a library routine (numpy, torch SDPA, torch's float8_e4m3fn), or the
OCP 8-bit floating point definition.  CPU only.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from paged_kv_decode_06_amd import workloads as W
from tests import brute


# ---------------------------------------------------------------- helpers ---

def host_step(wl: W.Workload):
    """Host copies of a workload after the oracle's append of this step's token."""
    k = W.cache_host(wl.k_cache).copy()
    v = W.cache_host(wl.v_cache).copy()
    ks = None if wl.k_scale is None else wl.k_scale.cpu().numpy().copy()
    vs = None if wl.v_scale is None else wl.v_scale.cpu().numpy().copy()
    oracle.kv_append(W.bf16_bits(wl.k_new), W.bf16_bits(wl.v_new), wl.slot_mapping_np,
                     k, v, ks, vs)
    return dict(q=W.bf16_bits(wl.q), k=k, v=v, bt=wl.block_tables_np,
                cl=wl.lengths.astype(np.int32), ks=ks, vs=vs, scale=wl.scale)


def run_oracle(h, **kw):
    return oracle.paged_decode_attention(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"],
                                         k_scale=h["ks"], v_scale=h["vs"], **kw)


def small(B=3, Hq=8, Hkv=2, D=64, BS=16, lengths=(5, 16, 40), kv="bf16", seed=7, poison=False,
          NB=None, scale=None):
    return W.build_workload("t", B, Hq, Hkv, D, BS, list(lengths), kv_dtype=kv, seed=seed,
                            NB=NB, scale=scale, poison=poison)


SHAPES = [
    # (B, Hq, Hkv, D, BS, lengths, kv)
    (4, 8, 2, 64, 16, (1, 17, 33, 100), "bf16"),     # the tiny configuration's shapes
    (3, 4, 4, 64, 16, (2, 31, 64), "bf16"),          # G = 1 (plain multi-head)
    (2, 8, 4, 128, 16, (15, 49), "bf16"),            # G = 2
    (2, 8, 1, 128, 32, (33, 97), "bf16"),            # G = 8 (multi-query)
    (3, 16, 2, 128, 32, (1, 32, 65), "fp8"),         # fp8, G = 8
    (2, 8, 2, 64, 16, (16, 77), "fp8"),              # fp8, G = 4
    (2, 32, 2, 64, 16, (9, 70), "bf16"),             # G = 16
]


# ------------------------------------------------------ scalar formats ----

def test_bf16_widening_known_values():
    # bf16 = the upper 16 bits of an IEEE binary32
    cases = {0x3F80: 1.0, 0xC000: -2.0, 0x0000: 0.0, 0x3E80: 0.25,
             0x0001: 2.0 ** -133, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x4049: 3.140625}
    lib = oracle._load()
    for bits, val in cases.items():
        assert lib.pkvo_bf16_to_f64(bits) == val


def test_e4m3fn_decode_matches_library_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_decode(codes)
    lib = brute.e4m3fn_to_f64_torch(codes)
    assert np.array_equal(np.isnan(mine), np.isnan(lib))
    ok = ~np.isnan(lib)
    assert np.array_equal(mine[ok], lib[ok])
    # only S.1111.111 is NaN in the "fn" variant: two codes
    assert np.isnan(mine).sum() == 2 and np.isnan(mine[0x7F]) and np.isnan(mine[0xFF])


def test_e4m3fn_spec_limits():
    # OCP OFP8 E4M3: max normal S.1111.110 = 448, min normal S.0001.000 = 2^-6,
    # max subnormal S.0000.111 = 0.875 * 2^-6, min subnormal S.0000.001 = 2^-9
    d = oracle.e4m3fn_decode(np.array([0x7E, 0x08, 0x07, 0x01, 0x38, 0xB8, 0x80], np.uint8))
    assert list(d[:6]) == [448.0, 2.0 ** -6, 0.875 * 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]
    assert d[6] == 0.0 and math.copysign(1.0, d[6]) == -1.0


def test_e4m3fn_encode_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = oracle.e4m3fn_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def test_e4m3fn_encode_ties_to_even_and_saturation():
    pos = oracle.e4m3fn_decode(np.arange(0, 0x7F, dtype=np.uint8))  # 0 .. 448 ascending
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # exact in fp32
    enc = oracle.e4m3fn_encode(mids).astype(int)
    lo = np.arange(0, 0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)  # tie goes to the even code
    assert np.array_equal(enc, expect)
    # just above / below a midpoint round to the nearer code
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    assert np.array_equal(oracle.e4m3fn_encode(up).astype(int), lo + 1)
    assert np.array_equal(oracle.e4m3fn_encode(dn).astype(int), lo)
    # saturation: anything at or beyond 448 in magnitude is +-448
    big = np.array([448, 449, 464, 480, 1e6, 3.0e38, -448, -500, -1e30], np.float32)
    assert list(oracle.e4m3fn_encode(big)) == [0x7E] * 6 + [0xFE] * 3
    # sign of zero and of values that round to zero
    tiny = np.array([0.0, -0.0, 2.0 ** -11, -(2.0 ** -11), 2.0 ** -10, -(2.0 ** -10)], np.float32)
    assert list(oracle.e4m3fn_encode(tiny)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]


def test_e4m3fn_encode_matches_library_on_clamped_values():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * 50,
        rng.standard_normal(20000).astype(np.float32) * 0.01,
        (rng.uniform(-448, 448, 20000)).astype(np.float32),
    ])
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode(x), lib)


# --------------------------------------------------------- attention ------

@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}Hq{s[1]}Hkv{s[2]}D{s[3]}BS{s[4]}{s[6]}")
def test_oracle_matches_dense_bruteforce_and_library(shape):
    B, Hq, Hkv, D, BS, lengths, kv = shape
    wl = small(B, Hq, Hkv, D, BS, lengths, kv=kv, seed=B * 100 + D)
    h = host_step(wl)
    ref = run_oracle(h)
    npy = brute.dense_attention_numpy(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"], h["ks"], h["vs"])
    sdpa = brute.dense_attention_torch_sdpa(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"], h["ks"], h["vs"])
    assert np.allclose(ref, npy, rtol=1e-12, atol=1e-13)
    assert np.allclose(ref, sdpa, rtol=1e-10, atol=1e-12)


def test_tiny_configuration_against_bruteforce():
    wl = W.make_config_workload("tiny")
    h = host_step(wl)
    ref = run_oracle(h)
    npy = brute.dense_attention_numpy(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"])
    assert np.allclose(ref, npy, rtol=1e-12, atol=1e-13)
    # the tiny lengths append at offsets 0, 0, 0, 3: three of four open a block
    assert list((wl.lengths - 1) % wl.BS) == [0, 0, 0, 3]


def test_worked_example_closed_form():
    """Hand-built case: D=2, BS=2, history of 3 tokens in blocks [3, 0].
    Scores scale*<q,k_t> = 0, 1, 2 -> weights e^s / (1 + e + e^2)."""
    D, BS, NB = 2, 2, 4
    f = lambda a: np.array(a, np.float32).view(np.uint32).astype(np.uint64) >> 16
    bits = lambda a: f(a).astype(np.uint16)
    q = bits([[[1.0, 0.0]]])                           # [1,1,2]
    k = np.zeros((NB, BS, 1, D), np.uint16)
    v = np.zeros((NB, BS, 1, D), np.uint16)
    # token 0 -> block 3 slot 0, token 1 -> block 3 slot 1, token 2 -> block 0 slot 0
    for t, (blk, off) in enumerate([(3, 0), (3, 1), (0, 0)]):
        k[blk, off, 0] = bits([float(t), 5.0])
        v[blk, off, 0] = bits([2.0 ** t, -float(t)])
    k[0, 1, 0] = bits([100.0, 100.0])                  # past the length: must be ignored
    v[0, 1, 0] = bits([1e4, 1e4])
    bt = np.array([[3, 0]], np.int32)
    cl = np.array([3], np.int32)
    out = oracle.paged_decode_attention(q, k, v, bt, cl, 1.0)
    e = math.e
    Z = 1 + e + e * e
    w = np.array([1, e, e * e]) / Z
    assert np.allclose(out[0, 0], [w @ [1, 2, 4], w @ [0, -1, -2]], rtol=1e-15, atol=0)


def test_block_permutation_invariance_is_bitwise():
    """Paging is only a mapping ("Decode Phase" glossary, PagedAttention entry):
    relabelling physical blocks must not change a single bit of the result."""
    for kv in ("bf16", "fp8"):
        wl = small(3, 8, 2, 64, 16, (20, 47, 64), kv=kv, seed=3, NB=12)
        h = host_step(wl)
        ref = run_oracle(h)
        perm = np.random.default_rng(5).permutation(wl.NB)
        inv = np.argsort(perm)
        h2 = dict(h)
        h2["k"] = h["k"][inv]          # block p moves to slot perm[p]
        h2["v"] = h["v"][inv]
        if h["ks"] is not None:
            h2["ks"] = h["ks"][inv]
            h2["vs"] = h["vs"][inv]
        bt = h["bt"].copy()
        bt[bt >= 0] = perm[bt[bt >= 0]]
        h2["bt"] = bt
        assert np.array_equal(run_oracle(h2), ref)


def test_length_one_returns_first_value_exactly():
    """context_lens counts the appended token, so L=1 attends to that token
    alone: softmax of one element is 1 and out = v_0."""
    wl = small(2, 8, 2, 64, 16, (1, 1), seed=9)
    h = host_step(wl)
    out = run_oracle(h)
    v_new = brute.bf16_bits_to_f64(W.bf16_bits(wl.v_new))   # [B, Hkv, D]
    G = wl.G
    for b in range(2):
        for hq in range(wl.Hq):
            assert np.array_equal(out[b, hq], v_new[b, hq // G])


def test_identical_keys_give_mean_of_values():
    wl = small(2, 4, 2, 64, 16, (21, 50), seed=4, poison=True)
    h = host_step(wl)
    # overwrite every key with one row: all scores equal, weights uniform
    k = h["k"].copy()
    k[...] = k[wl.block_tables_np[0, 0], 0, 0][None, None, None, :]
    h["k"] = k
    out = run_oracle(h)
    Vf = brute.dequant_cache(h["v"], None)
    for b in range(2):
        L = int(h["cl"][b])
        V = brute.gather_history(Vf, h["bt"][b], L, wl.BS)
        for hq in range(wl.Hq):
            assert np.allclose(out[b, hq], V[:, hq // wl.G].mean(axis=0), rtol=1e-13, atol=1e-15)
    # scale = 0 has the same effect with the original keys
    h["k"] = host_step(wl)["k"]
    h["scale"] = 0.0
    out0 = run_oracle(h)
    for b in range(2):
        L = int(h["cl"][b])
        V = brute.gather_history(Vf, h["bt"][b], L, wl.BS)
        assert np.allclose(out0[b, 0], V[:, 0].mean(axis=0), rtol=1e-13, atol=1e-15)


def test_weights_are_a_distribution_over_the_history_only():
    wl = small(3, 8, 2, 64, 16, (3, 16, 70), seed=12)
    h = host_step(wl)
    _, w = run_oracle(h, return_weights=True)
    for b in range(3):
        L = int(h["cl"][b])
        assert (w[b, :, :L] >= 0).all()
        assert np.allclose(w[b, :, :L].sum(axis=1), 1.0, rtol=0, atol=1e-15 * L + 1e-15)
        assert (w[b, :, L:] == 0).all()


def test_masked_result_differs_from_zero_padded_gather():
    """The first page's closing caveat: zero-padding shorter sequences to the
    longest length lets the pads take softmax weight.  The oracle must match
    the masked definition and differ from the padded one for short rows."""
    wl = small(3, 8, 2, 64, 16, (4, 30, 120), seed=21)
    h = host_step(wl)
    ref = run_oracle(h)
    npy = brute.dense_attention_numpy(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"])
    pad = brute.zero_padded_attention_numpy(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"])
    assert np.allclose(ref, npy, rtol=1e-12, atol=1e-13)
    assert np.allclose(ref[2], pad[2], rtol=1e-12, atol=1e-13)      # the longest row has no pad
    assert np.abs(ref[0] - pad[0]).max() > 1e-2                      # 116 pads steal weight


def test_bottom_right_causal_mask_reduces_to_no_mask_for_one_query():
    """"Prefill Forward Prefix Caching Explained", the causal-mask section:
    query i sees key j iff j <= i + (kv_len - q_len).  With q_len = 1 (decode)
    the single query sees every key j < kv_len, so the masked dense result
    equals the unmasked one."""
    wl = small(2, 8, 2, 64, 16, (9, 57), seed=2)
    h = host_step(wl)
    ref = run_oracle(h)
    q = brute.bf16_bits_to_f64(h["q"])
    Kf = brute.dequant_cache(h["k"], None)
    Vf = brute.dequant_cache(h["v"], None)
    for b in range(2):
        L = int(h["cl"][b])
        K = np.repeat(brute.gather_history(Kf, h["bt"][b], L, wl.BS), wl.G, axis=1)
        V = np.repeat(brute.gather_history(Vf, h["bt"][b], L, wl.BS), wl.G, axis=1)
        q_len, i = 1, 0
        allowed = np.arange(L) <= i + (L - q_len)
        assert allowed.all()
        s = np.einsum("hd,thd->ht", q[b], K) * float(np.float32(h["scale"]))
        s = np.where(allowed[None, :], s, -np.inf)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        w /= w.sum(axis=1, keepdims=True)
        assert np.allclose(ref[b], np.einsum("ht,thd->hd", w, V), rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("t_star", [0, 15, 16, 31, 47, 63, 64, 99])
def test_needle_selects_one_position(t_star):
    """K[t*] = c * q_h with c large: the softmax limit puts all weight on t*,
    so out -> v_{t*} for that head.  Sweeps first/last/partial blocks."""
    wl = small(1, 4, 1, 64, 16, (100,), seed=5, NB=9)
    h = host_step(wl)
    q = brute.bf16_bits_to_f64(h["q"])[0, 0]
    blk, off = h["bt"][0, t_star // 16], t_star % 16
    k = h["k"].copy()
    needle = (q * 8.0).astype(np.float32)      # exact in bf16: q is bf16, *8 is exact
    k[blk, off, 0] = (needle.view(np.uint32) >> 16).astype(np.uint16)
    h["k"] = k
    out = run_oracle(h)
    v = brute.bf16_bits_to_f64(h["v"][blk, off, 0])
    # weight of every other token is e^{s_t - s*} with s* - s_t >= ~ 8|q|^2/8 - ...
    assert np.allclose(out[0, 0], v, atol=1e-6)


@pytest.mark.parametrize("page", [0, 1, 3, 6])
def test_page_marker_counts_tokens_on_one_page(page):
    """scale = 0 and V = 64 on one page, 0 elsewhere: out = 64 * (tokens of the
    history on that page) / L.  A dropped or doubled page changes the count."""
    L = 100
    wl = small(1, 2, 1, 64, 16, (L,), seed=6, NB=10)
    h = host_step(wl)
    h["scale"] = 0.0
    v = np.zeros_like(h["v"])
    sixty_four = np.uint16(0x4280)                 # 64.0 in bf16
    v[h["bt"][0, page]] = sixty_four
    h["v"] = v
    out = run_oracle(h)
    on_page = min(16, L - 16 * page)
    assert np.allclose(out[0], 64.0 * on_page / L, rtol=1e-14, atol=0)


def test_nan_poison_outside_history_is_never_read():
    for kv in ("bf16", "fp8"):
        clean = small(3, 8, 2, 64, 16, (5, 16, 37), kv=kv, seed=8, NB=10)
        dirty = small(3, 8, 2, 64, 16, (5, 16, 37), kv=kv, seed=8, NB=10, poison=True)
        hc, hd = host_step(clean), host_step(dirty)
        # poisoned bytes are really there
        if kv == "bf16":
            assert np.isnan(brute.bf16_bits_to_f64(hd["k"])).any()
        else:
            assert (hd["k"] == W.E4M3FN_NAN_CODE).any() and np.isnan(hd["ks"]).any()
        oc, od = run_oracle(hc), run_oracle(hd)
        assert np.isfinite(od).all()
        assert np.array_equal(oc, od)


def test_unused_table_entries_and_zero_length():
    wl = small(2, 4, 2, 64, 16, (3, 40), seed=10)
    h = host_step(wl)
    assert (h["bt"][0, 1:] == -1).all()          # entries past the history are -1
    ref = run_oracle(h)
    h["cl"] = np.array([0, 40], np.int32)         # no history: defined as 0
    out = run_oracle(h)
    assert (out[0] == 0).all() and np.array_equal(out[1], ref[1])


def test_fp8_attention_uses_scaled_codes():
    """fp8 cache: value = e4m3fn(code) * scale[block, head].  Multiplying one
    block's V scale by 2 doubles that block's V contribution: the same as
    attending over doubled V values."""
    wl = small(1, 8, 2, 64, 32, (70,), kv="fp8", seed=13, NB=4)
    h = host_step(wl)
    blk = h["bt"][0, 1]
    h2 = dict(h)
    h2["vs"] = h["vs"].copy()
    h2["vs"][blk] *= 2
    a, b_ = run_oracle(h), run_oracle(h2)
    _, w = run_oracle(h, return_weights=True)
    Vf = brute.dequant_cache(h["v"], h["vs"])
    extra = np.zeros_like(a)
    for hq in range(wl.Hq):
        g = hq // wl.G
        t = np.arange(32, 64)
        extra[0, hq] = w[0, hq, t] @ Vf[blk, t - 32, g]
    assert np.allclose(b_ - a, extra, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------- kv_append ----

def test_kv_append_bf16_writes_only_the_slot_rows():
    wl = small(3, 8, 2, 64, 16, (1, 16, 70), seed=14, NB=10)
    k0, v0 = W.cache_host(wl.k_cache).copy(), W.cache_host(wl.v_cache).copy()
    k, v = k0.copy(), v0.copy()
    slots = wl.slot_mapping_np.copy()
    slots_skip = slots.copy()
    slots_skip[1] = -1                               # negative slot: no write
    oracle.kv_append(W.bf16_bits(wl.k_new), W.bf16_bits(wl.v_new), slots_skip, k, v)
    kn, vn = W.bf16_bits(wl.k_new), W.bf16_bits(wl.v_new)
    touched = np.zeros((wl.NB, wl.BS), bool)
    for i, s in enumerate(slots_skip):
        if s < 0:
            continue
        blk, off = divmod(int(s), wl.BS)
        assert np.array_equal(k[blk, off], kn[i]) and np.array_equal(v[blk, off], vn[i])
        touched[blk, off] = True
    assert np.array_equal(k[~touched], k0[~touched]) and np.array_equal(v[~touched], v0[~touched])
    # the slot positions follow "tiny-vllm part 5": block = pos // 16, offset = pos % 16
    for b in range(3):
        pos = int(wl.lengths[b]) - 1
        assert slots[b] == wl.block_tables_np[b, pos // 16] * 16 + pos % 16


def test_kv_append_fp8_scale_and_codes():
    wl = small(4, 8, 2, 128, 32, (1, 33, 40, 64), kv="fp8", seed=15, NB=12, poison=True)
    k = W.cache_host(wl.k_cache).copy()
    v = W.cache_host(wl.v_cache).copy()
    ks0, vs0 = wl.k_scale.numpy().copy(), wl.v_scale.numpy().copy()
    ks, vs = ks0.copy(), vs0.copy()
    k_before = k.copy()
    oracle.kv_append(W.bf16_bits(wl.k_new), W.bf16_bits(wl.v_new), wl.slot_mapping_np, k, v, ks, vs)
    x = brute.bf16_bits_to_f64(W.bf16_bits(wl.k_new)).astype(np.float32)   # exact
    for i, s in enumerate(wl.slot_mapping_np):
        blk, off = divmod(int(s), wl.BS)
        for g in range(wl.Hkv):
            sc = ks[blk, g]
            if off == 0:
                # a token opening a block sets the scale from its own amax
                assert sc == np.float32(np.abs(x[i, g]).max()) / np.float32(448.0)
                # ... so its largest element lands on +-448 exactly
                j = np.argmax(np.abs(x[i, g]))
                assert k[blk, off, g, j] in (0x7E, 0xFE)
            else:
                assert sc == ks0[blk, g] or (np.isnan(sc) and np.isnan(ks0[blk, g]))
            # library encode of the fp32 quotient, clamped to the saturation bound
            y = (x[i, g] / sc).astype(np.float32)
            lib = torch.from_numpy(np.clip(y, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(k[blk, off, g], lib)
            # RNE error bound: half an ulp of e4m3 (2^-4 relative, 2^-10 absolute in subnormals)
            dec = oracle.e4m3fn_decode(k[blk, off, g]) * sc
            err = np.abs(dec - x[i, g])
            bound = np.maximum(np.abs(x[i, g]) * 2.0 ** -4, 2.0 ** -10 * sc) * (1 + 1e-6)
            assert (err <= bound).all()
    # nothing but the appended rows and the opened blocks' scales changed
    touched = np.zeros((wl.NB, wl.BS), bool)
    for s in wl.slot_mapping_np:
        touched[divmod(int(s), wl.BS)] = True
    assert np.array_equal(k[~touched], k_before[~touched])


def test_kv_append_fp8_saturates_in_an_open_block():
    """A token appended into an already-open block keeps the block's scale and
    saturates values beyond 448 * scale (no re-quantisation of older tokens)."""
    NB, BS, Hkv, D = 2, 16, 1, 64
    k = np.zeros((NB, BS, Hkv, D), np.uint8)
    v = np.zeros_like(k)
    ks = np.full((NB, Hkv), 0.01, np.float32)
    vs = ks.copy()
    x = np.linspace(-10, 10, D, dtype=np.float32)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)[None, None, :]
    oracle.kv_append(xb, xb, np.array([BS + 5], np.int32), k, v, ks, vs)
    assert ks[1, 0] == np.float32(0.01)
    vals = oracle.e4m3fn_decode(k[1, 5, 0])
    xs = brute.bf16_bits_to_f64(xb[0, 0])
    sat = np.abs(xs / np.float32(0.01)) >= 448
    assert sat.any() and (np.abs(vals[sat]) == 448).all()


def test_large_scores_stay_finite_and_match_bruteforce():
    """Softmax is shift-invariant, so only the choice of shift keeps exp in
    range: with scores in the hundreds the result must still be finite and
    equal to the dense definition (which shifts by the row maximum)."""
    wl = small(2, 8, 2, 64, 16, (40, 90), seed=17, scale=40.0)
    h = host_step(wl)
    ref = run_oracle(h)
    npy = brute.dense_attention_numpy(h["q"], h["k"], h["v"], h["bt"], h["cl"], h["scale"])
    s_range = 40.0 * 64 ** 0.5 * 3
    assert s_range > 710            # exp of an unshifted score would overflow fp64
    assert np.isfinite(ref).all()
    assert np.allclose(ref, npy, rtol=1e-11, atol=1e-12)


def test_kv_append_fp8_all_zero_token_opening_a_block():
    """amax = 0 would make amax/448 a zero scale; the reading taken is scale 1.0,
    and the zero token is stored as +0 codes (a later token in the block then
    quantises against 1.0)."""
    NB, BS, Hkv, D = 2, 16, 2, 64
    k = np.full((NB, BS, Hkv, D), 0x7F, np.uint8)
    v = k.copy()
    ks = np.full((NB, Hkv), np.nan, np.float32)
    vs = ks.copy()
    z = np.zeros((1, Hkv, D), np.uint16)
    oracle.kv_append(z, z, np.array([BS], np.int32), k, v, ks, vs)
    assert (ks[1] == 1.0).all() and (vs[1] == 1.0).all()
    assert (k[1, 0] == 0).all() and (v[1, 0] == 0).all()
    assert np.isnan(ks[0]).all() and (k[0] == 0x7F).all() and (k[1, 1:] == 0x7F).all()
