"""The C ABI library loads and exports every symbol include/pkv.h declares,
and rejects bad host-side arguments before touching a GPU (CPU only)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from paged_kv_decode_06_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.library_path()):
        pytest.fail("libpkv.so is not built (run __graft_entry__.build())")
    return ops.lib()


def test_header_declares_the_two_calls():
    names = declared_functions()
    assert "pkv_paged_decode_attention" in names and "pkv_kv_append" in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for st, text in [(0, "ok"), (-1, "null pointer"), (-4, "workspace too small")]:
        assert lib.pkv_status_string(st).decode() == text


NULL = None


def attn(lib, **over):
    args = dict(q=8, k=16, v=32, ks=NULL, vs=NULL, bt=48, cl=64, scale=0.125, out=80,
                B=2, Hq=8, Hkv=2, D=64, BS=16, NB=4, MBS=2, kv=0, ws=96, wsb=1 << 20, stream=NULL)
    args.update(over)
    P = ctypes.c_void_p
    a = args
    return lib.pkv_paged_decode_attention(
        P(a["q"]) if a["q"] else None, P(a["k"]) if a["k"] else None,
        P(a["v"]) if a["v"] else None, P(a["ks"]) if a["ks"] else None,
        P(a["vs"]) if a["vs"] else None, P(a["bt"]) if a["bt"] else None,
        P(a["cl"]) if a["cl"] else None, ctypes.c_float(a["scale"]),
        P(a["out"]) if a["out"] else None, a["B"], a["Hq"], a["Hkv"], a["D"], a["BS"],
        a["NB"], a["MBS"], a["kv"], P(a["ws"]) if a["ws"] else None,
        ctypes.c_size_t(a["wsb"]), None)


def test_attention_argument_checks_fail_before_launch(lib):
    # these are checked before any HIP call, so they work without a GPU
    assert attn(lib, q=0) == -1
    assert attn(lib, out=0) == -1
    assert attn(lib, Hq=6, Hkv=4) == -2            # Hq % Hkv != 0
    assert attn(lib, D=96) == -3                   # unsupported head dim
    assert attn(lib, BS=8) == -3                   # unsupported block size
    assert attn(lib, Hq=64, Hkv=2) == -3           # G = 32
    assert attn(lib, Hq=24, Hkv=8) == -3           # G = 3
    assert attn(lib, kv=7) == -3
    assert attn(lib, kv=1) == -1                   # fp8 without scales
    assert attn(lib, ks=128, vs=144) == -2         # bf16 with scales
    assert attn(lib, B=-1) == -2
    assert attn(lib, B=100000) == -3
    assert attn(lib, q=9) == -6                    # misaligned
    assert "Hq" in lib.pkv_last_error().decode() or lib.pkv_last_error().decode()


def test_kv_append_argument_checks(lib):
    P = ctypes.c_void_p
    f = lib.pkv_kv_append
    ok = [P(16), P(32), P(48), P(64), P(80), None, None, 2, 2, 64, 16, 4, 0, None]
    bad = list(ok); bad[0] = None
    assert f(*bad) == -1
    bad = list(ok); bad[9] = 80
    assert f(*bad) == -3
    bad = list(ok); bad[12] = 1                     # fp8 without scales
    assert f(*bad) == -1
    bad = list(ok); bad[7] = -1
    assert f(*bad) == -2
    bad = list(ok); bad[0] = P(17)
    assert f(*bad) == -6
    zero = list(ok); zero[7] = 0                    # N = 0: nothing to do
    assert f(*zero) == 0


def test_decode_step_argument_checks(lib):
    P = ctypes.c_void_p

    def step(**over):
        a = dict(q=8, kn=16, vn=32, k=48, v=64, bt=80, cl=96, out=112, B=2, Hq=8, Hkv=2, D=64,
                 BS=16, NB=4, MBS=2, kv=0)
        a.update(over)
        p = lambda x: P(x) if x else None  # noqa: E731
        return lib.pkv_decode_step(p(a["q"]), p(a["kn"]), p(a["vn"]), p(a["k"]), p(a["v"]),
                                   None, None, p(a["bt"]), p(a["cl"]), ctypes.c_float(0.125),
                                   p(a["out"]), a["B"], a["Hq"], a["Hkv"], a["D"], a["BS"],
                                   a["NB"], a["MBS"], a["kv"], P(128), ctypes.c_size_t(1 << 20),
                                   None)

    assert step(kn=0) == -1                        # the new token is required
    assert step(vn=0) == -1
    assert step(q=0) == -1
    assert step(kn=17) == -6                       # misaligned new token
    assert step(D=96) == -3
    assert step(Hq=6, Hkv=4) == -2
    assert step(B=0, q=0, kn=0, vn=0) == 0         # empty batch: nothing to do


def test_rope_kv_append_argument_checks(lib):
    """Checked before any HIP call, so this runs without a GPU."""
    f = lib.pkv_rope_kv_append
    P = None
    llama3 = (500000.0, 32.0, 1.0, 4.0, 8192.0)
    assert f(P, P, P, P, P, P, P, P, P, P, 0, 8, 2, 64, 16, 4, 0, *llama3, P) == 0   # N = 0
    assert f(P, P, P, P, P, P, P, P, P, P, 1, 8, 16, 64, 16, 4, 0, *llama3, P) == -3  # Hkv > 8
    assert f(P, P, P, P, P, P, P, P, P, P, 1, 8, 2, 96, 16, 4, 0, *llama3, P) == -3   # D = 96
    assert f(P, P, P, P, P, P, P, P, P, P, 1, 8, 2, 64, 16, 4, 0,
             500000.0, 32.0, 4.0, 1.0, 8192.0, P) == -2                              # low >= high
    assert f(P, P, P, P, P, P, P, P, P, P, 1, 8, 2, 64, 16, 4, 0, *llama3, P) == -1   # NULL tensors


def test_decode_step_rope_argument_checks(lib):
    """Rope parameters and D are checked before any HIP call (no GPU needed)."""
    f = lib.pkv_decode_step_rope
    P = None
    args = lambda theta, factor, low, high, orig, D=64: f(   # noqa: E731
        P, P, P, P, P, P, P, P, P, 0.125, theta, factor, low, high, orig, P,
        2, 8, 2, D, 16, 4, 4, 0, P, 0, P)
    assert args(1.0, 32.0, 1.0, 4.0, 8192.0) == -2               # theta must exceed 1
    assert args(500000.0, 0.0, 1.0, 4.0, 8192.0) == -2           # factor > 0
    assert args(500000.0, 32.0, 4.0, 1.0, 8192.0) == -2          # low < high
    assert args(500000.0, 32.0, 1.0, 4.0, 0.0) == -2             # original_max_len > 0
    assert args(500000.0, 32.0, 1.0, 4.0, 8192.0, D=96) == -3    # D in {64, 128}


def test_validate_inputs_host_checks(lib):
    """The validation call runs the attention call's host checks first (no GPU needed)."""
    f = lib.pkv_validate_inputs
    P = None
    assert f(P, P, P, P, P, P, P, 0.125, P, 0, 8, 2, 64, 16, 4, 4, 0, P, 0, P) == 0    # B = 0
    assert f(P, P, P, P, P, P, P, 0.125, P, 2, 8, 2, 64, 16, 4, 4, 0, P, 0, P) == -1   # NULL q
    assert f(P, P, P, P, P, P, P, 0.125, P, 2, 8, 2, 96, 16, 4, 4, 0, P, 0, P) == -3   # D = 96
    assert lib.pkv_status_string(-7).decode() == "device-resident input breaks the contract"


def test_process_wide_switches_check_their_argument(lib):
    """The pkv_select_* switches accept their documented values only
    (PKV_ERR_UNSUPPORTED otherwise; no GPU needed)."""
    unsupported = -3   # PKV_ERR_UNSUPPORTED
    assert lib.pkv_select_run_cost(9) == unsupported
    assert lib.pkv_select_run_cost(-1) == unsupported
    for v in (0, 8, 2):
        assert lib.pkv_select_run_cost(v) == 0
    for f in (lib.pkv_select_result_parking, lib.pkv_select_share_combine,
              lib.pkv_select_unit_heads):
        assert f(2) == unsupported and f(-1) == unsupported
        assert f(0) == 0
    assert lib.pkv_select_result_parking(1) == 0
    assert lib.pkv_select_share_combine(1) == 0
    assert lib.pkv_select_unit_heads(0) == 0
    assert lib.pkv_select_run_cost(2) == 0
