"""The attention kernels' widening of every one-byte code, exactly.

With one key (L = 1) the softmax weight is exactly 1, so out[h] is the
decoded V row of head h's kv head, times the block's V scale, rounded to
bf16 - and that value is already a bf16 number when the scale is a power of
two.  A V row of Hkv = 2 heads x D = 128 holds all 256 codes, so one call
pins the kernel's decode of every e4m3fn code (against torch's CPU cast,
itself pinned to the oracle's decoder by the CPU tests) and of every int8
code (code * scale), value for value (-0.0 comes out +0.0: the product
accumulates onto +0).  The two NaN codes of e4m3fn must come out NaN.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops
from tests.test_gpu_parity import DEV, default_kernel, use_kernel

pytestmark = pytest.mark.gpu

HKV, D, BS = 2, 128, 16


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


def run(kind: str, v_codes: np.ndarray, v_scale: float, G: int) -> torch.Tensor:
    Hq = HKV * G
    q = torch.randn((1, Hq, D), device=DEV).to(torch.bfloat16)
    k_cache = torch.zeros((1, BS, HKV, D), dtype=torch.uint8, device=DEV)   # code 0 = 0.0
    v_cache = torch.zeros((1, BS, HKV, D), dtype=torch.uint8, device=DEV)
    v_cache[0, 0] = torch.from_numpy(v_codes.reshape(HKV, D)).to(DEV)
    ks = torch.ones((1, HKV), dtype=torch.float32, device=DEV)
    vs = torch.full((1, HKV), v_scale, dtype=torch.float32, device=DEV)
    if kind == "fp8":
        k_cache, v_cache = k_cache.view(torch.float8_e4m3fn), v_cache.view(torch.float8_e4m3fn)
    else:
        k_cache, v_cache = k_cache.view(torch.int8), v_cache.view(torch.int8)
    bt = torch.zeros((1, 1), dtype=torch.int32, device=DEV)
    cl = torch.ones(1, dtype=torch.int32, device=DEV)
    kvd = ops.KV_FP8 if kind == "fp8" else ops.KV_INT8
    ws = torch.zeros(ops.workspace_bytes(1, Hq, HKV, D, BS, 1, kvd), dtype=torch.uint8,
                     device=DEV)
    out = torch.empty_like(q)
    ops.paged_decode_attention(q, k_cache, v_cache, bt, cl, 0.0884, out, ks, vs, ws)
    torch.cuda.synchronize()
    return out[0].cpu()


@pytest.mark.parametrize("units", ["mfma", "mfma1", "valu"])
@pytest.mark.parametrize("G", [1, 4])
@pytest.mark.parametrize("v_scale", [1.0, 0.125])
def test_every_fp8_code(units, G, v_scale):
    use_kernel(units)
    codes = np.arange(256, dtype=np.uint8)
    out = run("fp8", codes, v_scale, G)
    ref = (torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32) * v_scale)
    ref = ref.to(torch.bfloat16).reshape(HKV, D)
    for h in range(HKV * G):
        got, want = out[h], ref[h // G]
        nan = torch.isnan(want)
        assert int(nan.sum()) == 1          # 0x7f in kv head 0's row, 0xff in head 1's
        assert torch.isnan(got[nan]).all(), f"head {h}: a NaN code did not give NaN"
        # values, not bits: code 0x80 (-0.0) comes out +0.0, the sign of zero
        # being lost when the product accumulates onto +0 (IEEE: +0 + -0 = +0)
        assert torch.equal(got[~nan].float(), want[~nan].float()), f"head {h}"


@pytest.mark.parametrize("units", ["mfma", "mfma1", "valu"])
@pytest.mark.parametrize("v_scale", [1.0, 0.0078125])
def test_every_int8_code(units, v_scale):
    use_kernel(units)
    codes = np.arange(-128, 128, dtype=np.int8)
    out = run("int8", codes.view(np.uint8), v_scale, 4)
    ref = (torch.from_numpy(codes.astype(np.float32)) * v_scale).to(torch.bfloat16)
    ref = ref.reshape(HKV, D)
    for h in range(HKV * 4):
        assert torch.equal(out[h].float(), ref[h // 4].float()), f"head {h}"
