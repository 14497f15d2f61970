"""The Python binding rejects inconsistent arguments before anything reaches
the library: every shape is checked against the others (the kernels index
the fp8 / int8 scales by (block, kv head), so a mis-shaped scale tensor would
otherwise be read and written out of bounds), and only then the device.
CPU only: CPU tensors pass the shape checks and stop at the device check."""
from __future__ import annotations

import pytest
import torch

from paged_kv_decode_06_amd import ops

NB, BS, HKV, D, B, HQ, MBS = 6, 16, 2, 64, 3, 8, 2


def caches(dtype=torch.bfloat16, scales=False, ks_shape=(NB, HKV), vs_shape=(NB, HKV),
           v_shape=(NB, BS, HKV, D)):
    k = torch.zeros((NB, BS, HKV, D), dtype=dtype)
    v = torch.zeros(v_shape, dtype=dtype)
    ks = torch.ones(ks_shape) if scales else None
    vs = torch.ones(vs_shape) if scales else None
    return k, v, ks, vs


def attn_inputs():
    q = torch.zeros((B, HQ, D), dtype=torch.bfloat16)
    bt = torch.zeros((B, MBS), dtype=torch.int32)
    cl = torch.ones(B, dtype=torch.int32)
    return q, bt, cl


def call_attention(k, v, ks, vs):
    q, bt, cl = attn_inputs()
    ops.paged_decode_attention(q, k, v, bt, cl, 0.125, torch.empty_like(q), ks, vs,
                               workspace=torch.zeros(16, dtype=torch.uint8))


def call_general(k, v, ks, vs):
    q, bt, cl = attn_inputs()
    ops.paged_attention(q, k, v, bt, cl, 0.125, torch.empty_like(q),
                        q_start=torch.arange(B + 1, dtype=torch.int32), k_scale=ks, v_scale=vs,
                        workspace=torch.zeros(16, dtype=torch.uint8))


def call_step(k, v, ks, vs):
    q, bt, cl = attn_inputs()
    kn = torch.zeros((B, HKV, D), dtype=torch.bfloat16)
    ops.decode_step(q, kn, kn.clone(), k, v, bt, cl, 0.125, torch.empty_like(q), ks, vs,
                    workspace=torch.zeros(16, dtype=torch.uint8))


def call_append(k, v, ks, vs):
    kn = torch.zeros((B, HKV, D), dtype=torch.bfloat16)
    ops.kv_append(kn, kn.clone(), torch.zeros(B, dtype=torch.int32), k, v, ks, vs)


def call_prepared_append(k, v, ks, vs):
    kn = torch.zeros((B, HKV, D), dtype=torch.bfloat16)
    ops.PreparedAppend(kn, kn.clone(), torch.zeros(B, dtype=torch.int32), k, v, ks, vs)


def call_rope_append(k, v, ks, vs):
    q = torch.zeros((B, HQ, D), dtype=torch.bfloat16)
    kn = torch.zeros((B, HKV, D), dtype=torch.bfloat16)
    pos = torch.zeros(B, dtype=torch.int32)
    ops.rope_kv_append(q, kn, kn.clone(), pos, pos.clone(), k, v, ks, vs)


CALLS = [call_attention, call_general, call_step, call_append, call_prepared_append,
         call_rope_append]


@pytest.mark.parametrize("call", CALLS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("dtype", [torch.uint8, torch.int8], ids=["fp8", "int8"])
def test_scales_must_be_blocks_by_kv_heads(call, dtype):
    for ks_shape, vs_shape in [((NB, HKV + 1), (NB, HKV)), ((NB, HKV), (NB - 1, HKV)),
                               ((HKV, NB), (HKV, NB))]:
        with pytest.raises(ValueError, match="scale must be"):
            call(*caches(dtype, True, ks_shape, vs_shape))


@pytest.mark.parametrize("call", CALLS, ids=lambda f: f.__name__)
def test_v_cache_must_match_k_cache(call):
    with pytest.raises(ValueError, match="differs from k_cache"):
        call(*caches(v_shape=(NB, BS, HKV + 1, D)))
    with pytest.raises(ValueError, match="differs from k_cache"):
        call(*caches(v_shape=(NB + 1, BS, HKV, D)))


@pytest.mark.parametrize("call", CALLS, ids=lambda f: f.__name__)
def test_bf16_cache_takes_no_scales(call):
    k, v, _, _ = caches()
    with pytest.raises(ValueError, match="no scales"):
        call(k, v, torch.ones(NB, HKV), torch.ones(NB, HKV))


@pytest.mark.parametrize("call", CALLS, ids=lambda f: f.__name__)
@pytest.mark.parametrize("kind", ["bf16", "fp8"])
def test_consistent_cpu_arguments_stop_at_the_device_check(call, kind):
    args = caches() if kind == "bf16" else caches(torch.uint8, True)
    with pytest.raises(ValueError, match="must be on the GPU"):
        call(*args)
