"""The attention calls under HIP graph capture.

The calls enqueue their kernels on the caller's stream, allocate nothing
and never synchronise with the host, so a caller can capture them once and
replay them.  Each case captures one call in a torch CUDA graph (HIP graph
underneath), replays it several times with eager work on the stream between
the replays (fill kernels over the output and the workspace, so a replay
that reused stale memory would show), and checks every replay against the
eager call on a twin of the inputs, bit for bit.  A decode step re-appends
its token to the same slot on every replay, which leaves the caches as they
were, so its outputs repeat exactly too.
"""
from __future__ import annotations

import torch
import pytest

from paged_kv_decode_06_amd import ops
from tests import gpu_support as GS
from tests.test_gpu_decode_step import bits, step, twin
from tests.test_gpu_general import build as build_general
from tests.test_gpu_parity import DEV, build, default_kernel, say, use_kernel

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(autouse=True)
def _restore():
    yield
    default_kernel()


def replay_and_check(call, out, ws, ref, what):
    """Capture call() (which writes `out`), then replay it REPLAYS times."""
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm up off the capture (grid sizes are cached)
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(REPLAYS):
        out.fill_(float("nan"))
        ws.fill_(0xA5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(bits(out), bits(ref)), f"{what}: replay {i} differs from the eager call"
    say(f"{what}: {REPLAYS} replays equal the eager call")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("units", ["mfma", "mfma1", "valu"])
def test_decode_step_replays(kv, units):
    use_kernel(units)
    wl = build(6, 32, 8, 128, 16, (1, 17, 700, 2100, 4000, 33), kv=kv, seed=5)
    eager = twin(wl)
    ref = step(eager)
    torch.cuda.synchronize()
    out = torch.empty_like(wl.q)
    ws = GS.workspace_for(wl)

    def call():
        ops.decode_step(wl.q, wl.k_new, wl.v_new, wl.k_cache, wl.v_cache, wl.block_tables,
                        wl.context_lens, wl.scale, out, wl.k_scale, wl.v_scale, ws)

    replay_and_check(call, out, ws, ref, f"decode step {kv} {units}")
    assert torch.equal(bits(wl.k_cache), bits(eager.k_cache))
    assert torch.equal(bits(wl.v_cache), bits(eager.v_cache))


def test_decode_attention_replays():
    wl = build(5, 64, 8, 128, 32, (40, 999, 3000, 1, 64), kv="fp8", seed=8)
    GS.append_in_order(wl)
    ref = GS.gpu_step(wl, append=False).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(wl.q)
    ws = GS.workspace_for(wl)

    def call():
        ops.paged_decode_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables,
                                   wl.context_lens, wl.scale, out, wl.k_scale, wl.v_scale, ws)

    replay_and_check(call, out, ws, ref, "decode attention fp8")


@pytest.mark.parametrize("Hq,q_lens", [(32, (4, 1, 3, 4)), (64, (4, 2, 3, 4))],
                         ids=["one-tile", "two-tiles"])
def test_general_attention_replays(Hq, q_lens):
    wl = build_general(4, Hq, 8, 128, 16, (50, 900, 2500, 4), q_lens, seed=12,
                       sinks=16, window=512)
    GS.append_in_order(wl)
    mq = int(wl.q_lens.max())
    n = ops.attention_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, ops.KV_BF16, mq)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)
    ref = torch.empty_like(wl.q)
    ops.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                        wl.scale, ref, q_start=wl.q_start, max_q_len=mq, sinks=wl.sinks,
                        window=wl.window, workspace=ws)
    torch.cuda.synchronize()
    out = torch.empty_like(wl.q)

    def call():
        ops.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                            wl.scale, out, q_start=wl.q_start, max_q_len=mq, sinks=wl.sinks,
                            window=wl.window, workspace=ws)

    replay_and_check(call, out, ws, ref, f"general attention, window and sinks, Hq={Hq}")


@pytest.mark.parametrize("units", ["mfma", "mfma1"])
def test_rope_step_replays(units):
    """Two-head units run the fused kernel; one head per wave runs the RoPE
    append and the attention (three launches) inside the graph."""
    use_kernel(units)
    wl = build(4, 32, 8, 128, 16, (1, 17, 900, 5000), kv="int8", seed=21)
    eager = twin(wl)
    kvd = GS.KV_KIND[wl.kv_dtype]
    n = ops.decode_step_rope_workspace_bytes(wl.B, wl.Hq, wl.Hkv, wl.D, wl.BS, wl.MBS, kvd)
    ref = torch.empty_like(wl.q)
    ops.decode_step_rope(eager.q, eager.k_new, eager.v_new, eager.k_cache, eager.v_cache,
                         eager.block_tables, eager.context_lens, eager.scale, ref,
                         eager.k_scale, eager.v_scale, torch.zeros(n, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    out = torch.empty_like(wl.q)
    ws = torch.zeros(n, dtype=torch.uint8, device=DEV)

    def call():
        ops.decode_step_rope(wl.q, wl.k_new, wl.v_new, wl.k_cache, wl.v_cache, wl.block_tables,
                             wl.context_lens, wl.scale, out, wl.k_scale, wl.v_scale, ws)

    replay_and_check(call, out, ws, ref, f"rope step {units}")
    assert torch.equal(bits(wl.k_cache), bits(eager.k_cache))
    assert torch.equal(wl.k_scale.view(torch.int32), eager.k_scale.view(torch.int32))
