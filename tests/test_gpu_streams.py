"""Independent calls on separate streams, from separate host threads.

The library keeps no per-call state outside the caller's workspace; its
host side shares only a mutex-guarded cache of grid sizes and a per-thread
error string.  Two different workloads, each with its own workspace and
stream, are run many times concurrently from two host threads (ctypes
releases the interpreter lock during the calls); each stream's result must
equal the same call run alone, bit for bit.
"""
from __future__ import annotations

import threading

import pytest
import torch

from paged_kv_decode_06_amd import ops
from tests import gpu_support as GS
from tests.test_gpu_decode_step import bits
from tests.test_gpu_parity import DEV, build, say

pytestmark = pytest.mark.gpu

ROUNDS = 20


def attention(wl, out, ws, stream=None):
    ops.paged_decode_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_tables, wl.context_lens,
                               wl.scale, out, wl.k_scale, wl.v_scale, ws, stream=stream)


def test_two_streams_two_threads():
    a = build(8, 32, 8, 128, 16, (1, 40, 700, 2100, 4000, 33, 999, 1500), seed=31)
    b = build(5, 64, 8, 128, 32, (64, 3000, 5, 1200, 2222), kv="fp8", seed=32)
    for wl in (a, b):
        GS.append_in_order(wl)
    ws = [GS.workspace_for(a), GS.workspace_for(b)]
    ref = []
    for wl, w in zip((a, b), ws):       # alone, on the default stream
        r = torch.empty_like(wl.q)
        attention(wl, r, w)
        ref.append(r)
    torch.cuda.synchronize()

    streams = [torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)]
    outs = [[torch.empty_like(a.q) for _ in range(ROUNDS)], [torch.empty_like(b.q) for _ in range(ROUNDS)]]
    errors = []

    def worker(i, wl):
        try:
            torch.cuda.set_device(DEV)
            with torch.cuda.stream(streams[i]):
                for r in range(ROUNDS):
                    attention(wl, outs[i][r], ws[i], stream=streams[i])
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(i, wl)) for i, wl in enumerate((a, b))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(ROUNDS):
            assert torch.equal(bits(outs[i][r]), bits(ref[i])), f"stream {i}, round {r}"
    say(f"{2 * ROUNDS} concurrent calls equal the calls run alone")
