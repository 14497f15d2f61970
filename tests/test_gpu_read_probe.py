"""The streaming-read probe (pkv_read_probe) reads every whole 1 KB unit of
its buffer exactly once: wave w folds units w, w + W, w + 2W, ... into one
XOR word, which must equal the same fold computed on the host (integer
work, bit-exact).  A tail under 1 KB is not read."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_decode_06_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("units,tail", [(1, 0), (777, 0), (20000, 300)])
def test_probe_reads_every_unit_once(units, tail):
    W = ops.read_probe_waves()
    assert W > 0 and W % 4 == 0
    rng = np.random.default_rng(units)
    host = rng.integers(0, 2 ** 32, size=(units * 1024 + tail) // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda:0")
    sink = torch.full((W,), -1, dtype=torch.int32, device="cuda:0")
    ops.read_probe(buf, sink)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    per_unit = np.bitwise_xor.reduce(host[: units * 256].reshape(units, 256), axis=1)
    want = np.zeros(W, np.uint32)
    for w in range(W):
        if w < units:
            want[w] = np.bitwise_xor.reduce(per_unit[w::W])
    assert np.array_equal(got, want)


def test_probe_rejects_a_small_sink():
    buf = torch.zeros(4096, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(ops.read_probe_waves() - 1, dtype=torch.int32, device="cuda:0")
    with pytest.raises(ops.PkvError) as e:
        ops.read_probe(buf, sink)
    assert e.value.status == -4
