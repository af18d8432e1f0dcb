"""GPU: the streaming-read reference (pa_stream_read_probe) through the C ABI.

It is a measurement tool, not part of attention; the test checks that it reads
every byte exactly once: the XOR of all 32-bit words matches numpy's, on a
buffer of many grid strides with a ragged tail, on one 16-byte vector, and
when xor_out starts from a non-zero value.
"""
from __future__ import annotations

import numpy as np
import pytest

from paged_kv_cache_275_amd import ops

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)


@pytest.mark.parametrize("words", [4, (64 << 20) // 4 + 12, (1 << 20) + 4])
def test_stream_read_probe_xor(words):
    print(f"[gpu] stream read probe words={words}", flush=True)
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**32, words, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(host.view(np.int32)).to("cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    ops.stream_read_probe(src, out)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host)
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want)
    # a non-zero start value is folded in as well
    out.fill_(0x12345678)
    ops.stream_read_probe(src, out)
    torch.cuda.synchronize()
    assert int(out.cpu().numpy().view(np.uint32)[0]) == int(want) ^ 0x12345678
