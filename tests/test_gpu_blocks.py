"""GPU parity for copy on write and for a continuous-batching replay.

pa_copy_blocks must copy blocks bit for bit.  The replay drives the host block
manager (arrivals with prompts, forks that share a prefix, departures, one new
token per running sequence per step) and runs every step through the C ABI
(pa_copy_blocks, pa_reshape_and_cache for prompts, pa_decode_append); the same
steps run through the Python block-manager model and the fp64 oracle, and the
pools must agree bit for bit and the outputs within the bf16 tolerance.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle.block_manager import OK, OracleBlockManager
from paged_kv_cache_275_amd import ops
from paged_kv_cache_275_amd.blocks import BlockManager, copy_blocks
from tests._gpu import to_dev, to_host, widen_dev
from tests._helpers import assert_attention_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)


def _bf16(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_copy_blocks_bit_exact(dtype):
    rng = np.random.default_rng(5)
    nb, hkv, d = 64, 4, 128
    if dtype == "f32":
        kc = rng.standard_normal((nb, 16, hkv, d)).astype(np.float32)
        vc = rng.standard_normal((nb, 16, hkv, d)).astype(np.float32)
    else:
        kc, vc = _bf16(rng, (nb, 16, hkv, d)), _bf16(rng, (nb, 16, hkv, d))
    perm = rng.permutation(nb)
    pairs = np.stack([perm[:20], perm[20:40]], 1).astype(np.int32)   # 20 sources, 20 other destinations
    dk, dv = to_dev(kc), to_dev(vc)
    copy_blocks(dk, dv, to_dev(pairs))
    torch.cuda.synchronize()
    kc[pairs[:, 1]] = kc[pairs[:, 0]]
    vc[pairs[:, 1]] = vc[pairs[:, 0]]
    assert to_host(dk).tobytes() == kc.tobytes()
    assert to_host(dv).tobytes() == vc.tobytes()


def test_continuous_batching_replay():
    rng = np.random.default_rng(2024)
    nb, hq, hkv, d, mb = 256, 8, 2, 64, 24
    scale = 1.0 / np.sqrt(d)
    cpp, ref = BlockManager(nb), OracleBlockManager(nb)
    kc = np.full((nb, 16, hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    dk, dv = to_dev(kc), to_dev(vc)
    running, next_id = [], 0
    ws = None
    for step in range(14):
        # departures and arrivals (prompts written with pa_reshape_and_cache)
        for sid in list(running):
            if rng.random() < 0.15:
                cpp.free(sid)
                assert ref.free(sid) == OK
                running.remove(sid)
        for _ in range(int(rng.integers(1, 4))):
            plen = int(rng.integers(1, 120))
            if ref.add_sequence(next_id, plen) != OK:
                continue
            cpp.add_sequence(next_id, plen)
            bt, _ = cpp.batch_tables([next_id], mb)
            t = np.arange(plen)
            slots = (bt[0, t // 16].astype(np.int64) * 16 + t % 16).astype(np.int32)
            k, v = _bf16(rng, (plen, hkv, d)), _bf16(rng, (plen, hkv, d))
            ops.reshape_and_cache(to_dev(k), to_dev(v), dk, dv, to_dev(slots))
            oracle.reshape_and_cache(k, v, kc, vc, slots)
            running.append(next_id)
            next_id += 1
        if running and rng.random() < 0.5:                # a request sharing another's prompt
            parent = int(rng.choice(running))
            cpp.fork(parent, next_id)
            assert ref.fork(parent, next_id) == OK
            running.append(next_id)
            next_id += 1
        running = [s for s in running if len(ref.seqs[s][0]) < mb]   # keep within the table width
        if not running:
            continue
        # one decode step: new token per running sequence
        st, slots_ref, copies_ref = ref.append_batch(running)
        assert st == OK
        slots, copies = cpp.append_batch(running)
        assert slots.tolist() == slots_ref and copies == copies_ref
        if copies:
            pairs = np.asarray(copies, np.int32)
            copy_blocks(dk, dv, to_dev(pairs))
            kc[pairs[:, 1]] = kc[pairs[:, 0]]
            vc[pairs[:, 1]] = vc[pairs[:, 0]]
        bt, cl = cpp.batch_tables(running, mb)
        rows, lens = ref.tables(running, mb)
        assert bt.tolist() == rows and cl.tolist() == lens
        s = len(running)
        q, kn, vn = _bf16(rng, (s, hq, d)), _bf16(rng, (s, hkv, d)), _bf16(rng, (s, hkv, d))
        out = torch.empty((s, hq, d), dtype=torch.bfloat16, device="cuda")
        if ws is None or ws.numel() < ops.decode_workspace_size(s, hq, hkv, d, mb):
            ws = torch.zeros(ops.decode_workspace_size(max(s, 64), hq, hkv, d, mb), dtype=torch.uint8,
                             device="cuda")
        print(f"[gpu] replay step {step}: S={s} copies={len(copies)} free={cpp.num_free}", flush=True)
        ops.decode_append(out, to_dev(q), to_dev(kn), to_dev(vn), dk, dv, to_dev(bt), to_dev(cl), scale,
                          workspace=ws)
        torch.cuda.synchronize()
        oracle.reshape_and_cache(kn, vn, kc, vc, slots)
        ref_out = oracle.decode(q, kc, vc, bt, cl, scale)
        assert_attention_close(widen_dev(out), ref_out, "bf16", f"replay step {step}")
        assert to_host(dk).tobytes() == kc.tobytes(), f"K pool differs after step {step}"
        assert to_host(dv).tobytes() == vc.tobytes(), f"V pool differs after step {step}"
    assert next_id > 10
    cpp.close()
