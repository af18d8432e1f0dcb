"""GPU parity: KV append and decode through the C ABI against the fp64 oracle.

Every workload is seeded and synthetic (paged_kv_cache_275_amd.workloads).
The cache write must be bit-exact over the WHOLE pool (untouched slots keep
their NaN poison); attention must be within the stated tolerance (fp32:
max-abs 1e-5; bf16: max-abs 2e-2 and per-(row, head) relative 1e-2).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from paged_kv_cache_275_amd import ops
from paged_kv_cache_275_amd import workloads as W
from tests import _oracle_threads as oracle_threads
from tests._gpu import DevWorkload, to_host, widen_dev
from tests._helpers import assert_attention_close, widen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - collected on CPU hosts too
    pytest.skip("no GPU", allow_module_level=True)


def _oracle_pool_after_append(wl):
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.reshape_and_cache(wl.k_new, wl.v_new, kc, vc, wl.slot_mapping)
    return kc, vc


def _run_append_and_decode(wl):
    dw = DevWorkload(wl)
    ops.reshape_and_cache(dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, dw.slot_mapping)
    ops.decode(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, wl.scale)
    torch.cuda.synchronize()
    return dw


def _check_workload(wl, label, threaded=False):
    print(f"[gpu] {label}: S={wl.num_seqs} sumN={int(wl.context_lens.sum())} "
          f"NB={wl.num_blocks} dtype={wl.dtype}", flush=True)
    dw = _run_append_and_decode(wl)
    kc, vc = _oracle_pool_after_append(wl)
    assert to_host(dw.k_cache).tobytes() == kc.tobytes(), f"{label}: K cache differs"
    assert to_host(dw.v_cache).tobytes() == vc.tobytes(), f"{label}: V cache differs"
    if threaded:
        ref = oracle_threads.decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale)
    else:
        ref = oracle.decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale)
    got = widen_dev(dw.out)
    mx, rel = assert_attention_close(got, ref, wl.dtype, label)
    print(f"[gpu] {label}: max-abs {mx:.3e} row-rel {rel:.3e}", flush=True)
    return dw, kc, vc, ref


# Small variants of every shape: several partitions and a ragged last block,
# quick for the oracle.
@pytest.mark.parametrize("name,num_seqs", [("tiny_fp32", None), ("qwen3_0p6b", 6),
                                           ("llama3_8b", 8), ("long_skewed", 2),
                                           ("mixed_prefill", 6)])
@pytest.mark.parametrize("seed", [0, 100, 200])
def test_decode_small(name, num_seqs, seed):
    wl = W.make_workload(name, seed=seed + W.CONFIG_NAMES.index(name), num_seqs=num_seqs)
    _check_workload(wl, f"{name}/s{seed}/n{num_seqs}")


# Full-size workloads, exactly as the bench builds them (seed = config index),
# and the same shapes at seeds + 100 and + 200.
@pytest.mark.parametrize("name", list(W.CONFIG_NAMES))
@pytest.mark.parametrize("seed_offset", [0, 100, 200])
def test_decode_full_size(name, seed_offset):
    wl = W.make_workload(name, seed=W.CONFIG_NAMES.index(name) + seed_offset)
    _check_workload(wl, f"{name}/full/+{seed_offset}", threaded=True)


def test_decode_deterministic_and_block_permutation_invariant():
    wl = W.make_workload("qwen3_0p6b", seed=7, num_seqs=5)
    dw = _run_append_and_decode(wl)
    first = to_host(dw.out).copy()
    ops.decode(dw.out, dw.q, dw.k_cache, dw.v_cache, dw.block_tables, dw.context_lens, wl.scale)
    torch.cuda.synchronize()
    assert to_host(dw.out).tobytes() == first.tobytes(), "repeated decode is not bit-identical"
    # relabel physical blocks: new block perm[b] holds old block b
    rng = np.random.default_rng(70)
    perm = torch.from_numpy(rng.permutation(wl.num_blocks)).cuda()
    kc2 = torch.empty_like(dw.k_cache)
    vc2 = torch.empty_like(dw.v_cache)
    kc2[perm] = dw.k_cache
    vc2[perm] = dw.v_cache
    bt = dw.block_tables.long()
    bt2 = torch.where(bt >= 0, perm[bt.clamp(min=0)], bt).to(torch.int32).contiguous()
    out2 = torch.empty_like(dw.out)
    ops.decode(out2, dw.q, kc2, vc2, bt2, dw.context_lens, wl.scale)
    torch.cuda.synchronize()
    assert to_host(out2).tobytes() == first.tobytes(), "block relabelling changed the output"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_single_token_context_returns_v_exactly(dtype):
    wl = W.make_workload("tiny_fp32" if dtype == "f32" else "llama3_8b", seed=3, num_seqs=4)
    wl.context_lens[:] = 1
    # the one token of each sequence is the appended one, at slot block_tables[s,0]*16
    wl.slot_mapping[:] = wl.block_tables[:, 0] * 16
    dw = _run_append_and_decode(wl)
    got = to_host(dw.out)
    g = wl.num_q_heads // wl.num_kv_heads
    want = np.repeat(wl.v_new, g, axis=1)           # [S, Hq, D]
    assert got.tobytes() == np.ascontiguousarray(want).tobytes()


def test_zero_length_context_gives_zeros():
    wl = W.make_workload("llama3_8b", seed=4, num_seqs=3)
    wl.context_lens[1] = 0
    wl.slot_mapping[1] = -1                         # nothing appended for it
    dw = _run_append_and_decode(wl)
    got = widen_dev(dw.out)
    assert np.all(got[1] == 0.0)
    kc, vc = _oracle_pool_after_append(wl)
    ref = oracle.decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale)
    assert_attention_close(got, ref, wl.dtype, "zero-length")


def _bf16_bits(rng, shape):
    return (rng.standard_normal(shape).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _random_bf16_case(rng, hq, hkv, d, lens, spare_blocks=4):
    """A bf16 pool holding len(lens) sequences in shuffled blocks (NaN elsewhere)."""
    s = len(lens)
    need = [-(-int(n) // 16) for n in lens]
    nb = sum(need) + spare_blocks
    mb = max(1, max(need))
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((s, mb), -1, np.int32)
    off = 0
    for i, k in enumerate(need):
        bt[i, :k] = perm[off:off + k]
        off += k
    kc = np.full((nb, 16, hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    tok = np.concatenate([np.arange(int(n)) for n in lens]) if sum(lens) else np.zeros(0, np.int64)
    seq = np.repeat(np.arange(s), lens)
    slot = bt[seq, tok // 16].astype(np.int64) * 16 + tok % 16
    kc.reshape(-1, hkv, d)[slot] = _bf16_bits(rng, (len(slot), hkv, d))
    vc.reshape(-1, hkv, d)[slot] = _bf16_bits(rng, (len(slot), hkv, d))
    q = _bf16_bits(rng, (s, hq, d))
    return q, kc, vc, bt, np.asarray(lens, np.int32)


def _decode_bf16(q, kc, vc, bt, lens, scale):
    from tests._gpu import to_dev
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    ops.decode(out, to_dev(q), to_dev(kc), to_dev(vc), to_dev(bt), to_dev(lens), scale)
    torch.cuda.synchronize()
    return widen_dev(out)


def test_group_sizes_and_head_dims():
    """GQA groups 1, 2, 3, 8, 16 and head_dim 64 on a reshaped small workload."""
    for hq, hkv, d in [(8, 8, 128), (6, 2, 64), (24, 3, 128), (16, 2, 64), (32, 2, 128)]:
        rng = np.random.default_rng(hq * 1000 + hkv)
        q, kc, vc, bt, lens = _random_bf16_case(rng, hq, hkv, d, [1, 37, 300], spare_blocks=40)
        got = _decode_bf16(q, kc, vc, bt, lens, 0.09)
        ref = oracle.decode(q, kc, vc, bt, lens, 0.09)
        assert_attention_close(got, ref, "bf16", f"hq{hq}/hkv{hkv}/d{d}")


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (32, 4, 128)])
def test_decode_max_sequences(hq, hkv, d):
    """8192 sequences (the most one call takes) of 0..40 tokens: every wave
    closes many segments, more than it can stage at once."""
    rng = np.random.default_rng(8192 + hq)
    lens = rng.integers(0, 41, 8192)
    lens[rng.random(8192) < 0.05] = 0
    print(f"[gpu] max sequences hq={hq} hkv={hkv} d={d} sumN={int(lens.sum())}", flush=True)
    q, kc, vc, bt, lens = _random_bf16_case(rng, hq, hkv, d, lens.tolist())
    got = _decode_bf16(q, kc, vc, bt, lens, 1.0 / np.sqrt(d))
    ref = oracle.decode(q, kc, vc, bt, lens, 1.0 / np.sqrt(d))
    assert np.all(got[lens == 0] == 0.0)
    assert_attention_close(got, ref, "bf16", f"S=8192 hq{hq}/hkv{hkv}/d{d}")


@pytest.mark.parametrize("ticks", ["0", "1", "64"])
def test_decode_switch_cost_does_not_change_results(ticks):
    """The segment cost only moves the split points between wave groups."""
    wl = W.make_workload("llama3_8b", seed=31, num_seqs=40)
    with ops.decode_launch(switch_ticks=int(ticks)):
        _check_workload(wl, f"switch_ticks={ticks}")


def test_invalid_arguments_raise():
    q = torch.zeros((2, 6, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((4, 16, 4, 128), dtype=torch.bfloat16, device="cuda")
    bt = torch.zeros((2, 4), dtype=torch.int32, device="cuda")
    cl = torch.ones(2, dtype=torch.int32, device="cuda")
    with pytest.raises(ops.PAError) as e:
        ops.decode(torch.empty_like(q), q, kc, kc, bt, cl, 0.1)   # 6 % 4 != 0
    assert e.value.status == ops.PA_EINVAL


@pytest.mark.parametrize("stages", ["2", "3", "4"])
def test_decode_ring_depths(stages):
    """Every built ring depth (pa_decode_set_launch) gives a correct result,
    fused and unfused, also for a context of many windows."""
    wl = W.make_workload("llama3_8b", seed=51, num_seqs=10)
    with ops.decode_launch(stages=int(stages)):
        _check_workload(wl, f"stages={stages}")
        _check_fused(W.make_workload("long_skewed", seed=52, num_seqs=2), f"stages={stages}/long")


@pytest.mark.parametrize("waves", ["4", "8", "60", "4096"])
def test_decode_launch_shapes(waves):
    """The result must not depend on how the units are split over waves: one
    workgroup (several LDS windows per wave), few waves, an odd count and the
    largest grid (mostly empty ranges)."""
    with ops.decode_launch(waves=int(waves)):
        wl = W.make_workload("llama3_8b", seed=21, num_seqs=12)
        _check_workload(wl, f"waves={waves}")
        wl = W.make_workload("long_skewed", seed=22, num_seqs=2)
        _check_workload(wl, f"waves={waves}/long")


# ---------------------------------------------------------------- fused append
def _run_fused(wl):
    """pa_decode_append with the decode tokens (the last num_seqs new tokens);
    prefill tokens, if any, are appended first with pa_reshape_and_cache."""
    dw = DevWorkload(wl)
    s = wl.num_seqs
    t = wl.k_new.shape[0]
    if t > s:
        ops.reshape_and_cache(dw.k_new[:t - s], dw.v_new[:t - s], dw.k_cache, dw.v_cache,
                              dw.slot_mapping[:t - s])
    ops.decode_append(dw.out, dw.q, dw.k_new[t - s:], dw.v_new[t - s:], dw.k_cache, dw.v_cache,
                      dw.block_tables, dw.context_lens, wl.scale)
    torch.cuda.synchronize()
    return dw


def _check_fused(wl, label):
    print(f"[gpu] fused {label}: S={wl.num_seqs} sumN={int(wl.context_lens.sum())}", flush=True)
    dw = _run_fused(wl)
    kc, vc = _oracle_pool_after_append(wl)
    assert to_host(dw.k_cache).tobytes() == kc.tobytes(), f"{label}: K cache differs"
    assert to_host(dw.v_cache).tobytes() == vc.tobytes(), f"{label}: V cache differs"
    ref = oracle.decode(wl.q, kc, vc, wl.block_tables, wl.context_lens, wl.scale)
    mx, rel = assert_attention_close(widen_dev(dw.out), ref, wl.dtype, f"fused {label}")
    print(f"[gpu] fused {label}: max-abs {mx:.3e} row-rel {rel:.3e}", flush=True)


@pytest.mark.parametrize("name,num_seqs", [("tiny_fp32", None), ("qwen3_0p6b", 6), ("llama3_8b", 8),
                                           ("long_skewed", 2), ("mixed_prefill", 6), ("llama3_8b", None),
                                           ("mixed_prefill", None)])
def test_decode_append_equals_append_then_decode(name, num_seqs):
    """Fused KV append + decode: the whole pool bit for bit as pa_reshape_and_cache
    leaves it, and attention within tolerance of the oracle."""
    seed = W.CONFIG_NAMES.index(name) + 300
    _check_fused(W.make_workload(name, seed=seed, num_seqs=num_seqs), f"{name}/{num_seqs}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_append_single_token_returns_new_v(dtype):
    """A context of one token is the new token alone: out equals its value row
    exactly, read from the input (its cache slot held NaN before the call)."""
    name = "tiny_fp32" if dtype == "f32" else "llama3_8b"
    wl = W.make_workload(name, seed=41, num_seqs=4)
    wl.context_lens[:] = 1
    t = wl.k_new.shape[0]
    for s in range(wl.num_seqs):
        wl.slot_mapping[t - wl.num_seqs + s] = int(wl.block_tables[s, 0]) * 16
    dw = _run_fused(wl)
    got = to_host(dw.out)
    hq, hkv = wl.num_q_heads, wl.num_kv_heads
    for h in range(hq):
        np.testing.assert_array_equal(got[:, h], wl.v_new[t - wl.num_seqs:, h // (hq // hkv)])


def test_decode_append_block_boundaries_and_empty():
    """New tokens at the first and last slot of a block, and a sequence with no
    tokens (nothing appended, zero row)."""
    rng = np.random.default_rng(77)
    hq, hkv, d = 32, 8, 128
    lens = [1, 15, 16, 17, 32, 33, 48, 0, 5]
    q, kc, vc, bt, lens = _random_bf16_case(rng, hq, hkv, d, lens, spare_blocks=8)
    s = len(lens)
    # the new tokens' slots must not hold history: poison them, keep the rows aside
    key = _bf16_bits(rng, (s, hkv, d))
    value = _bf16_bits(rng, (s, hkv, d))
    slots = np.array([int(bt[i, (n - 1) // 16]) * 16 + (n - 1) % 16 if n > 0 else -1
                      for i, n in enumerate(lens)], np.int32)
    for i, sl in enumerate(slots):
        if sl >= 0:
            kc.reshape(-1, hkv, d)[sl] = 0x7FC0
            vc.reshape(-1, hkv, d)[sl] = 0x7FC0
    from tests._gpu import to_dev
    dkc, dvc = to_dev(kc), to_dev(vc)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    ops.decode_append(out, to_dev(q), to_dev(key), to_dev(value), dkc, dvc, to_dev(bt), to_dev(lens), 0.088)
    torch.cuda.synchronize()
    okc, ovc = kc.copy(), vc.copy()
    oracle.reshape_and_cache(key, value, okc, ovc, slots)
    assert to_host(dkc).tobytes() == okc.tobytes()
    assert to_host(dvc).tobytes() == ovc.tobytes()
    got = widen_dev(out)
    assert np.all(got[7] == 0.0)
    ref = oracle.decode(q, okc, ovc, bt, lens, 0.088)
    assert_attention_close(got, ref, "bf16", "fused boundaries")


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (32, 8, 128)])
def test_decode_append_max_sequences(hq, hkv, d):
    """8192 sequences in one fused call (more than the merge kernel has
    workgroups, so each copies the new rows of several), 5% of them empty."""
    rng = np.random.default_rng(4096 + hq)
    lens = rng.integers(1, 41, 8192)
    lens[rng.random(8192) < 0.05] = 0
    print(f"[gpu] fused max sequences hq={hq} hkv={hkv} d={d} sumN={int(lens.sum())}", flush=True)
    q, kc, vc, bt, lens = _random_bf16_case(rng, hq, hkv, d, lens.tolist())
    s = len(lens)
    key = _bf16_bits(rng, (s, hkv, d))
    value = _bf16_bits(rng, (s, hkv, d))
    slots = np.array([int(bt[i, (n - 1) // 16]) * 16 + (n - 1) % 16 if n > 0 else -1
                      for i, n in enumerate(lens)], np.int32)
    from tests._gpu import to_dev
    dkc, dvc = to_dev(kc), to_dev(vc)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    scale = 1.0 / np.sqrt(d)
    ops.decode_append(out, to_dev(q), to_dev(key), to_dev(value), dkc, dvc, to_dev(bt), to_dev(lens), scale)
    torch.cuda.synchronize()
    okc, ovc = kc.copy(), vc.copy()
    oracle.reshape_and_cache(key, value, okc, ovc, slots)
    assert to_host(dkc).tobytes() == okc.tobytes()
    assert to_host(dvc).tobytes() == ovc.tobytes()
    got = widen_dev(out)
    assert np.all(got[lens == 0] == 0.0)
    ref = oracle.decode(q, okc, ovc, bt, lens, scale)
    assert_attention_close(got, ref, "bf16", f"fused S=8192 hq{hq}/hkv{hkv}/d{d}")


# ---------------------------------------------------------------- large pools and groups
def _scatter_to_big_pool(kc_small, vc_small, bt_small, nb_big, rng):
    """Place the blocks of a compact pool at chosen ids of a pool of nb_big
    blocks (allocated on the GPU, never read elsewhere).  Returns the device
    caches and the remapped block table; the oracle keeps the compact pool
    (its result does not depend on block ids)."""
    nb_small = kc_small.shape[0]
    # half the blocks beyond 4 GiB of byte offset, half near the start
    hi = rng.choice(np.arange(nb_big - 4096, nb_big), size=nb_small - nb_small // 2, replace=False)
    lo = rng.choice(np.arange(0, 4096), size=nb_small // 2, replace=False)
    new_id = np.concatenate([lo, hi]).astype(np.int64)
    rng.shuffle(new_id)
    bt_big = np.where(bt_small >= 0, new_id[np.maximum(bt_small, 0)], -1).astype(np.int32)
    from tests._gpu import to_dev
    shape = (nb_big,) + kc_small.shape[1:]
    dt = torch.bfloat16 if kc_small.dtype == np.uint16 else torch.uint8
    kbig = torch.empty(shape, dtype=dt, device="cuda")
    vbig = torch.empty(shape, dtype=dt, device="cuda")
    idx = torch.from_numpy(new_id).cuda()
    kbig[idx] = to_dev(kc_small)
    vbig[idx] = to_dev(vc_small)
    return kbig, vbig, bt_big


def test_decode_and_prefill_in_a_pool_beyond_4gib():
    """Blocks whose byte offsets exceed 2^32 (a 6 GiB pool per cache): every
    address computation must be 64-bit.  Unfused and fused decode, and prefill."""
    from tests._gpu import to_dev
    rng = np.random.default_rng(4242)
    hq, hkv, d = 32, 8, 128
    lens = [300, 1, 17, 1000]
    q, kc, vc, bt, cl = _random_bf16_case(rng, hq, hkv, d, lens, spare_blocks=2)
    nb_big = 196608                                   # 32 KiB blocks: 6 GiB per cache
    assert (nb_big - 4096) * 16 * hkv * d * 2 > 2 ** 32
    kbig, vbig, bt_big = _scatter_to_big_pool(kc, vc, bt, nb_big, rng)
    print(f"[gpu] pool beyond 4 GiB: {kbig.numel() * 2 / 2**30:.1f} GiB per cache", flush=True)
    ref = oracle.decode(q, kc, vc, bt, cl, 0.09)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
    ops.decode(out, to_dev(q), kbig, vbig, to_dev(bt_big), to_dev(cl), 0.09)
    torch.cuda.synchronize()
    assert_attention_close(widen_dev(out), ref, "bf16", "decode, pool > 4 GiB")
    # fused: the new token of each sequence goes to a slot beyond 4 GiB or near 0
    key = _bf16_bits(rng, (len(lens), hkv, d))
    value = _bf16_bits(rng, (len(lens), hkv, d))
    okc, ovc = kc.copy(), vc.copy()
    slots = np.array([int(bt[i, (n - 1) // 16]) * 16 + (n - 1) % 16 for i, n in enumerate(lens)], np.int32)
    oracle.reshape_and_cache(key, value, okc, ovc, slots)
    ops.decode_append(out, to_dev(q), to_dev(key), to_dev(value), kbig, vbig, to_dev(bt_big), to_dev(cl), 0.09)
    torch.cuda.synchronize()
    assert_attention_close(widen_dev(out), oracle.decode(q, okc, ovc, bt, cl, 0.09), "bf16", "fused, pool > 4 GiB")
    big_slots = [int(bt_big[i, (n - 1) // 16]) * 16 + (n - 1) % 16 for i, n in enumerate(lens)]
    for i, sl in enumerate(big_slots):
        got = kbig.view(-1, hkv, d)[sl].view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(got, key[i]), f"appended K row {i} (slot {sl})"
    # prefill: the last 40 tokens of sequence 3 as a chunk over the same pool
    qsl = np.array([0, 40], np.int32)
    pq = _bf16_bits(rng, (40, hq, d))
    pout = torch.empty((40, hq, d), dtype=torch.bfloat16, device="cuda")
    ops.prefill_chunk(pout, to_dev(pq), kbig, vbig, to_dev(bt_big[3:4]), to_dev(qsl), to_dev(cl[3:4]), 0.09)
    torch.cuda.synchronize()
    pref = oracle.prefill(pq, okc, ovc, bt[3:4], qsl, cl[3:4], 0.09)
    assert_attention_close(widen_dev(pout), pref, "bf16", "prefill, pool > 4 GiB")


@pytest.mark.parametrize("waves", [8, 12, 16, 20, 256, 300])
def test_decode_merge_paths(waves):
    """One long context split over every wave of a small grid (one kv head:
    each wave is a wave group of its own, so the context has about as many
    parts as there are waves).  That reaches each way the merge kernel folds
    a segment: 8 parts (one batch of records), 12 and 16 (a second batch), 20
    and 256 (the two-pass merge for many parts), 300 (beyond the two-pass
    limit, batched again)."""
    rng = np.random.default_rng(900 + waves)
    q, kc, vc, bt, lens = _random_bf16_case(rng, 4, 1, 128, [8192, 33, 1])
    with ops.decode_launch(waves=waves):
        got = _decode_bf16(q, kc, vc, bt, lens, 0.05)
    assert_attention_close(got, oracle.decode(q, kc, vc, bt, lens, 0.05), "bf16", f"waves {waves}")


@pytest.mark.parametrize("hq,hkv,d", [(64, 1, 128), (128, 2, 64)])
def test_decode_largest_group(hq, hkv, d):
    """64 query heads per kv head, the most a call takes (8 head groups of 8)."""
    rng = np.random.default_rng(hq + d)
    q, kc, vc, bt, lens = _random_bf16_case(rng, hq, hkv, d, [1, 50, 700], spare_blocks=5)
    got = _decode_bf16(q, kc, vc, bt, lens, 0.07)
    assert_attention_close(got, oracle.decode(q, kc, vc, bt, lens, 0.07), "bf16", f"group {hq // hkv}")


@pytest.mark.parametrize("fused", [False, True])
def test_decode_workspace_reused(fused):
    """One workspace across calls of different shapes, largest first: each call
    matches the oracle, whatever earlier calls left in the workspace.  The
    shapes split contexts over a handful of waves, over every wave of the grid
    (65536 tokens), and over waves whose share is smaller than one block."""
    from tests._gpu import to_dev
    rng = np.random.default_rng(8080 + fused)
    hq, hkv, d = 32, 8, 128
    ws = torch.zeros(ops.decode_workspace_size(64, hq, hkv, d, 4096), dtype=torch.uint8, device="cuda")
    cases = [[65536, 3000, 17, 1, 64],
             rng.integers(1, 3000, 48).tolist(),
             [40, 1, 300, 5],
             [1, 1, 2]]
    for i, lens in enumerate(cases):
        print(f"[gpu] workspace reuse fused={fused} case={i} lens={lens[:6]}", flush=True)
        q, kc, vc, bt, lens_a = _random_bf16_case(rng, hq, hkv, d, lens)
        scale = 1.0 / np.sqrt(d)
        out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda")
        dkc, dvc = to_dev(kc), to_dev(vc)
        if fused:
            s = len(lens_a)
            key = _bf16_bits(rng, (s, hkv, d))
            value = _bf16_bits(rng, (s, hkv, d))
            slots = np.array([int(bt[j, (n - 1) // 16]) * 16 + (n - 1) % 16 for j, n in enumerate(lens_a)],
                             np.int32)
            ops.decode_append(out, to_dev(q), to_dev(key), to_dev(value), dkc, dvc, to_dev(bt), to_dev(lens_a),
                              scale, workspace=ws)
            oracle.reshape_and_cache(key, value, kc, vc, slots)
        else:
            ops.decode(out, to_dev(q), dkc, dvc, to_dev(bt), to_dev(lens_a), scale, workspace=ws)
        torch.cuda.synchronize()
        if fused:
            assert to_host(dkc).tobytes() == kc.tobytes()
            assert to_host(dvc).tobytes() == vc.tobytes()
        ref = oracle.decode(q, kc, vc, bt, lens_a, scale)
        assert_attention_close(widen_dev(out), ref, "bf16", f"workspace reuse case {i}")


@pytest.mark.parametrize("dtype,hq,hkv", [("f32", 16, 16), ("bf16", 32, 32)])
def test_decode_append_many_kv_heads(dtype, hq, hkv):
    """Fused append with one query head per kv head and many kv heads: a new
    token's K row (Hkv * D * e bytes, 512 vectors of 16 bytes here) is wider
    than one pass of the merge workgroup's copy (4 vectors for each of its 64
    threads), so the copy into the cache takes several chunks."""
    from tests._gpu import to_dev
    rng = np.random.default_rng(515 + hq)
    d = 128
    lens = [1, 17, 40, 200, 33]
    print(f"[gpu] fused many kv heads dtype={dtype} hq={hq} hkv={hkv}", flush=True)
    q, kc, vc, bt, lens_a = _random_bf16_case(rng, hq, hkv, d, lens)
    s = len(lens_a)
    key = _bf16_bits(rng, (s, hkv, d))
    value = _bf16_bits(rng, (s, hkv, d))
    if dtype == "f32":  # the same values, exactly, as fp32 (NaN poison stays NaN)
        def f32(x):
            return (x.astype(np.uint32) << 16).view(np.float32)
        q, kc, vc, key, value = f32(q), f32(kc), f32(vc), f32(key), f32(value)
    slots = np.array([int(bt[j, (n - 1) // 16]) * 16 + (n - 1) % 16 for j, n in enumerate(lens_a)], np.int32)
    dkc, dvc = to_dev(kc), to_dev(vc)
    dq = to_dev(q)
    out = torch.empty_like(dq)
    scale = 1.0 / np.sqrt(d)
    ops.decode_append(out, dq, to_dev(key), to_dev(value), dkc, dvc, to_dev(bt), to_dev(lens_a), scale)
    torch.cuda.synchronize()
    oracle.reshape_and_cache(key, value, kc, vc, slots)
    assert to_host(dkc).tobytes() == kc.tobytes()
    assert to_host(dvc).tobytes() == vc.tobytes()
    ref = oracle.decode(q, kc, vc, bt, lens_a, scale)
    assert_attention_close(widen_dev(out), ref, dtype, f"fused many kv heads {dtype}")
