"""GPU parity: causal chunked prefill through the C ABI against the fp64 oracle.

bf16 attention must be within max-abs 2e-2 and per-(row, head) relative 1e-2
of the oracle.  At full size the oracle is evaluated on sampled rows only
(every row of a chunk is independent, so a sample is an exact check of those
rows).
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from paged_kv_cache_275_amd import ops
from paged_kv_cache_275_amd import workloads as W
from tests._gpu import DevWorkload, to_dev, widen_dev
from tests import _oracle_threads as oracle_threads
from tests._helpers import assert_attention_close

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)


def _append_and_prefill(wl):
    dw = DevWorkload(wl)
    ops.reshape_and_cache(dw.k_new, dw.v_new, dw.k_cache, dw.v_cache, dw.slot_mapping)
    ops.prefill_chunk(dw.pout, dw.pq, dw.k_cache, dw.v_cache, dw.p_block_tables, dw.p_qsl,
                      dw.p_context_lens, wl.scale)
    torch.cuda.synchronize()
    return dw


def _oracle_pool(wl):
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    oracle.reshape_and_cache(wl.k_new, wl.v_new, kc, vc, wl.slot_mapping)
    return kc, vc


@pytest.mark.parametrize("seed", [4, 104])
def test_prefill_mixed_workload_every_row(seed):
    """Full-size mixed workload, every row of the four 512-row chunks against
    the oracle (in the launch configuration the benchmark times)."""
    wl = W.make_workload("mixed_prefill", seed=seed)
    p = wl.prefill
    print(f"[gpu] prefill every row seed={seed} ctx={p.context_lens.tolist()}", flush=True)
    dw = _append_and_prefill(wl)
    kc, vc = _oracle_pool(wl)
    got = widen_dev(dw.pout)
    ref = oracle_threads.prefill(p.q, kc, vc, p.block_tables, p.query_start_loc, p.context_lens, wl.scale)
    mx, rel = assert_attention_close(got, ref, "bf16", f"prefill every row seed={seed}")
    print(f"[gpu] prefill every row seed={seed}: max-abs {mx:.3e} row-rel {rel:.3e}", flush=True)


@pytest.mark.parametrize("seed", [204])
def test_prefill_mixed_workload_sampled_rows(seed):
    """Full-size mixed workload (4 chunks of 512 rows over 1-3K prefixes)."""
    wl = W.make_workload("mixed_prefill", seed=seed)
    p = wl.prefill
    print(f"[gpu] prefill seed={seed} ctx={p.context_lens.tolist()}", flush=True)
    dw = _append_and_prefill(wl)
    kc, vc = _oracle_pool(wl)
    got = widen_dev(dw.pout)
    rng = np.random.default_rng(seed)
    rows = []
    for s in range(len(p.context_lens)):
        r0, r1 = int(p.query_start_loc[s]), int(p.query_start_loc[s + 1])
        rows += [r0, r0 + 1, r1 - 1] + list(rng.choice(np.arange(r0, r1), size=13, replace=False))
    rows = sorted(set(rows))
    # oracle on single rows: a one-row chunk whose position is the row's own
    for r in rows:
        s = int(np.searchsorted(p.query_start_loc, r, side="right") - 1)
        r0, r1 = int(p.query_start_loc[s]), int(p.query_start_loc[s + 1])
        n_row = int(p.context_lens[s]) - (r1 - 1 - r)     # tokens visible to row r
        ref = oracle.decode(p.q[r:r + 1], kc, vc, p.block_tables[s:s + 1],
                            np.array([n_row], np.int32), wl.scale)
        assert_attention_close(got[r:r + 1], ref, "bf16", f"row {r}")


@pytest.mark.parametrize("case", ["no_prefix", "ragged", "single_row", "tiny_prefix"])
def test_prefill_small_full_oracle(case):
    """Small chunks checked on every row: chunk = whole context, chunk lengths
    that are not multiples of the row tile, one-row chunks, prefixes shorter
    than a block."""
    rng = np.random.default_rng({"no_prefix": 1, "ragged": 2, "single_row": 3, "tiny_prefix": 4}[case])
    hq, hkv, d = 32, 8, 128
    if case == "no_prefix":
        chunks, prefixes = [40, 100], [0, 0]
    elif case == "ragged":
        chunks, prefixes = [33, 7, 65], [300, 17, 64]
    elif case == "single_row":
        chunks, prefixes = [1, 1, 1], [0, 15, 200]
    else:
        chunks, prefixes = [20, 9], [3, 1]
    _run_small(rng, hq, hkv, d, chunks, prefixes, 1.0 / np.sqrt(d))


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (6, 2, 64), (16, 2, 128), (32, 2, 64)])
def test_prefill_group_sizes(hq, hkv, d):
    rng = np.random.default_rng(hq * 100 + hkv + d)
    _run_small(rng, hq, hkv, d, [37, 70], [90, 5], 0.1)


def _bf16(x):
    from tests._helpers import bf16_bits_from_float
    return bf16_bits_from_float(x)


def _run_small(rng, hq, hkv, d, chunks, prefixes, scale):
    lens = [c + p for c, p in zip(chunks, prefixes)]
    s = len(chunks)
    need = [-(-n // 16) for n in lens]
    nb = 2 * sum(need) + 4
    mb = max(need)
    perm = rng.permutation(nb).astype(np.int32)
    bt = np.full((s, mb), -1, np.int32)
    off = 0
    for i, k in enumerate(need):
        bt[i, :k] = perm[off:off + k]
        off += k
    kc = np.full((nb, 16, hkv, d), 0x7FC0, np.uint16)
    vc = kc.copy()
    for i, n in enumerate(lens):
        t = np.arange(n)
        slot = bt[i, t // 16].astype(np.int64) * 16 + t % 16
        kc.reshape(-1, hkv, d)[slot] = _bf16(rng.standard_normal((n, hkv, d)))
        vc.reshape(-1, hkv, d)[slot] = _bf16(rng.standard_normal((n, hkv, d)))
    qsl = np.concatenate([[0], np.cumsum(chunks)]).astype(np.int32)
    q = _bf16(rng.standard_normal((int(qsl[-1]), hq, d)))
    cl = np.asarray(lens, np.int32)
    out = torch.empty((int(qsl[-1]), hq, d), dtype=torch.bfloat16, device="cuda")
    ops.prefill_chunk(out, to_dev(q), to_dev(kc), to_dev(vc), to_dev(bt), to_dev(qsl), to_dev(cl), scale)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, kc, vc, bt, qsl, cl, scale)
    assert_attention_close(widen_dev(out), ref, "bf16", f"chunks={chunks} prefixes={prefixes}")


@pytest.mark.parametrize("num_seqs", [600, 1100])
def test_prefill_many_sequences(num_seqs):
    """More sequences than one workgroup scans at a time (512), with empty
    chunks among them, so the item lookup crosses batches."""
    rng = np.random.default_rng(num_seqs)
    chunks = [int(x) for x in rng.integers(0, 4, num_seqs)]
    prefixes = [int(x) for x in rng.integers(0, 41, num_seqs)]
    chunks[-1] = max(chunks[-1], 1)   # the last sequence's items end the grid
    print(f"[gpu] prefill {num_seqs} sequences, {sum(chunks)} rows", flush=True)
    _run_small(rng, 4, 2, 64, chunks, prefixes, 0.125)


def test_prefill_rejects_fp32():
    q = torch.zeros((4, 4, 64), dtype=torch.float32, device="cuda")
    kc = torch.zeros((2, 16, 2, 64), dtype=torch.float32, device="cuda")
    bt = torch.zeros((1, 2), dtype=torch.int32, device="cuda")
    qsl = torch.tensor([0, 4], dtype=torch.int32, device="cuda")
    cl = torch.tensor([4], dtype=torch.int32, device="cuda")
    with pytest.raises(ops.PAError) as e:
        ops.prefill_chunk(torch.empty_like(q), q, kc, kc, bt, qsl, cl, 0.1)
    assert e.value.status == ops.PA_EUNSUPPORTED


@pytest.mark.parametrize("scale", [0.0, -0.0, -0.09])
def test_prefill_zero_and_negative_scale(scale):
    """A zero scale makes every score 0 (each row the mean of the V it sees),
    also where the causal mask cuts keys off; a negative scale flips the
    scores.  Decode on the same contexts for comparison."""
    rng = np.random.default_rng(99)
    _run_small(rng, 32, 8, 128, [33, 70, 1], [40, 0, 9], scale)
