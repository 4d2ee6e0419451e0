"""Parity of idx_sparse_attn (the top-k's consumer) with the CPU oracle, on the GPU.

Bar: |gpu - oracle| <= output_scale * 2^-10 * max|v| + 1e-5 * |oracle| per output element,
where max|v| is over the row's valid slots of the KV head.  The kernel rounds each softmax
weight to fp16 for the PV product (relative error <= 2^-11 per weight, so the weighted mean
moves by at most 2^-11 * max|v|); the QK dot products are exact bf16 x e4m3 products summed
in fp32.  The bound takes twice that.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_score_amd as sai
from sparse_attention_indexer_score_amd import workloads as wl

pytestmark = pytest.mark.gpu


def run_gpu(a):
    dev = "cuda"
    out = sai.idx_sparse_attn(torch.from_numpy(a.q.view(np.int16)).to(dev), torch.from_numpy(a.k_cache).to(dev),
                              torch.from_numpy(a.v_cache).to(dev), torch.from_numpy(a.slots).to(dev),
                              a.softmax_scale, a.output_scale)
    return out.cpu().numpy().astype(np.float64)


def check(a, rows=None):
    got = run_gpu(a)
    rows = range(a.rows) if rows is None else rows
    sub = list(rows)
    ref = oracle.sparse_attention(a.q[sub], a.k_cache, a.v_cache, a.slots[sub], a.softmax_scale, a.output_scale)
    vd = np.abs(oracle.decode_e4m3(a.v_cache))
    hkv = a.k_cache.shape[1]
    group = a.q.shape[1] // hkv
    n = a.k_cache.shape[0]
    for i, r in enumerate(sub):
        sl = a.slots[r]
        sl = sl[(sl >= 0) & (sl < n)]
        for h in range(a.q.shape[1]):
            vmax = vd[sl, h // group, :].max() if sl.size else 0.0
            lim = a.output_scale * 2.0 ** -10 * vmax + 1e-5 * np.abs(ref[i, h])
            err = np.abs(got[r, h] - ref[i, h])
            assert np.all(err <= lim), f"row {r} head {h}: max err {err.max():.3g} (limit {lim.max():.3g})"
        if sl.size == 0:
            assert np.all(got[r] == 0.0), f"row {r} has no valid slot but a nonzero output"


def test_attn_small_ragged():
    """24 query heads over 2 KV heads, 300 slots per row (a partial last tile), short and
    empty selections, slots beyond the cache."""
    a = wl.sparse_attn(rows=40, width=300, num_slots=5000, seed=11, short_every=4)
    a.slots[5, 7] = 5000          # out of range: ignored
    a.slots[6, :] = -1
    a.slots[6, 3] = 17            # a single valid slot
    check(a)


def test_attn_masked_reads_do_not_leak():
    """Invalid slots (negative, past the cache) and the positions past the row's width in its
    last tile are read from slot 0 and masked. No row selects slot 0, so the output must not
    change, bit for bit, when slot 0's K and V bytes are e4m3 NaN codes instead of zeros."""
    a = wl.sparse_attn(rows=16, width=200, num_slots=3000, seed=12, short_every=3)
    a.slots[a.slots == 0] = 1
    a.slots[2, ::5] = -7
    a.slots[3, ::3] = 3000 + 5
    a.k_cache[0] = 0
    a.v_cache[0] = 0
    clean = run_gpu(a)
    a.k_cache[0] = 0x7F
    a.v_cache[0] = 0x7F
    poisoned = run_gpu(a)
    assert np.isfinite(poisoned).all()
    assert np.array_equal(poisoned, clean)
    a.k_cache[0] = 0
    a.v_cache[0] = 0
    check(a)  # (the oracle refuses NaN codes anywhere in the cache)


@pytest.mark.parametrize("hq,hkv", [(32, 1), (4, 4), (8, 2), (3, 1)])
def test_attn_group_shapes(hq, hkv):
    a = wl.sparse_attn(rows=9, hq=hq, hkv=hkv, width=97, num_slots=700, seed=hq + 7 * hkv, short_every=3)
    check(a)


def test_attn_scales_and_width_zero():
    a = wl.sparse_attn(rows=6, width=64, num_slots=300, seed=3, short_every=0)
    a.softmax_scale, a.output_scale = 0.5, 3.0
    check(a)
    z = wl.sparse_attn(rows=3, width=0, num_slots=10, seed=4, short_every=0)
    assert np.all(run_gpu(z) == 0.0)


def test_attn_full_size_sampled_rows():
    """512 rows x 2048 selected slots, 24 / 2 heads, a 262144-slot cache; oracle on 12 rows."""
    a = wl.sparse_attn()
    check(a, rows=[0, 1, 15, 16, 100, 255, 256, 300, 400, 479, 510, 511])


def test_attn_deterministic():
    a = wl.sparse_attn(rows=16, width=500, num_slots=4000, seed=9)
    assert np.array_equal(run_gpu(a), run_gpu(a))
