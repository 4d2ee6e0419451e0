"""Rare paths of the fused top-k and the selection, forced from the host, on the GPU.

* Exact fallback (K4) forced on every workload format: MXFP4 with 32 heads (four rows per
  wave in the score kernel, two in the fallback) and paged e4m3 keys, with the threshold
  forced to +inf (every sampled row underflows), to -inf (rows longer than the slab
  overflow), on every third row, and with a small slab; key spans within one fallback
  chunk and across many (the queued rows then re-scored by many workgroups, the first
  32 of them, and the rest row by row), and rows of 2^18 keys or more (the fallback's
  sampled select with the long-row sample).  The result must equal the oracle's selection
  over the GPU's materialised scores, bit for bit.
* The slab select's tie-buffer overflow: more than 4096 equal candidates at the k-th
  value (every key a candidate: threshold -inf and a slab as long as the row), and the
  tie-capacity hook that sends ordinary rows through the rescan.
* Rows with exactly k visible keys (k = 512 and 2048) and the slab-size edges.
* Launches of 65,536 rows or more (flat 1-D grids: the LiteTopK page, section 3, reports a
  grid.y limit failing at that many rows).
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_score_amd as sai
from sparse_attention_indexer_score_amd import workloads as wl
from helpers import e4m3_problem, check_topk_invariants

pytestmark = pytest.mark.gpu


def lengths(p):
    return (p.ke.astype(np.int64) - p.ks.astype(np.int64)).astype(np.int32)


def gpu_scores(dp, p):
    V = lengths(p)
    return sai.idx_score(dp, ld=max(1, int(V.max()))).cpu().numpy(), V


def same_sets(a, b, what):
    a, b = np.sort(np.asarray(a), axis=1), np.sort(np.asarray(b), axis=1)
    bad = np.nonzero(np.any(a != b, axis=1))[0]
    assert len(bad) == 0, f"{what}: {len(bad)} rows differ, first {bad[:5].tolist()}"


FAMILIES = {
    "long_mxfp4_32h": lambda: wl.long_context(rows=40, num_keys=12000, band_keys=2000, topk=256, seed=61),
    "decode_paged": lambda: wl.decode(num_req=6, ctx_lo=3000, ctx_hi=20000, topk=256, seed=62),
    "prefill_e4m3_64h": lambda: wl.prefill(rows=40, num_keys=5000, topk=256, seed=8),
    # key spans of many 4K-key chunks: queued rows are re-scored by the parallel pass
    # (the first 32 queued rows) and by the per-row pass (the rest)
    "long_mxfp4_32h_wide": lambda: wl.long_context(rows=40, num_keys=40000, band_keys=3000, topk=256, seed=63),
    "decode_paged_wide": lambda: wl.decode(num_req=10, ctx_lo=20000, ctx_hi=60000, topk=256, seed=64),
    # rows of 2^18 keys or more: the fallback's select takes the long-row sample
    "long_mxfp4_32h_300k": lambda: wl.long_context(rows=8, num_keys=300000, band_keys=3000, topk=256, seed=65),
}


@pytest.mark.parametrize("family", sorted(FAMILIES))
@pytest.mark.parametrize("mode,row_mod,cap", [(1, 0, 0), (2, 0, 0), (1, 3, 0), (0, 0, 512), (2, 5, 1500)])
def test_forced_fallback_on_every_format(family, mode, row_mod, cap):
    p = FAMILIES[family]()
    k = 256
    dp = sai.DeviceProblem.from_host(p)
    dp.debug = sai.IdxDebug(cap=cap, threshold_mode=mode, threshold_row_mod=row_mod)
    sc, V = gpu_scores(dp, p)
    ref = oracle.select_rows(sc, V, k)
    got, st = sai.idx_fused_topk(dp, k, stats=True)
    same_sets(got.cpu().numpy(), ref, f"{family} forced mode={mode} row_mod={row_mod} cap={cap}")
    capv = cap if cap > 0 else 4 * k
    forced = [r for r in range(p.rows) if mode and (row_mod <= 0 or r % row_mod == 0)]
    expect_min = sum(1 for r in forced if (mode == 1 and V[r] > 0) or (mode == 2 and V[r] > capv))
    assert st["fallback_rows"] >= expect_min
    print(f"[rare] {family} mode={mode} row_mod={row_mod} cap={cap}: fallback rows {st['fallback_rows']}",
          flush=True)
    if mode in (1, 2) and row_mod == 0:
        assert st["fallback_rows"] > 0


def zero_key_problem(rows=4, n=6000, nzero=5000, topk=1100, seed=70):
    """Integer e4m3 inputs (exact scores): n keys of which nzero are the zero vector (score
    exactly 0, all tied) at random positions; the rest random integers (scores mostly > 0)."""
    rng = np.random.default_rng(seed)
    q = rng.integers(-4, 5, size=(rows, 32, 128)).astype(np.float32)
    w = rng.integers(0, 4, size=(rows, 32)).astype(np.float32)
    keys = rng.integers(-4, 5, size=(n, 128)).astype(np.float32)
    keys[rng.choice(n, size=nzero, replace=False)] = 0.0
    ke = np.array([n, n - 7, n - 300, n - 100][:rows], dtype=np.int32)
    ks = np.array([0, 5, 0, 100][:rows], dtype=np.int32)
    return e4m3_problem(q, w, keys, ks, ke, topk=topk, heads=32)


def test_slab_select_tie_overflow():
    """Every key a candidate (threshold -inf, slab as long as the row), and more than 4096
    candidates tied at the k-th value (0): the slab select's boundary bin overflows the tie
    buffer and the row is resolved by rescans.  Exact integer scores: equal to the oracle's
    own selection (ties to the lower index)."""
    p = zero_key_problem()
    dp = sai.DeviceProblem.from_host(p)
    V = lengths(p)
    ref = oracle.topk(p)
    for r in range(p.rows):
        s = oracle.row_scores(p, r)
        kth = np.sort(s)[::-1][p.topk - 1]
        assert kth == 0.0 and np.sum(s == 0.0) > 4096, "the construction must tie more than 4096 keys at the k-th value"
    dp.debug = sai.IdxDebug(cap=8192, threshold_mode=2)
    got, st = sai.idx_fused_topk(dp, p.topk, stats=True)
    assert st["fallback_rows"] == 0 and st["max_count"] <= 8192     # the slab select handled every row
    same_sets(got.cpu().numpy(), ref, "slab select with tie overflow")
    dp.debug = None
    same_sets(sai.idx_fused_topk(dp, p.topk).cpu().numpy(), ref, "default route")
    sc, _ = gpu_scores(dp, p)
    for split in (0, 4):
        sel = sai.idx_select(torch.from_numpy(sc).cuda(), torch.from_numpy(V).cuda(), p.topk, split=split)
        same_sets(sel.cpu().numpy(), ref, f"idx_select split={split}")


@pytest.mark.parametrize("tie_cap", [1, 64, 700])
def test_tie_cap_hook_forces_rescans(tie_cap):
    """A small tie capacity sends ordinary slab rows, and the fallback's rows, through the
    rescan path; the result is unchanged."""
    p = wl.long_context(rows=24, num_keys=9000, band_keys=1500, topk=512, seed=71)
    dp = sai.DeviceProblem.from_host(p)
    sc, V = gpu_scores(dp, p)
    ref = oracle.select_rows(sc, V, 512)
    dp.debug = sai.IdxDebug(tie_cap=tie_cap)
    same_sets(sai.idx_fused_topk(dp, 512).cpu().numpy(), ref, f"slab select, tie_cap={tie_cap}")
    dp.debug = sai.IdxDebug(tie_cap=tie_cap, threshold_mode=1, threshold_row_mod=2)
    got, st = sai.idx_fused_topk(dp, 512, stats=True)
    assert st["fallback_rows"] > 0
    same_sets(got.cpu().numpy(), ref, f"fallback, tie_cap={tie_cap}")


@pytest.mark.parametrize("k", [512, 2048])
def test_rows_with_exactly_k_keys(k):
    """V == k, k - 1, k + 1, cap = 4k, cap + 1, 0, 1 and a full row (integer inputs: scores and
    sets bit-exact against the oracle)."""
    cap = 4 * k
    n = cap + 800
    p = wl.tiny(rows=8, num_keys=n, topk=k, seed=72 + k)
    V = np.array([k, k - 1, k + 1, cap, cap + 1, 0, 1, n], dtype=np.int32)
    ks = np.array([0, 3, 17, 0, 700, 5, n - 1, 0], dtype=np.int32)
    p.ks, p.ke = ks, (ks + V).astype(np.int32)
    assert np.all(p.ke <= n)
    dp = sai.DeviceProblem.from_host(p)
    sc, Vd = gpu_scores(dp, p)
    for r in range(p.rows):
        assert np.array_equal(sc[r, :Vd[r]], oracle.row_scores(p, r)), r
    got, st = sai.idx_fused_topk(dp, k, stats=True)
    got = got.cpu().numpy()
    same_sets(got, oracle.topk(p), f"V edges at k={k}")
    assert st["rows_store_all"] == 6 and st["rows_sampled"] == 2    # V <= cap keeps every key
    for r in range(p.rows):
        check_topk_invariants(sc[r, :Vd[r]], got[r], k)


def test_page_slots_70000_rows():
    rng = np.random.default_rng(80)
    rows, k, num_req, max_pages = 70000, 8, 700, 16
    pt = rng.permutation(num_req * max_pages).reshape(num_req, max_pages).astype(np.int32)
    req = rng.integers(0, num_req, size=rows).astype(np.int32)
    ks = rng.integers(0, 64, size=rows).astype(np.int32)
    idx = rng.integers(-1, max_pages * 64 - 64, size=(rows, k)).astype(np.int32)
    got = sai.idx_page_slots(torch.from_numpy(idx).cuda(), torch.from_numpy(pt).cuda(), torch.from_numpy(req).cuda(),
                             ks=torch.from_numpy(ks).cuda()).cpu().numpy()
    for r in range(0, rows):
        pos = np.where(idx[r] >= 0, idx[r] + ks[r], -1)
        want = oracle.page_transform(pos, pt[req[r]])
        if not np.array_equal(got[r], want):
            raise AssertionError(f"row {r}: {got[r]} != {want}")


@pytest.mark.parametrize("split", [0, None])
def test_select_70000_rows(split):
    rng = np.random.default_rng(81)
    rows, ld, k = 70000, 256, 16
    x = rng.standard_normal((rows, ld)).astype(np.float32)
    x[:, ::7] = np.float32(0.5)                                       # ties
    n = rng.integers(0, ld + 1, size=rows).astype(np.int32)
    ref = oracle.select_rows(x, n, k)
    got = sai.idx_select(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k, split=split).cpu().numpy()
    same_sets(got, ref, f"70000 rows, split={split}")


def test_fused_66000_rows():
    """66,000 rows of up to 1024 integer-valued e4m3 keys, k = 64 (cap 256: rows longer than
    that are sampled): fused == idx_select(idx_score) on every row and == the oracle on every
    250th row (exact scores)."""
    rows, n, k = 66000, 1024, 64
    p = wl.tiny(rows=rows, num_keys=n, topk=k, seed=82)
    rng = np.random.default_rng(83)
    p.ks = np.zeros(rows, dtype=np.int32)
    p.ke = rng.integers(1, n + 1, size=rows).astype(np.int32)
    dp = sai.DeviceProblem.from_host(p)
    got, st = sai.idx_fused_topk(dp, k, stats=True)
    got = got.cpu().numpy()
    assert st["rows_sampled"] + st["rows_store_all"] == rows
    sc = sai.idx_score(dp, ld=n)
    sel = sai.idx_select(sc, dp.ke - dp.ks, k).cpu().numpy()
    same_sets(got, sel, "fused vs idx_select(idx_score)")
    sample = list(range(0, rows, 250)) + [rows - 1]
    same_sets(got[sample], oracle.topk(p, rows=sample), "fused vs oracle (sampled rows)")
    sch = sc.cpu().numpy()
    for r in sample[::10]:
        assert np.array_equal(sch[r, :p.ke[r]], oracle.row_scores(p, r)), r


@pytest.mark.parametrize("k", [512, 2048])
def test_select_long_rows(k):
    """Rows of pitch >= 2^18 (the long-row sample: 6144 keys in runs of 8): lengths from
    below the candidate buffer to the whole pitch, with clustered runs of high values (as
    the long workload plants them) and ties; every row equals the oracle's selection, with
    the sampled route and with one workgroup per row forced."""
    rng = np.random.default_rng(90 + k)
    rows, ld = 20, 300000
    x = rng.standard_normal((rows, ld)).astype(np.float32)
    for r in range(rows):                     # runs of 16..64 high values, about 2k in all
        for _ in range(rng.integers(20, 60)):
            at, ln = int(rng.integers(0, ld - 64)), int(rng.integers(16, 65))
            x[r, at:at + ln] = (3.0 + 0.5 * rng.standard_normal(ln)).astype(np.float32)
    x[:, ::97] = np.float32(2.5)              # ties
    n = np.array([ld, ld - 1, 1000, 6144, 6145, 2 * k, k, k - 1, 0, 262144] +
                 list(rng.integers(0, ld + 1, size=rows - 10)), dtype=np.int32)
    ref = oracle.select_rows(x, n, k)
    xd, nd = torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda()
    for split in (None, 0):
        got = sai.idx_select(xd, nd, k, split=split).cpu().numpy()
        same_sets(got, ref, f"long rows, k={k}, split={split}")
