"""Parity of the HIP path (through the C ABI) with the CPU oracle, on the GPU.

Bars:
* integer-valued e4m3 inputs: scores bit-exact, index sets bit-exact;
* real-valued inputs: |gpu - oracle| <= 1e-4 + 1e-5 * |oracle| per score; selection over
  the GPU's own scores bit-exact (oracle select == idx_select == idx_fused_topk), which
  also gives selected-value recall 1.0; against the oracle's scores every selected key
  lies within that tolerance of the oracle's k-th value.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_score_amd as sai
from sparse_attention_indexer_score_amd import workloads as wl
from helpers import golden, e1_problem, check_topk_invariants

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-5


def dev(p):
    return sai.DeviceProblem.from_host(p)


def lengths(p):
    return (p.ke.astype(np.int64) - p.ks.astype(np.int64)).astype(np.int32)


def gpu_scores(dp, p):
    V = lengths(p)
    ld = max(1, int(V.max()))
    return sai.idx_score(dp, ld=ld).cpu().numpy(), V


def assert_same_sets(a, b, what=""):
    a = np.sort(np.asarray(a), axis=1)
    b = np.sort(np.asarray(b), axis=1)
    bad = np.nonzero(np.any(a != b, axis=1))[0]
    assert len(bad) == 0, f"{what}: {len(bad)} rows differ, first {bad[:5]}"


def check_scores_close(p, sc, rows):
    kd = oracle.all_keys(p) if p.page_table is None else None
    worst = 0.0
    for r in rows:
        V = int(p.ke[r] - p.ks[r])
        ref = oracle.row_scores(p, r, kd_all=kd).astype(np.float64)
        got = sc[r, :V].astype(np.float64)
        err = np.abs(got - ref)
        lim = ATOL + RTOL * np.abs(ref)
        if V:
            worst = max(worst, float((err / lim).max()))
        assert np.all(err <= lim), f"row {r}: max err {err.max():.3g} at {int(np.argmax(err - lim))}"
    print(f"[scores] {p.name} ({p.fmt}, H={p.heads}): max |err| / (1e-4 + 1e-5 |oracle|) = {worst:.3g} "
          f"over {len(list(rows))} rows", flush=True)
    return worst


def full_check(p, k, score_rows=None, fused_kw=None):
    """Scores within tolerance (sampled rows), selection bit-exact over the GPU scores,
    fused == idx_select(idx_score), invariants and tolerance-aware oracle agreement."""
    dp = dev(p)
    sc, V = gpu_scores(dp, p)
    rows = range(p.rows) if score_rows is None else score_rows
    check_scores_close(p, sc, rows)
    ref_sel = oracle.select_rows(sc, V, k)                     # oracle select over the GPU's scores
    sel = sai.idx_select(torch.from_numpy(sc).cuda(), torch.from_numpy(V).cuda(), k).cpu().numpy()
    assert_same_sets(sel, ref_sel, "idx_select vs oracle select")
    fused, st = sai.idx_fused_topk(dp, k, stats=True, **(fused_kw or {}))
    fused = fused.cpu().numpy()
    assert_same_sets(fused, ref_sel, "idx_fused_topk vs oracle select")
    for r in range(p.rows):
        check_topk_invariants(sc[r, :V[r]], fused[r], k)
        assert oracle.selected_value_recall(sc[r, :V[r]], fused[r], k) == 1.0
    kd = oracle.all_keys(p) if p.page_table is None else None
    for r in rows:
        ref = oracle.row_scores(p, r, kd_all=kd)
        n = min(k, len(ref))
        if n == 0:
            continue
        kth = np.sort(ref)[::-1][n - 1]
        got = ref[fused[r, :n]]
        assert np.all(got >= kth - (ATOL + RTOL * abs(kth))), f"row {r}: a selected key is below the oracle k-th value"
    return st


# ----------------------------------------------------------------------------- hand-worked

def test_e1_scores_and_topk_on_gpu():
    g = golden("e1_scoring_ties_causal.json")
    p = e1_problem(heads=32)
    dp = dev(p)
    sc = sai.idx_score(dp, ld=8).cpu().numpy()
    assert list(sc[0]) == g["scores"]
    for c in g["cases"]:
        pp = e1_problem(ke=c["ke"], topk=c["k"], heads=32)
        got = sai.idx_fused_topk(dev(pp), c["k"]).cpu().numpy()[0]
        assert sorted(got) == sorted(c["selected"])


def test_e2_key_scale_on_gpu():
    g = golden("e2_key_scale.json")
    p = e1_problem(k_scale=g["kscale"], heads=64)
    assert list(sai.idx_score(dev(p), ld=8).cpu().numpy()[0]) == g["scores"]
    for c in g["cases"]:
        got = sai.idx_fused_topk(dev(e1_problem(ke=c["ke"], k_scale=g["kscale"], topk=c["k"], heads=64)), c["k"])
        assert sorted(got.cpu().numpy()[0]) == sorted(c["selected"])


def test_e3_signed_zeros_on_gpu():
    g = golden("e3_signed_zero_ties.json")
    x = np.array([float(v) for v in g["x"]], dtype=np.float32)
    for c in g["cases"]:
        got = sai.idx_select(torch.from_numpy(x[None]).cuda(), torch.tensor([8], dtype=torch.int32).cuda(), c["k"])
        assert sorted(got.cpu().numpy()[0]) == sorted(c["selected"])


# ----------------------------------------------------------------------------- workloads

def test_tiny_integer_workload_bit_exact():
    """64 rows x 4096 keys, 32 heads, integer e4m3: scores and sets bit-exact vs the oracle."""
    p = wl.tiny()
    dp = dev(p)
    sc, V = gpu_scores(dp, p)
    for r in range(p.rows):
        assert np.array_equal(sc[r, :V[r]], oracle.row_scores(p, r)), f"row {r}"
    ref = oracle.topk(p)
    assert_same_sets(sai.idx_fused_topk(dp, p.topk).cpu().numpy(), ref, "fused vs oracle")
    sel = sai.idx_select(torch.from_numpy(sc).cuda(), torch.from_numpy(V).cuda(), p.topk).cpu().numpy()
    assert_same_sets(sel, ref, "select vs oracle")


@pytest.mark.parametrize("split", [None, 0, 4, 8])
def test_selection_workload_bit_exact(split):
    """64 rows x 131072 fp32 with dense ties and a planted band; k = 2048."""
    sp = wl.select_only()
    ref = oracle.select_rows(sp.x, sp.length, sp.topk)
    got = sai.idx_select(torch.from_numpy(sp.x).cuda(), torch.from_numpy(sp.length).cuda(), sp.topk,
                         split=split).cpu().numpy()
    assert_same_sets(got, ref, f"split={split}")


def test_prefill_family_reduced():
    p = wl.prefill(rows=96, num_keys=16384)
    st = full_check(p, 2048, score_rows=range(0, 96, 7))
    assert st["rows_sampled"] > 0


def test_prefill_family_small_k():
    p = wl.prefill(rows=64, num_keys=6000, topk=512, seed=13)
    st = full_check(p, 512, score_rows=range(0, 64, 9))
    assert st["rows_sampled"] == 64


def test_long_family_reduced_mxfp4():
    p = wl.long_context(rows=64, num_keys=32768, band_keys=4096)
    st = full_check(p, 2048, score_rows=range(0, 64, 9))
    assert st["rows_sampled"] == 64


def test_decode_family_reduced_paged():
    p = wl.decode(num_req=6, ctx_lo=3000, ctx_hi=40000)
    st = full_check(p, 2048, score_rows=range(0, p.rows, 5))
    assert st["rows_store_all"] + st["rows_sampled"] == p.rows


def test_mxfp4_64_heads():
    """MXFP4 keys with 64 heads (two rows per wave, two head tiles per row)."""
    p = wl.long_context(rows=40, num_keys=20000, heads=64, band_keys=3000, seed=31)
    st = full_check(p, 1024, score_rows=range(0, 40, 6))
    assert st["rows_sampled"] + st["rows_store_all"] == p.rows


def test_paged_32_heads():
    """Paged e4m3 keys with 32 heads."""
    p = wl.decode(num_req=5, ctx_lo=3000, ctx_hi=25000, heads=32, seed=37)
    st = full_check(p, 2048, score_rows=range(0, p.rows, 3))
    assert st["rows_sampled"] + st["rows_store_all"] == p.rows


def test_paged_row_pairs_straddling_requests():
    """Three rows per request: row pairs (0,1), (2,3), ... mix requests, so the paged kernel
    scores such a pair one row at a time, each through its own request's pages."""
    p = wl.decode(num_req=7, q_len=3, ctx_lo=2500, ctx_hi=30000, seed=17)
    st = full_check(p, 1024, score_rows=range(p.rows))
    assert st["rows_store_all"] + st["rows_sampled"] == p.rows


def test_decode_persistent_workgroups():
    """A decode batch large enough that the paged score + filter launch takes most of its work
    items by ticket: 40 requests of up to 262,144 keys give 64 key chunks x 40 row quads,
    against two persistent workgroups per CU."""
    p = wl.decode(num_req=40, ctx_lo=8192, ctx_hi=262144, seed=19)
    st = full_check(p, 2048, score_rows=[0, p.rows - 1])
    assert st["rows_store_all"] + st["rows_sampled"] == p.rows


# ----------------------------------------------------------------------------- edges

@pytest.mark.parametrize("k", [1, 7, 100, 1000, 2048])
def test_fused_k_range_ragged_mxfp4(k):
    """k from 1 to the maximum on MXFP4 keys with a ragged shape: 21 rows (one full 16-row
    block and a partial one), 9001 keys (a partial last tile), rows starting at different
    keys.  Small k gives odd sample strides down to 1; k = 2048 keeps most rows whole."""
    p = wl.long_context(rows=21, num_keys=9001, band_keys=1000, seed=40 + k)
    p.ks = np.minimum((np.arange(p.rows, dtype=np.int32) * 37) % 500, p.ke).astype(np.int32)
    st = full_check(p, k, score_rows=range(0, p.rows, 4))
    assert st["rows_sampled"] + st["rows_store_all"] == p.rows


def test_edge_lengths_e4m3():
    """Empty rows, V < k, V > k, V == cap, V == cap + 1 and full rows, with offset starts;
    k = 512, cap = 2048 (V == k exactly: test_gpu_rare_paths.py)."""
    p = wl.tiny(rows=12, num_keys=4096, topk=512, seed=5)
    ke = np.array([0, 1, 7, 511, 512, 513, 2048, 2049, 3000, 4095, 4096, 4096], dtype=np.int32)
    ks = np.array([0, 0, 3, 0, 100, 0, 0, 0, 1000, 0, 0, 37], dtype=np.int32)
    ke = np.maximum(ke, ks)
    ke[1] = 1
    p.ks, p.ke = ks, ke
    dp = dev(p)
    sc, V = gpu_scores(dp, p)
    for r in range(p.rows):
        assert np.array_equal(sc[r, :V[r]], oracle.row_scores(p, r))
    ref = oracle.topk(p)
    assert_same_sets(sai.idx_fused_topk(dp, 512).cpu().numpy(), ref, "fused")


@pytest.mark.parametrize("fmt,num_keys", [("e4m3", 127), ("e4m3", 128), ("e4m3", 129), ("e4m3", 1000),
                                          ("mxfp4", 255), ("mxfp4", 256), ("mxfp4", 257), ("mxfp4", 1800)])
def test_stage_boundaries_at_key_array_end(fmt, num_keys):
    """Key tiles are staged 128 (e4m3) or 256 (MXFP4) keys at a time from a workgroup's first
    tile: a stage wholly inside the key array is loaded as a dense copy, one that reaches past
    its end through the per-key clamped path.  Key counts just below, at and above a stage,
    rows starting at different tiles and some ending early put the array's end at every
    kind of position in the last stage; scores of every row against the oracle, selection
    bit-exact over the GPU's scores (k = 64: rows over 256 keys are sampled)."""
    rows = 24
    if fmt == "e4m3":
        p = wl.prefill(rows=rows, num_keys=num_keys, topk=64, seed=500 + num_keys)
    else:
        p = wl.long_context(rows=rows, num_keys=num_keys, band_keys=64, topk=64, seed=500 + num_keys)
    r = np.arange(rows)
    p.ke = (num_keys - (r % 3) * (r % 5)).astype(np.int32)
    p.ks = np.minimum((r * 37) % max(1, num_keys // 2), p.ke).astype(np.int32)
    st = full_check(p, 64, score_rows=range(rows))
    assert st["rows_sampled"] + st["rows_store_all"] == rows


def test_select_all_equal_rows_force_rescan():
    rows, ld = 3, 131072
    x = np.full((rows, ld), 0.5, dtype=np.float32)
    x[1, ::2] = -0.0
    x[1, 1::2] = 0.0
    n = np.array([ld, ld, 5000], dtype=np.int32)
    ref = oracle.select_rows(x, n, 2048)
    for split in (0, 4):
        got = sai.idx_select(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), 2048, split=split).cpu().numpy()
        assert_same_sets(got, ref, f"split={split}")


def _sample_positions(n, seg=64, nseg=32):
    """Positions the single-workgroup select samples: 32 runs of 64 consecutive elements,
    run g starting at floor(g (n - 64) / 31)."""
    starts = [i * (n - seg) // (nseg - 1) for i in range(nseg)]
    return np.concatenate([np.arange(a, a + seg) for a in starts])


@pytest.mark.parametrize("workspace", [True, False])
def test_select_sampled_threshold_misjudged(workspace):
    """Rows built so the sampled threshold misjudges them: too few candidates (the sample
    holds the only large values), too many (the sample holds the only small ones), a
    sample that lands exactly on the k-th value, and a short row below the buffer size.
    Every case must still equal the oracle (the exact fallback takes over), with and
    without a workspace passed through the C ABI."""
    rng = np.random.default_rng(21)
    ld, k = 65536, 2048
    x = rng.uniform(0.0, 0.5, size=(5, ld)).astype(np.float32)
    pos = _sample_positions(ld)
    x[0, pos[:300]] = 1.0 + rng.uniform(0, 1e-3, size=300).astype(np.float32)   # count(>= T) < k
    x[1] += 1.0                                                                  # count(>= T) > buffer
    x[1, pos] = rng.uniform(0.0, 0.5, size=len(pos)).astype(np.float32)
    x[2, :] = np.float32(0.25)                                                   # all equal: rescan
    x[3, pos] = np.float32(0.75)                                                 # 2048 equal sample values
    n = np.array([ld, ld, ld, ld, 6000], dtype=np.int32)
    ref = oracle.select_rows(x, n, k)
    got = sai.idx_select(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k, split=0,
                         workspace=workspace).cpu().numpy()
    assert_same_sets(got, ref, f"sampled select (workspace={workspace})")


@pytest.mark.parametrize("workspace", [True, False])
def test_select_short_and_empty_rows(workspace):
    rng = np.random.default_rng(3)
    x = rng.standard_normal((5, 300)).astype(np.float32)
    n = np.array([0, 1, 10, 299, 300], dtype=np.int32)
    ref = oracle.select_rows(x, n, 64)
    got = sai.idx_select(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), 64,
                         workspace=workspace).cpu().numpy()
    assert_same_sets(got, ref)


@pytest.mark.parametrize("split", [0, 4])
def test_select_sampled_rows_ragged_and_unaligned(split):
    """Sampled rows (longer than the 6144-entry candidate buffer) whose streaming pass ends in
    a partial step, with starts 0-3 floats past a 16-byte boundary (unaligned rows take the
    4-byte path): the loads past the end are clamped re-reads that must not be selected."""
    rng = np.random.default_rng(31)
    ld = 70000
    x = rng.standard_normal((8, ld)).astype(np.float32)
    rs = np.array([0, 1, 2, 3, 4, 0, 5, 0], dtype=np.int32)
    n = np.array([6145, 6145, 16383, 16385, 65537, 4097 * 4 + 3, 60000, 1], dtype=np.int32)
    k = 2048
    ref = oracle.select_rows(x, n, k, row_start=rs)
    got = sai.idx_select(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k,
                         row_start=torch.from_numpy(rs).cuda(), split=split).cpu().numpy()
    assert_same_sets(got, ref, f"split={split}")


@pytest.mark.parametrize("split", [2, 3, 7, 32])
def test_select_row_split_routes(split):
    """The row split (several workgroups per row, each appending its segment's candidates to
    the row's buffer; one workgroup per row refines them) on rows that take each of its
    routes: long rows with a planted band of high runs (refinement), one whose top values
    fill its last quarter (a segment overflows: exact multi-pass route), one whose sample
    holds the only large values (fewer candidates than k: exact route), rows shorter than
    the split length and with n <= k (selected whole), and an empty row.  The workspace
    starts filled with garbage, so the first call finds the per-row counters unset (rows
    then take the exact route); the second call finds them at zero.  Both equal the oracle."""
    rng = np.random.default_rng(40 + split)
    ld, k = 131072, 2048
    x = rng.normal(0.0, 0.05, size=(8, ld)).astype(np.float32)
    for r in (0, 1):
        for _ in range(80):
            a = int(rng.integers(0, ld - 32))
            x[r, a:a + 32] = (1.0 + 0.1 * rng.standard_normal(32)).astype(np.float32)
    x[2, 3 * ld // 4:] = np.float32(2.0)
    pos = _sample_positions(ld)
    x[3, pos[:300]] = 1.0 + rng.uniform(0, 1e-3, size=300).astype(np.float32)
    n = np.array([ld, ld - 5, ld, ld, 16383, 20000, k, 0], dtype=np.int32)
    ref = oracle.select_rows(x, n, k)
    run = sai.SelectRunner(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), k, split=split)
    run.ws.fill_(0xA5)
    for call in range(2):
        got = run().cpu().numpy()
        assert_same_sets(got, ref, f"split={split}, call {call}")


def test_select_row_start_offsets():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((4, 5000)).astype(np.float32)
    rs = np.array([0, 17, 999, 4000], dtype=np.int32)
    n = np.array([5000, 3000, 4001, 1000], dtype=np.int32)
    ref = oracle.select_rows(x, n, 300, row_start=rs)
    got = sai.idx_select(torch.from_numpy(x).cuda(), torch.from_numpy(n).cuda(), 300,
                         row_start=torch.from_numpy(rs).cuda()).cpu().numpy()
    assert_same_sets(got, ref)


# ----------------------------------------------------------------------------- determinism

def test_fused_is_deterministic():
    p = wl.long_context(rows=32, num_keys=20000, band_keys=3000, topk=1024, seed=17)
    dp = dev(p)
    a = np.sort(sai.idx_fused_topk(dp, 1024).cpu().numpy(), axis=1)
    b = np.sort(sai.idx_fused_topk(dp, 1024).cpu().numpy(), axis=1)
    assert np.array_equal(a, b)


# ----------------------------------------------------------------------------- page slots

def test_page_slots_golden_e6():
    """Hand-worked page transform (LiteTopK page, section 3): page_row [7, 2]."""
    g = golden("e6_page_transform.json")
    pos = torch.tensor([g["pos"] + [0, 0, 0]], dtype=torch.int32).cuda()          # k = 8 (vector path)
    pt = torch.tensor([g["page_row"]], dtype=torch.int32).cuda()
    req = torch.zeros(1, dtype=torch.int32).cuda()
    got = sai.idx_page_slots(pos, pt, req).cpu().numpy()[0]
    assert got[:5].tolist() == g["slot"]
    pos5 = torch.tensor([g["pos"]], dtype=torch.int32).cuda()                        # k = 5 (scalar path)
    assert sai.idx_page_slots(pos5, pt, req).cpu().numpy()[0].tolist() == g["slot"]


def test_page_slots_of_fused_decode_output():
    """The fused top-k of a paged problem, mapped to physical slots, equals the oracle's
    page transform of the oracle's selection on every row (ks offsets included)."""
    p = wl.decode(num_req=5, ctx_lo=3000, ctx_hi=20000, seed=23)
    p.ks = np.minimum(p.ks + 37, p.ke).astype(np.int32)                             # nonzero first keys
    dp = dev(p)
    sc, V = gpu_scores(dp, p)
    ref_sel = oracle.select_rows(sc, V, 1024)
    fused = sai.idx_fused_topk(dp, 1024)
    got = sai.idx_page_slots(fused, dp.page_table, dp.row_req, ks=dp.ks).cpu().numpy()
    for r in range(p.rows):
        pos = np.where(ref_sel[r] >= 0, ref_sel[r] + p.ks[r], -1)
        want = oracle.page_transform(pos, p.page_table[p.row_req[r]])
        assert np.array_equal(np.sort(got[r]), np.sort(want)), r
    inplace = fused.clone()
    sai.idx_page_slots(inplace, dp.page_table, dp.row_req, ks=dp.ks, out=inplace)
    assert np.array_equal(inplace.cpu().numpy(), got)
