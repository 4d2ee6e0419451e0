"""Pins of the CPU oracle to things other than itself (CPU only).

* exhaustive decode tables against torch's own fp8 / e8m0 / bf16 conversions and the
  OCP e2m1 value table;
* the hand-worked fixtures under tests/golden (E1..E7, E7 = selected-value recall);
* brute force in pure Python on tiny random inputs (decoded through torch, not the
  oracle's tables) with the top-k checked against its definition;
* closed forms: one head with unit weight and non-negative inputs reduces the score to
  a plain dot product (torch float64 matmul); a power-of-two key scale scales every
  score exactly;
* invariants of the selection on every workload family at reduced size;
* per-row offsets of the selection-only entry against selection by rank counting;
* planted mistakes: mutated copies of the oracle must fail at least one pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_indexer_score_amd import workloads as wl
from helpers import golden, e1_problem, e4m3_problem, check_topk_invariants


# ----------------------------------------------------------------------------- decoders

def test_e4m3_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.E4M3_TABLE
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero and the extremes
    assert math.copysign(1.0, got[0x80]) == -1.0 and got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9


def test_e8m0_table_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.E8M0_TABLE
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_bf16_decode_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e2m1_table_is_ocp_value_list():
    g = golden("e4_mxfp4.json")
    ref = np.array(g["e2m1_values"], dtype=np.float64)
    assert np.array_equal(oracle.E2M1_TABLE, ref)
    assert np.array_equal(np.signbit(oracle.E2M1_TABLE), np.signbit(ref))


def test_mxfp4_golden_pair_and_block_dot():
    g = golden("e4_mxfp4.json")
    packed = np.zeros((1, 64), dtype=np.uint8)
    packed[0, 0] = g["byte"]
    sf = np.full((1, 4), g["scale"], dtype=np.uint8)
    v = oracle.decode_mxfp4(packed, sf)
    assert v[0, 0] == g["pair"][0] and v[0, 1] == g["pair"][1]
    b = g["block_dot"]
    qp = np.full((1, 64), b["q_code"] | (b["q_code"] << 4), dtype=np.uint8)
    kp = np.full((1, 64), b["k_code"] | (b["k_code"] << 4), dtype=np.uint8)
    qv = oracle.decode_mxfp4(qp, np.full((1, 4), b["q_scale"], dtype=np.uint8))
    kv = oracle.decode_mxfp4(kp, np.full((1, 4), b["k_scale"], dtype=np.uint8))
    assert float(qv[0, :32] @ kv[0, :32]) == b["dot"]


def test_mxfp4_roundtrip_of_representable_values():
    """Encoder (workloads) and decoder (oracle) are separate code: values on the e2m1 grid
    times a power of two, with a block maximum of 6 or 4 (which fixes the shared exponent),
    must survive encode -> decode exactly."""
    rng = np.random.default_rng(11)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    x = grid[rng.integers(0, 8, size=(50, 4, 32))] * rng.choice([-1.0, 1.0], size=(50, 4, 32))
    x[:, :, 0] = rng.choice([6.0, -6.0, 4.0, -4.0], size=(50, 4))
    t = rng.integers(-20, 20, size=(50, 4, 1)).astype(np.float64)
    x = (x * np.exp2(t)).reshape(50, 128).astype(np.float32)
    packed, sf = wl.encode_mxfp4(x)
    back = oracle.decode_mxfp4(packed, sf)
    assert np.array_equal(back, x.astype(np.float64))


def test_e4m3_integer_codes():
    g = golden("e5_e4m3_integers.json")
    codes = wl.encode_e4m3(np.array(g["values"], dtype=np.float32))
    assert list(codes) == g["codes"]
    assert list(oracle.decode_e4m3(np.array(g["codes"], dtype=np.uint8))) == g["values"]
    assert 128 * 16 * 3 * 32 == g["worst_case_score"] and g["worst_case_score"] < 2 ** 24


# ----------------------------------------------------------------------------- worked examples

def test_e1_scores_and_selection():
    g = golden("e1_scoring_ties_causal.json")
    p = e1_problem()
    assert list(oracle.row_scores(p, 0)) == g["scores"]
    for c in g["cases"]:
        pp = e1_problem(ke=c["ke"], topk=c["k"])
        got = oracle.topk(pp)[0]
        n = min(c["k"], c["ke"])
        assert sorted(got[:n]) == sorted(x for x in c["selected"] if x >= 0)
        assert list(got[n:]) == [x for x in c["selected"] if x < 0]


def test_e1_embedded_in_32_heads():
    """Zero-weight, zero-query extra heads leave every score unchanged."""
    g = golden("e1_scoring_ties_causal.json")
    p = e1_problem(heads=32)
    assert list(oracle.row_scores(p, 0)) == g["scores"]


def test_e2_key_scale():
    g = golden("e2_key_scale.json")
    p = e1_problem(k_scale=g["kscale"])
    assert list(oracle.row_scores(p, 0)) == g["scores"]
    for c in g["cases"]:
        got = oracle.topk(e1_problem(ke=c["ke"], k_scale=g["kscale"], topk=c["k"]))[0]
        assert sorted(got) == sorted(c["selected"])


def test_e3_signed_zero_ties():
    g = golden("e3_signed_zero_ties.json")
    x = np.array([float(v) for v in g["x"]], dtype=np.float32)
    assert np.signbit(x[1]) and not np.signbit(x[3])
    for c in g["cases"]:
        got = oracle.select_topk(x, c["k"])
        n = min(c["k"], len(x))
        assert sorted(got[:n]) == sorted(v for v in c["selected"] if v >= 0)
        assert list(got[n:]) == [v for v in c["selected"] if v < 0]


def test_e6_page_transform():
    g = golden("e6_page_transform.json")
    got = oracle.page_transform(np.array(g["pos"]), np.array(g["page_row"]))
    assert list(got) == g["slot"]


# ----------------------------------------------------------------------------- brute force

def _torch_e4m3(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _brute_scores(qv, wv, kv, kscale):
    """Pure-Python loops: qv [H][128], wv [H], kv [n][128] (python floats)."""
    out = []
    for s in range(len(kv)):
        tot = 0.0
        for h in range(len(qv)):
            d = 0.0
            for j in range(128):
                d += qv[h][j] * kv[s][j]
            tot += wv[h] * (d if d > 0 else 0.0)
        out.append(tot * (1.0 if kscale is None else kscale[s]))
    return np.array(out, dtype=np.float64).astype(np.float32)


def _brute_select(x, k):
    """Top-k by definition: i beats j iff x_i > x_j or (x_i == x_j and i < j)."""
    n = len(x)
    rank = [sum(1 for j in range(n) if x[j] > x[i] or (x[j] == x[i] and j < i)) for i in range(n)]
    sel = sorted(i for i in range(n) if rank[i] < k)
    return sel + [-1] * (k - len(sel))


def _bf16_vals(bits):
    return torch.from_numpy(np.asarray(bits).view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_bruteforce_e4m3_contiguous(seed):
    rng = np.random.default_rng(100 + seed)
    rows, H, n = 3, 4, 24
    q = wl.encode_e4m3(rng.standard_normal((rows, H, 128)).astype(np.float32))
    k = wl.encode_e4m3(rng.standard_normal((n, 128)).astype(np.float32))
    sc = rng.uniform(0.5, 2.0, size=n).astype(np.float32)
    w = wl.encode_bf16(rng.uniform(0, 0.25, size=(rows, H)))
    ks = np.array([0, 3, 5], dtype=np.int32)
    ke = np.array([24, 17, 6], dtype=np.int32)
    p = wl.Problem("bf", wl.FMT_E4M3, rows, H, q, None, k, None, sc, w, ks, ke, 7, n)
    qd, kd, wd = _torch_e4m3(q), _torch_e4m3(k), _bf16_vals(w)
    for r in range(rows):
        s0, s1 = int(ks[r]), int(ke[r])
        ref = _brute_scores(qd[r].tolist(), wd[r].tolist(), kd[s0:s1].tolist(), sc[s0:s1].tolist())
        got = oracle.row_scores(p, r)
        np.testing.assert_array_max_ulp(got, ref, maxulp=1)
        assert sorted(oracle.select_topk(got, 7)) == sorted(_brute_select(got.tolist(), 7))


def _brute_mxfp4(packed, sf):
    vals = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = []
    for row_b, row_s in zip(packed.reshape(-1, 64), sf.reshape(-1, 4)):
        v = []
        for i, b in enumerate(row_b):
            for nib in (int(b) & 0xF, int(b) >> 4):
                mag = vals[nib & 7]
                v.append(-mag if nib & 8 else mag)
        v = [x * math.ldexp(1.0, int(row_s[j // 32]) - 127) for j, x in enumerate(v)]
        out.append(v)
    return out


def test_bruteforce_mxfp4():
    rng = np.random.default_rng(7)
    rows, H, n = 2, 3, 20
    q, q_sf = wl.encode_mxfp4(rng.standard_normal((rows, H, 128)).astype(np.float32) * 3)
    k, k_sf = wl.encode_mxfp4(rng.standard_normal((n, 128)).astype(np.float32))
    w = wl.encode_bf16(rng.uniform(0, 0.1, size=(rows, H)))
    ks = np.array([0, 2], dtype=np.int32)
    ke = np.array([20, 11], dtype=np.int32)
    p = wl.Problem("bf4", wl.FMT_MXFP4, rows, H, q, q_sf, k, k_sf, None, w, ks, ke, 5, n)
    kd = _brute_mxfp4(k, k_sf)
    wd = _bf16_vals(w)
    for r in range(rows):
        qd = _brute_mxfp4(q[r], q_sf[r])
        ref = _brute_scores(qd, wd[r].tolist(), kd[int(ks[r]):int(ke[r])], None)
        got = oracle.row_scores(p, r)
        np.testing.assert_array_max_ulp(got, ref, maxulp=1)


def test_bruteforce_paged():
    """Paged keys: brute force walks the page table by hand."""
    rng = np.random.default_rng(9)
    H, num_pages = 2, 5
    k = wl.encode_e4m3(rng.standard_normal((num_pages, 64, 128)).astype(np.float32))
    sc = rng.uniform(0.5, 2, size=num_pages * 64).astype(np.float32)
    q = wl.encode_e4m3(rng.standard_normal((3, H, 128)).astype(np.float32))
    w = wl.encode_bf16(rng.uniform(0, 0.2, size=(3, H)))
    pt = np.array([[3, 0, -1], [4, 1, 2]], dtype=np.int32)
    row_req = np.array([0, 1, 1], dtype=np.int32)
    ks = np.array([0, 0, 60], dtype=np.int32)
    ke = np.array([100, 170, 140], dtype=np.int32)
    p = wl.Problem("bfp", wl.FMT_E4M3, 3, H, q, None, k, None, sc, w, ks, ke, 4, num_pages * 64,
                   page_table=pt, row_req=row_req)
    kflat = _torch_e4m3(k).reshape(-1, 128)
    qd, wd = _torch_e4m3(q), _bf16_vals(w)
    for r in range(3):
        slots = []
        for s in range(int(ks[r]), int(ke[r])):
            page, off = divmod(s, 64)
            slots.append(int(pt[row_req[r], page]) * 64 + off)
        ref = _brute_scores(qd[r].tolist(), wd[r].tolist(), kflat[slots].tolist(), sc[slots].tolist())
        np.testing.assert_array_max_ulp(oracle.row_scores(p, r), ref, maxulp=1)


@pytest.mark.parametrize("seed", range(6))
def test_selection_matches_definition_with_dense_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 40))
    x = rng.choice(np.array([0.0, -0.0, 0.5, 1.0, -1.0, 0.25], dtype=np.float32), size=n)
    for k in (1, 3, n, n + 2):
        assert sorted(oracle.select_topk(x, k)) == sorted(_brute_select(x.tolist(), k))


# ----------------------------------------------------------------------------- closed forms

def test_single_head_unit_weight_is_a_dot_product():
    rng = np.random.default_rng(5)
    n = 300
    q = wl.encode_e4m3(np.abs(rng.standard_normal((1, 1, 128))).astype(np.float32))
    k = wl.encode_e4m3(np.abs(rng.standard_normal((n, 128))).astype(np.float32))
    w = wl.encode_bf16(np.ones((1, 1)))
    p = wl.Problem("h1", wl.FMT_E4M3, 1, 1, q, None, k, None, None, w,
                   np.array([0], np.int32), np.array([n], np.int32), 10, n)
    ref = (torch.from_numpy(_torch_e4m3(k)) @ torch.from_numpy(_torch_e4m3(q)[0, 0])).numpy()
    assert np.array_equal(oracle.row_scores(p, 0), ref.astype(np.float32))


def test_power_of_two_key_scale_is_exact():
    p = wl.prefill(rows=4, num_keys=512, heads=64, seed=21)
    s1 = oracle.row_scores(p, 2)
    p.k_scale = p.k_scale * np.float32(4.0)
    assert np.array_equal(oracle.row_scores(p, 2), s1 * np.float32(4.0))


# ----------------------------------------------------------------------------- invariants

@pytest.mark.parametrize("fam,kw", [
    ("tiny", dict(rows=8, num_keys=640, topk=100)),
    ("prefill", dict(rows=6, num_keys=1200, topk=128)),
    ("long", dict(rows=5, num_keys=3000, topk=64, band_keys=200)),
    ("decode", dict(num_req=2, q_len=3, ctx_lo=100, ctx_hi=900, topk=64)),
])
def test_invariants_on_families(fam, kw):
    p = wl.make(fam, **kw)
    sel = oracle.topk(p)
    for r in range(p.rows):
        check_topk_invariants(oracle.row_scores(p, r), sel[r], p.topk)


def test_invariants_on_selection_family():
    sp = wl.select_only(rows=3, ld=8192, min_len=100, topk=300, runs=8)
    sel = oracle.select_rows(sp.x, sp.length, sp.topk)
    for r in range(sp.rows):
        x = sp.x[r, :sp.length[r]]
        check_topk_invariants(x, sel[r], sp.topk)
        assert oracle.selected_value_recall(x, sel[r], sp.topk) == 1.0


def test_short_row_returns_everything():
    p = e1_problem(ke=3, topk=8)
    got = oracle.topk(p)[0]
    assert sorted(got[:3]) == [0, 1, 2] and list(got[3:]) == [-1] * 5


def test_empty_row():
    p = e1_problem(ke=0, topk=4)
    assert list(oracle.topk(p)[0]) == [-1] * 4


# ----------------------------------------------------------------------------- planted mistakes

def _pins_pass(score_fn, select_fn):
    """The hand-worked pins E1/E2/E3 evaluated against a (possibly mutated) oracle."""
    g1, g2, g3 = golden("e1_scoring_ties_causal.json"), golden("e2_key_scale.json"), golden("e3_signed_zero_ties.json")
    if list(score_fn(e1_problem(), 0)) != g1["scores"]:
        return False
    if list(score_fn(e1_problem(k_scale=g2["kscale"]), 0)) != g2["scores"]:
        return False
    x = np.array([float(v) for v in g3["x"]], dtype=np.float32)
    for c in g3["cases"]:
        if sorted(select_fn(x, c["k"])) != sorted(c["selected"]):
            return False
    for c in g1["cases"]:
        pp = e1_problem(ke=c["ke"], topk=c["k"])
        if sorted(select_fn(score_fn(pp, 0), c["k"])) != sorted(c["selected"]):
            return False
    return True


def test_pins_catch_planted_mistakes():
    assert _pins_pass(oracle.row_scores, oracle.select_topk)

    def no_relu(p, r):
        qd = oracle.dequant_q(p, [r])[0]
        kv = oracle.dequant_keys(p, oracle.physical_keys(p, r))
        return (oracle.decode_bf16(p.w[r]) @ (qd @ kv.T)).astype(np.float32)

    def weights_swapped(p, r):
        qd = oracle.dequant_q(p, [r])[0]
        kv = oracle.dequant_keys(p, oracle.physical_keys(p, r))
        return (oracle.decode_bf16(p.w[r])[::-1] @ np.maximum(qd @ kv.T, 0)).astype(np.float32)

    def relu_after_sum(p, r):
        qd = oracle.dequant_q(p, [r])[0]
        kv = oracle.dequant_keys(p, oracle.physical_keys(p, r))
        return np.maximum(oracle.decode_bf16(p.w[r]) @ (qd @ kv.T), 0).astype(np.float32)

    def scale_ignored(p, r):
        q = dataclass_replace(p, k_scale=None)
        return oracle.row_scores(q, r)

    def off_by_one_range(p, r):
        q = dataclass_replace(p, ke=p.ke + 0, ks=p.ks + 1)
        return np.concatenate([[np.float32(0)], oracle.row_scores(q, r)]).astype(np.float32)

    def unstable_sort(x, k):
        # ties broken by the higher index instead of the lower one
        order = sorted(range(len(x)), key=lambda i: (-float(x[i]), -i))
        out = np.full(k, -1, dtype=np.int32)
        out[:min(k, len(x))] = order[:min(k, len(x))]
        return out

    def signed_zero_bits(x, k):
        u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
        okey = np.where(u >> 31, 0xFFFFFFFF - u, u | 0x80000000)  # no -0 canonicalisation
        order = sorted(range(len(x)), key=lambda i: (-okey[i], i))
        out = np.full(k, -1, dtype=np.int32)
        out[:min(k, len(x))] = order[:min(k, len(x))]
        return out

    for bad in (no_relu, weights_swapped, relu_after_sum, scale_ignored, off_by_one_range):
        assert not _pins_pass(bad, oracle.select_topk), bad.__name__
    for bad in (unstable_sort, signed_zero_bits):
        assert not _pins_pass(oracle.row_scores, bad), bad.__name__


def dataclass_replace(p, **kw):
    import dataclasses
    return dataclasses.replace(p, **kw)


# ---------------------------------------------------------------- sparse attention oracle
# Pins of oracle.sparse_attention by closed forms: a single key gives its value vector,
# equal scores give the plain mean (numpy.mean, with repeated slots counted twice), a
# hand-worked two-key case with weights 1/4 and 3/4, slot padding and out-of-range slots
# take no part, a very large softmax scale gives the arg-max key's value, and grouped
# query heads read their own KV head.

def _attn_inputs(rows=2, hq=4, hkv=2, num_slots=10, seed=0):
    rng = np.random.default_rng(seed)
    q = wl.encode_bf16(rng.standard_normal((rows, hq, 128)))
    k = wl.encode_e4m3(rng.standard_normal((num_slots, hkv, 128)))
    v = wl.encode_e4m3(rng.standard_normal((num_slots, hkv, 128)))
    return q, k, v


def test_attn_single_key_is_its_value():
    q, k, v = _attn_inputs()
    slots = np.array([[3, -1, -1], [-1, 7, -1]], dtype=np.int32)
    out = oracle.sparse_attention(q, k, v, slots, 0.3, 2.0)
    vd = oracle.decode_e4m3(v)
    for h in range(4):
        assert np.array_equal(out[0, h], 2.0 * vd[3, h // 2])
        assert np.array_equal(out[1, h], 2.0 * vd[7, h // 2])


def test_attn_equal_scores_is_the_mean_with_repeats():
    _, k, v = _attn_inputs(rows=1)
    q = np.zeros((1, 4, 128), dtype=np.uint16)                 # every score 0
    slots = np.array([[2, 5, 5, 9, -1, 11, 0]], dtype=np.int32)  # 11 is out of range
    out = oracle.sparse_attention(q, k, v, slots, 1.0, 1.0)
    vd = oracle.decode_e4m3(v)
    for h in range(4):
        ref = np.mean(vd[[2, 5, 5, 9, 0], h // 2, :], axis=0)
        assert np.allclose(out[0, h], ref, rtol=0, atol=1e-12)


def test_attn_two_keys_hand_worked():
    """q = e0, k0 = 0, k1 = e0, softmax scale ln 3: scores 0 and ln 3, weights 1/4 and 3/4;
    v0 = 1, v1 = 2 at d = 0 gives 1.75, and v0 = -4, v1 = 4 at d = 5 gives 2."""
    q = np.zeros((1, 1, 128)); q[0, 0, 0] = 1.0
    k = np.zeros((2, 1, 128)); k[1, 0, 0] = 1.0
    v = np.zeros((2, 1, 128)); v[0, 0, 0], v[1, 0, 0] = 1.0, 2.0; v[0, 0, 5], v[1, 0, 5] = -4.0, 4.0
    out = oracle.sparse_attention(wl.encode_bf16(q), wl.encode_e4m3(k), wl.encode_e4m3(v),
                                  np.array([[0, 1]], dtype=np.int32), math.log(3.0), 1.0)
    assert abs(out[0, 0, 0] - 1.75) < 1e-12
    assert abs(out[0, 0, 5] - 2.0) < 1e-12
    assert np.all(out[0, 0, [1, 2, 3, 4, 6]] == 0.0)


def test_attn_padding_and_argmax_limit():
    q, k, v = _attn_inputs(rows=2, seed=3)
    slots = np.array([[-1, -1, 40, -7], [1, 4, 6, 8]], dtype=np.int32)
    out = oracle.sparse_attention(q, k, v, slots, 1e4, 1.0)
    assert np.all(out[0] == 0.0)                                  # nothing valid: zeros
    qd, kd, vd = oracle.decode_bf16(q), oracle.decode_e4m3(k), oracle.decode_e4m3(v)
    for h in range(4):
        g = h // 2
        dots = kd[[1, 4, 6, 8], g, :] @ qd[1, h, :]
        top = [1, 4, 6, 8][int(np.argmax(dots))]
        if np.sort(dots)[-1] - np.sort(dots)[-2] > 1e-2:           # a clear winner
            assert np.allclose(out[1, h], vd[top, g], rtol=0, atol=1e-9)


def test_attn_grouped_heads_read_their_kv_head():
    _, k, v = _attn_inputs(rows=1, hq=6, hkv=3, seed=5)
    q = np.zeros((1, 6, 128), dtype=np.uint16)
    slots = np.array([[4]], dtype=np.int32)
    out = oracle.sparse_attention(q, k, v, slots, 1.0, 1.0)
    vd = oracle.decode_e4m3(v)
    for h in range(6):
        assert np.array_equal(out[0, h], vd[4, h // 2])
        assert not np.array_equal(out[0, h], vd[4, (h // 2 + 1) % 3])


# ------------------------------------------------ selected-value recall and row offsets

def _recall_cases():
    from fractions import Fraction
    g = golden("e7_selected_value_recall.json")
    for row in g["rows"]:
        x = np.array(row["x"], dtype=np.float32)
        for c in row["cases"]:
            yield x, np.array(c["idx"], dtype=np.int32), c["k"], float(Fraction(c["recall"]))


def _recall_pins_pass(fn):
    return all(math.isclose(fn(x, idx, k), want, abs_tol=1e-12) for x, idx, k, want in _recall_cases())


def test_selected_value_recall_hand_worked():
    """E7: recall values worked by hand, including a tie-broken index set with recall 1
    and a repeated value counted with its multiplicity."""
    for x, idx, k, want in _recall_cases():
        assert math.isclose(oracle.selected_value_recall(x, idx, k), want, abs_tol=1e-12), (x, idx, k)


def test_recall_pins_catch_planted_mistakes():
    assert _recall_pins_pass(oracle.selected_value_recall)

    def always_one(x, idx, k):
        return 1.0

    def index_sets(x, idx, k):
        # compares index sets with the tie-broken top-k instead of value multisets
        n = min(k, len(x))
        ref = set(oracle.select_topk(x, k)[:n].tolist())
        return len(ref & set(int(i) for i in idx if i >= 0)) / n if n else 1.0

    def value_sets(x, idx, k):
        # distinct values instead of multisets
        n = min(k, len(x))
        best = set(np.sort(x.astype(np.float64))[::-1][:n].tolist())
        got = set(x[idx[idx >= 0]].astype(np.float64).tolist())
        return len(best & got) / len(best) if n else 1.0

    def over_k(x, idx, k):
        # divides by k even when the row is shorter than k
        r = oracle.selected_value_recall(x, idx, k)
        return r * min(k, len(x)) / k

    for bad in (always_one, index_sets, value_sets, over_k):
        assert not _recall_pins_pass(bad), bad.__name__


def _select_by_rank(v, k):
    """Definition by counting: element j is kept iff fewer than k elements precede it in
    the order (value descending, -0 == +0, lower index first)."""
    v = [float(a) for a in v]
    keep = []
    for j in range(len(v)):
        rank = sum(1 for i in range(len(v)) if v[i] > v[j] or (v[i] == v[j] and i < j))
        if rank < k:
            keep.append(j)
    return sorted(keep)


@pytest.mark.parametrize("seed", range(4))
def test_select_rows_row_start_brute_force(seed):
    """select_rows with per-row offsets against selection by rank counting on the slice
    x[r, row_start[r] : row_start[r] + length[r]], indices relative to the offset."""
    rng = np.random.default_rng(100 + seed)
    rows, ld, k = 6, 90, 11
    x = rng.integers(-6, 7, size=(rows, ld)).astype(np.float32) * np.float32(0.25)  # dense ties
    x[rng.random((rows, ld)) < 0.1] = np.float32(-0.0)
    rs = rng.integers(0, ld, size=rows).astype(np.int32)
    length = np.array([rng.integers(0, ld - s + 1) for s in rs], dtype=np.int32)
    length[0] = 0                                                    # empty row
    length[1] = min(5, ld - rs[1])                                   # shorter than k
    got = oracle.select_rows(x, length, k, row_start=rs)
    for r in range(rows):
        v = x[r, rs[r]:rs[r] + length[r]]
        want = _select_by_rank(v, k)
        n = min(k, len(v))
        assert sorted(got[r, :n].tolist()) == want, r
        assert np.all(got[r, n:] == -1)
    # the offsets matter: the same call without them differs on this input
    assert not np.array_equal(oracle.select_rows(x, length, k), got)
