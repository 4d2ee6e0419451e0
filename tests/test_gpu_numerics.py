"""Numerics of the scoring core, on the GPU.

Keys built to point against the common direction of a row's query heads have every head
dot < 0, so their exact score is 0 (oracle).  Checked on such keys, mixed with ordinary
ones:
* every stored score is >= +0 (no negative values, no -0.0);
* e4m3 (direct form, ReLU per head): the planted keys score exactly 0;
* MXFP4 (split form, (sum_h w_h |x_h| + u . k) / 2 with u on the matrix cores): the planted
  keys score a small value near 0;
* at the workloads' magnitudes every score is within |d| <= 1e-4 + 1e-5 |oracle|;
* at large legal e4m3 magnitudes (values near +-448, w up to 1, key scale 2) the error is
  bounded relative to the magnitude B = kscale * sum_h w_h sum_d |q_hd k_d| (the fp8
  MFMA's dropped low-order products scale with it);
* selection over the GPU's own scores is bit-exact (oracle select == idx_select ==
  idx_fused_topk), with rows whose top-k reaches into the zero scores.
And through idx_score, the fp8 MFMA's rounding of one head dot: a 1.0 product beside
products 2^18 times smaller loses at most the small products of its group of 8.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_attention_indexer_score_amd as sai
from helpers import negative_dot_problem, check_topk_invariants

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 1e-5
# |gpu - oracle| <= BETA * B at any magnitude (B as above); the measured ratio is printed
BETA = 2.0 ** -14


def magnitude(p, r, kd):
    """B(r, s) = kscale[s] * sum_h w[r, h] * sum_d |q[r, h, d] k[s, d]| (float64, oracle decode)."""
    V = int(p.ke[r] - p.ks[r])
    qd = np.abs(oracle.dequant_q(p, [r])[0])
    w = oracle.decode_bf16(p.w[r])
    kabs = np.abs(kd[int(p.ks[r]):int(p.ke[r])])     # already times the key scale (> 0)
    return w @ (qd @ kabs.T)


def run_case(p, neg, k, bound):
    """bound: "tolerance" (|d| <= 1e-4 + 1e-5 |oracle|) or "magnitude" (|d| <= BETA * B)."""
    dp = sai.DeviceProblem.from_host(p)
    V = (p.ke - p.ks).astype(np.int32)
    sc = sai.idx_score(dp, ld=int(V.max())).cpu().numpy()
    kd = oracle.all_keys(p)
    worst_lim, worst_b = 0.0, 0.0
    zero_exact = zero_total = 0
    for r in range(p.rows):
        got = sc[r, :V[r]]
        assert not np.any(np.signbit(got)), f"row {r}: negative or -0.0 score stored"
        ref = oracle.row_scores(p, r, kd_all=kd).astype(np.float64)
        err = np.abs(got.astype(np.float64) - ref)
        lim = ATOL + RTOL * np.abs(ref)
        B = magnitude(p, r, kd)
        worst_lim = max(worst_lim, float((err / lim).max()))
        worst_b = max(worst_b, float((err / np.maximum(B, 1e-300)).max()))
        planted = neg[int(p.ks[r]):int(p.ke[r])]
        assert np.all(ref[planted] == 0.0)
        zero_exact += int(np.sum(got[planted] == 0.0))
        zero_total += int(planted.sum())
    print(f"[numerics] {p.fmt} H={p.heads}: max err/limit {worst_lim:.3g}, max err/B {worst_b:.3g} "
          f"(2^{np.log2(max(worst_b, 1e-300)):.1f}), keys with exact score 0 stored as exactly 0: "
          f"{zero_exact}/{zero_total}", flush=True)
    if p.fmt == "e4m3":
        assert zero_exact == zero_total, "direct form: every key with all head dots < 0 must score exactly 0"
    if bound == "tolerance":
        assert worst_lim <= 1.0
    assert worst_b <= BETA
    # selection over the GPU's own scores: bit-exact among the three routes
    ref_sel = oracle.select_rows(sc, V, k)
    sel = sai.idx_select(torch.from_numpy(sc).cuda(), torch.from_numpy(V).cuda(), k).cpu().numpy()
    fused = sai.idx_fused_topk(dp, k).cpu().numpy()
    for name, got in (("idx_select", sel), ("idx_fused_topk", fused)):
        assert np.array_equal(np.sort(got, axis=1), np.sort(ref_sel, axis=1)), name
    reach = 0
    for r in range(p.rows):
        check_topk_invariants(sc[r, :V[r]], fused[r], k)
        reach += int(np.any(sc[r, fused[r][fused[r] >= 0]] == 0.0))
    print(f"[numerics] rows whose top-{k} includes zero scores: {reach}/{p.rows}", flush=True)
    return worst_lim, worst_b


def test_zero_score_keys_e4m3():
    """e4m3, 64 heads, N(0,1)-scale values, w ~ U(0, 1/64), key scale U[0.5, 2]; the heads
    share a direction, so the dots are ~10x those of independent heads and the fp8 MFMA's
    dropped products grow with them: bounded relative to B.  k = 2048 reaches past the
    ~40 % positive scores into the zeros."""
    p, neg = negative_dot_problem(rows=24, num_keys=3000, heads=64, sigma=1.0, w_hi=1 / 64, seed=1, topk=2048)
    run_case(p, neg, 2048, "magnitude")


def test_zero_score_keys_mxfp4():
    """MXFP4, 32 heads, w ~ U(0, 1/32) (four rows per wave): the split form's cancellation
    stays inside the absolute tolerance at these magnitudes."""
    p, neg = negative_dot_problem(fmt="mxfp4", rows=40, num_keys=5000, heads=32, sigma=1.0, w_hi=1 / 32,
                                  kscale=None, seed=2, topk=2048)
    run_case(p, neg, 2048, "tolerance")


def test_zero_score_keys_e4m3_large_magnitudes():
    """e4m3 values near +-448 (sigma 150, saturating), w ~ U(0, 1), key scale 2."""
    p, neg = negative_dot_problem(rows=24, num_keys=3000, heads=64, sigma=150.0, w_hi=1.0, kscale=(2.0, 2.0),
                                  seed=3, topk=1024)
    run_case(p, neg, 1024, "magnitude")


def test_fp8_mfma_rounding_of_one_head_dot():
    """One row, head 0 only (w = 1 there, 0 elsewhere): q_0 = k = (1, s, s, ..., s) with
    s = 2^-9, the smallest e4m3 subnormal, so the exact dot is 1 + 127 s^2.  The score is
    the MFMA's head dot itself.  The fp8 MFMA sums each group of 8 products at the scale of
    its largest one, so the group holding the 1.0 product may lose its 7 small products,
    and nothing else is lost: 1 + 120 s^2 <= score <= 1 + 127 s^2."""
    from helpers import e4m3_problem
    s2 = 2.0 ** -18
    q = np.zeros((1, 32, 128), dtype=np.float32)
    q[0, 0, :] = 2.0 ** -9
    q[0, 0, 0] = 1.0
    w = np.zeros((1, 32), dtype=np.float32)
    w[0, 0] = 1.0
    key = np.full((1, 128), 2.0 ** -9, dtype=np.float32)
    key[0, 0] = 1.0
    p = e4m3_problem(q, w, key, [0], [1], topk=1, heads=32)
    got = float(sai.idx_score(sai.DeviceProblem.from_host(p), ld=1).cpu().numpy()[0, 0])
    exact = 1.0 + 127 * s2
    assert float(oracle.row_scores(p, 0)[0]) == np.float32(exact)
    print(f"[numerics] fp8 MFMA head dot: exact 1 + 127 s^2, GPU 1 + {(got - 1.0) / s2:.1f} s^2", flush=True)
    assert 1.0 + 120 * s2 <= got <= exact
