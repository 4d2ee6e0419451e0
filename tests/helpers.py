"""Small-problem builders shared by the CPU and GPU tests (input construction only)."""
import json
import os

import numpy as np

from sparse_attention_indexer_score_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pad_dim(vecs, d=wl.HEAD_DIM):
    a = np.zeros((len(vecs), d), dtype=np.float32)
    for i, v in enumerate(vecs):
        a[i, :len(v)] = v
    return a


def e4m3_problem(q, w, keys, ks, ke, k_scale=None, topk=8, heads=None):
    """q: float [rows, H, d<=128]; w: float [rows, H]; keys: float [n, d]; exact e4m3 values."""
    q = np.asarray(q, dtype=np.float32)
    rows, H = q.shape[0], q.shape[1]
    heads = H if heads is None else heads
    qf = np.zeros((rows, heads, wl.HEAD_DIM), dtype=np.float32)
    qf[:, :H, :q.shape[2]] = q
    wf = np.zeros((rows, heads), dtype=np.float32)
    wf[:, :H] = np.asarray(w, dtype=np.float32)
    kf = pad_dim(np.asarray(keys, dtype=np.float32))
    return wl.Problem(
        "hand", wl.FMT_E4M3, rows, heads, wl.encode_e4m3(qf), None, wl.encode_e4m3(kf), None,
        None if k_scale is None else np.asarray(k_scale, dtype=np.float32),
        wl.encode_bf16(wf), np.asarray(ks, dtype=np.int32), np.asarray(ke, dtype=np.int32),
        topk, kf.shape[0])


def e1_problem(ke=8, k_scale=None, heads=None, topk=8):
    g = golden("e1_scoring_ties_causal.json")
    return e4m3_problem([g["q"]], [g["w"]], g["keys"], [0], [ke], k_scale=k_scale, topk=topk,
                        heads=heads)


def check_topk_invariants(x, sel, k):
    """x: fp32 scores of one row (index = relative key); sel: returned indices (-1 padded).

    Checks: |selected| = min(k, n); indices distinct and in [0, n); every unselected
    score <= the minimum selected score; ties at that minimum go to lower indices.
    """
    x = np.asarray(x, dtype=np.float32)
    n = x.shape[0]
    m = min(k, n)
    sel = np.asarray(sel)
    assert sel.shape[0] == k
    assert np.all(sel[m:] == -1), "padding must be -1"
    s = sel[:m]
    assert np.all((s >= 0) & (s < n)), "index out of range"
    assert len(np.unique(s)) == m, "duplicate index"
    if m == 0 or m == n:
        return
    mask = np.zeros(n, dtype=bool)
    mask[s] = True
    vmin = x[s].min()
    rest = x[~mask]
    assert np.all(rest <= vmin), "an unselected score exceeds the minimum selected score"
    tie_sel = np.nonzero(mask & (x == vmin))[0]
    tie_rest = np.nonzero(~mask & (x == vmin))[0]
    if len(tie_rest):
        assert tie_sel.max() < tie_rest.min(), "ties must go to the lower key index"
