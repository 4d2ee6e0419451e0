"""The entry points under HIP graph capture, on the GPU.

A call is captured into a graph (torch.cuda.CUDAGraph on a side stream) and replayed several
times; between replays the program does eager work of its own (the output cleared, other
launches) and synchronises.  Every replay must give exactly the eager result's index sets
(row by row; the order inside a row is unspecified): the library records kernel launches
only (no memset or copy nodes; every workspace word a call reads is written by that call
first), so a replay starts from the same state as a fresh call.
"""
import numpy as np
import pytest
import torch

import sparse_attention_indexer_score_amd as sai
from sparse_attention_indexer_score_amd import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 4

FAMILIES = {
    "long_mxfp4_32h": lambda: wl.long_context(rows=48, num_keys=40000, band_keys=3000, topk=512, seed=101),
    "prefill_e4m3_64h": lambda: wl.prefill(rows=40, num_keys=20000, topk=1024, seed=102),
    "decode_paged": lambda: wl.decode(num_req=12, ctx_lo=4000, ctx_hi=60000, topk=2048, seed=103),
    # enough work items that the paged filter's persistent workgroups take most by ticket
    "decode_paged_tickets": lambda: wl.decode(num_req=40, ctx_lo=8192, ctx_hi=262144, topk=2048, seed=105),
}


def capture(fn):
    """Warm up fn on a side stream, then capture one call of it."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    return g


def rows_sorted(x):
    """Each row's index set in ascending order (the order within a row is unspecified: the
    select emits through atomics)."""
    return torch.sort(x, dim=1).values


def replay_and_check(g, out, ref, noise, what):
    want = rows_sorted(ref)
    for i in range(REPLAYS):
        out.fill_(-7)                    # eager work between replays
        noise()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rows_sorted(out), want), f"{what}: replay {i} differs from the eager result"


@pytest.mark.parametrize("family", sorted(FAMILIES))
def test_fused_topk_graph_replays(family):
    p = FAMILIES[family]()
    dp = sai.DeviceProblem.from_host(p)
    runner = sai.FusedRunner(dp, p.topk)
    ref = runner()[0].clone()
    torch.cuda.synchronize()
    other = torch.randn(1 << 20, device="cuda")
    g = capture(lambda: runner())
    replay_and_check(g, runner.out, ref, lambda: other.mul_(1.0001), f"{family} fused")
    print(f"[graph] {family}: {REPLAYS} replays of idx_fused_topk equal the eager call", flush=True)


@pytest.mark.parametrize("family", ["decode_paged", "long_mxfp4_32h"])
def test_fused_topk_noalloc_graph_replays(family):
    """The allocation-free entry point, for callers that capture: eager call first (it
    resolves the device's scratch address), then capture and replays."""
    p = FAMILIES[family]()
    dp = sai.DeviceProblem.from_host(p)
    out = torch.empty((p.rows, p.topk), dtype=torch.int32, device="cuda")
    ref = sai.FusedRunner(dp, p.topk)()[0].clone()
    sai.idx_fused_topk_noalloc(dp, p.topk, out=out)
    torch.cuda.synchronize()
    assert torch.equal(rows_sorted(out), rows_sorted(ref))
    g = capture(lambda: sai.idx_fused_topk_noalloc(dp, p.topk, out=out))
    replay_and_check(g, out, ref, lambda: sai.FusedRunner(dp, p.topk)(), f"{family} noalloc")


@pytest.mark.parametrize("split", [0, 4])
def test_score_and_select_graph_replays(split):
    """idx_score then idx_select (the dense route) captured together; the row-split select
    keeps per-row counters in its workspace that each call leaves at zero for the next, so
    every replay must find them so."""
    p = wl.long_context(rows=16, num_keys=200000, band_keys=3000, topk=2048, seed=104)
    dp = sai.DeviceProblem.from_host(p)
    V = torch.from_numpy((p.ke - p.ks).astype(np.int32)).cuda()
    sr = sai.ScoreRunner(dp, ld=int(V.max()))
    sel = sai.SelectRunner(sr.out, V, p.topk, split=split)

    def dense():
        sr()
        return sel()

    ref = dense().clone()
    torch.cuda.synchronize()
    g = capture(dense)
    replay_and_check(g, sel.out, ref, lambda: sr.out.fill_(0.0), f"dense route split={split}")
