"""The fused step (hs_decode_step / hs_select_decode) when its launch is not
resident all at once, and when one of its waits cannot end.

The single launch is a persistent grid sized to what the GPU holds; a unit's
attention tasks wait for its scoring tasks, which run on other workgroups.
Every wait is bounded by wall-clock time, and an expired wait is reported in
the workspace's status word ("SGLang hierarchical sparse attention" section
2.2: the decode phase, selection then attention, that the step runs). The
second test forces an expiry from the host: one unit's scoring counter in the
workspace starts far below zero, so its attention tasks give up after the
bound while every kernel exits normally. The third runs several full-GPU
calls at the same time: each must either equal the separate calls or report
the expired wait, never return wrong results silently.
"""
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
from gpu_helpers import Problem, log
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

# 32 units x (8 scoring + 8 attention tasks) = 512 tasks: one launch fills the
# GPU (two workgroups per compute unit), so overlapping launches cannot all
# be resident
W = CONFIGS[3].scaled(T=65536, needles=4)
_P = {}


def problem():
    if "p" not in _P:
        log("setting up %s T=%d" % (W.name, W.T))
        _P["p"] = Problem.make(W)
    return _P["p"]


def reference(P, q, summ):
    ids, cnt = P.select(q, summ)
    out = P.decode(q, ids, cnt)
    torch.cuda.synchronize()
    return ids, cnt, out


def test_step_control_words_after_calls():
    """A correct call leaves the status word at zero, and repeated calls on
    one workspace give the separate calls' results."""
    P = problem()
    q = P.q()
    summ = P.summaries()
    ids_r, cnt_r, out_r = reference(P, q, summ)
    ws = None
    for call in range(3):
        ids, cnt, out, ws = P.decode_step(q, summ, W.nb - 1, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(ids, ids_r) and torch.equal(cnt, cnt_r), call
        assert torch.equal(out, out_r), call
        assert hs.hs_step_status(ws) == 0, call
        ctrl = ws[:hs.STEP_SELECT_BYTE].view(torch.int32)
        assert int(ctrl.abs().sum()) == 0, (call, ctrl.nonzero().reshape(-1).tolist())


def test_expired_wait_sets_status_word():
    """Unit 5's scoring counter starts at -2^30: its attention tasks' waits
    cannot end and expire after the bound; every kernel exits, the status word
    reads HS_STEP_WAIT_EXPIRED, the other units are unaffected, and after a
    zero-fill the same workspace works normally again."""
    P = problem()
    q = P.q()
    summ = P.summaries()
    ids_r, cnt_r, out_r = reference(P, q, summ)
    n = hs.hs_select_decode_workspace_size(P.kvs[0], summ["fine"], W.hq, W.top_k, W.window,
                                           W.max_selected)
    ws = hs.workspace(n, "cuda")
    unit = 5
    at = (hs.STEP_SELECT_BYTE + 256 * unit) // 4
    ws.view(torch.int32)[at] = -(1 << 30)
    torch.cuda.synchronize()
    log("calling hs_decode_step with unit %d's scoring counter at -2^30" % unit)
    ids, cnt, out, _ = P.decode_step(q, summ, W.nb - 1, ws=ws)
    torch.cuda.synchronize()
    assert hs.hs_step_status(ws) == hs.HS_STEP_WAIT_EXPIRED
    b, g = divmod(unit, W.hkv)
    for bb in range(W.batch):
        for gg in range(W.hkv):
            if (bb, gg) == (b, g):
                continue
            c = int(cnt_r[bb, gg])
            assert int(cnt[bb, gg]) == c and torch.equal(ids[bb, gg, :c], ids_r[bb, gg, :c])
            hq = slice(gg * W.G, (gg + 1) * W.G)
            assert torch.equal(out[bb, hq], out_r[bb, hq]), (bb, gg)
    # the bias stays (this call's arrivals were taken off again)
    assert int(ws.view(torch.int32)[at]) == -(1 << 30)
    ws.zero_()
    ids, cnt, out, _ = P.decode_step(q, summ, W.nb - 1, ws=ws)
    torch.cuda.synchronize()
    assert hs.hs_step_status(ws) == 0
    assert torch.equal(ids, ids_r) and torch.equal(cnt, cnt_r) and torch.equal(out, out_r)
    log("expired wait reported; workspace reusable after a zero-fill")


def test_overlapping_full_gpu_calls():
    """Four streams, three hs_decode_step calls each, every call sized to fill
    the GPU and given its own workspace and outputs: the launches overlap and
    are resident only in part. Each call either gives the separate calls'
    results with a zero status word, or reports HS_STEP_WAIT_EXPIRED."""
    P = problem()
    q = P.q()
    summ = P.summaries()
    ids_r, cnt_r, out_r = reference(P, q, summ)
    n = hs.hs_select_decode_workspace_size(P.kvs[0], summ["fine"], W.hq, W.top_k, W.window,
                                           W.max_selected)
    streams = [torch.cuda.Stream() for _ in range(4)]
    runs = []
    for rep in range(3):
        for s in streams:
            ws = hs.workspace(n, "cuda")
            ids = torch.full_like(ids_r, -7)  # entries past a count keep the fill, as in ids_r
            cnt = torch.full_like(cnt_r, -7)
            out = torch.full_like(out_r, float("nan"))
            runs.append((s, ws, ids, cnt, out))
    torch.cuda.synchronize()
    for s, ws, ids, cnt, out in runs:
        with torch.cuda.stream(s):
            hs.hs_decode_step(P.kvs[0], q, summ["fine"], W.top_k, W.window, W.nb - 1, ids, cnt,
                              out, ws, stream=s)
    torch.cuda.synchronize()
    expired = 0
    for i, (s, ws, ids, cnt, out) in enumerate(runs):
        st = hs.hs_step_status(ws, stream=s)
        ok = torch.equal(ids, ids_r) and torch.equal(cnt, cnt_r) and torch.equal(out, out_r)
        assert st in (0, hs.HS_STEP_WAIT_EXPIRED), (i, st)
        assert ok or st == hs.HS_STEP_WAIT_EXPIRED, "call %d: wrong results without a status" % i
        expired += st != 0
    log("%d overlapping full-GPU calls on %d streams: %d equal to the separate calls, %d "
        "reported an expired wait" % (len(runs), len(streams), len(runs) - expired, expired))


W2 = CONFIGS[4].scaled(batch=2, hq=2, hkv=2, T=16684, top_k=16, top_k_coarse=4, needles=0)


def test_two_level_head_expired_wait_sets_status_word():
    """The two-level step's head launch: a unit's coarse selector waits for
    its builder's rebuilt-row arrival, counted on the second word of the
    unit's coarse counter line. That word starts at -2^30 for unit 1, so the
    wait cannot end and expires after the bound; every kernel exits, the
    status word reads HS_STEP_WAIT_EXPIRED, the other units equal a normal
    call's results, the bias stays (the builder's arrival and the selector's
    take-off cancel), and after a zero-fill the workspace works normally."""
    if "p2" not in _P:
        log("setting up %s T=%d" % (W2.name, W2.T))
        _P["p2"] = Problem.make(W2)
    P = _P["p2"]
    q = P.q()
    summ = P.summaries()
    last = W2.nb - 1
    ids_r, cnt_r, out_r, ws_r = P.decode_step(q, summ, last)
    torch.cuda.synchronize()
    assert hs.hs_step_status(ws_r) == 0
    n = hs.hs_select_decode_workspace_size(P.kvs[0], summ["fine"], W2.hq, W2.top_k, W2.window,
                                           ids_r.shape[-1], summ["coarse"], W2.top_k_coarse)
    ws = hs.workspace(n, "cuda")
    unit, units = 1, W2.batch * W2.hkv
    at = (hs.STEP_SELECT_BYTE + 256 * units + 256 * unit + 4) // 4  # coarse line, word 1
    ws.view(torch.int32)[at] = -(1 << 30)
    torch.cuda.synchronize()
    log("calling the two-level hs_decode_step with unit %d's rebuilt-row word at -2^30" % unit)
    ids, cnt, out, _ = P.decode_step(q, summ, last, ws=ws)
    torch.cuda.synchronize()
    assert hs.hs_step_status(ws) == hs.HS_STEP_WAIT_EXPIRED
    b, g = divmod(unit, W2.hkv)
    for bb in range(W2.batch):
        for gg in range(W2.hkv):
            if (bb, gg) == (b, g):
                continue
            c = int(cnt_r[bb, gg])
            assert int(cnt[bb, gg]) == c and torch.equal(ids[bb, gg, :c], ids_r[bb, gg, :c])
            hq = slice(gg * W2.G, (gg + 1) * W2.G)
            assert torch.equal(out[bb, hq], out_r[bb, hq]), (bb, gg)
    assert int(ws.view(torch.int32)[at]) == -(1 << 30)
    ws.zero_()
    ids, cnt, out, _ = P.decode_step(q, summ, last, ws=ws)
    torch.cuda.synchronize()
    assert hs.hs_step_status(ws) == 0
    assert torch.equal(ids, ids_r) and torch.equal(cnt, cnt_r) and torch.equal(out, out_r)
    log("head's expired wait reported; workspace reusable after a zero-fill")
