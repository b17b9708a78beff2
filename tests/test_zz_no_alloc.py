"""hs_decode_step_noalloc (the decode step with the library's own device
array as its workspace, for callers that cannot allocate) against
hs_decode_step with a caller workspace: ids, counts, outputs and refreshed
summary tables must be bitwise equal, on two calls in a row, the second with
a smaller input (fewer sequences, a shorter context and another block
size), and on a two-level workload. (The refusal of a step whose workspace
would exceed the array is a host check, tested in test_capi_host.py.)"""
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
from gpu_helpers import Problem, log
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

C = CONFIGS
BIG = C[3].scaled(T=32768, seq_lens=(32768, 30000, 20001, 777))
SMALL = C[2].scaled(batch=2, hq=8, hkv=4, T=5000, seq_lens=(5000, 3100))
TWO = C[4].scaled(batch=2, hq=4, hkv=4, T=40000, top_k=40, top_k_coarse=8,
                  seq_lens=(40000, 25000))


def run_both(P):
    """Returns (reference results, no-alloc results) of one decode step."""
    w = P.w
    q = P.q()
    res = []
    for noalloc in (False, True):
        summ = P.summaries()
        rb = w.nb - 1
        if not noalloc:
            ids, cnt, out, _ = P.decode_step(q, summ, rb)
        else:
            cap = min(w.nb, min(w.top_k, w.nb) + -(-w.window // w.S) + 1)
            ids = torch.full((w.batch, w.hkv, cap), -7, dtype=torch.int32, device="cuda")
            cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
            out = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32,
                             device="cuda")
            hs.hs_decode_step_noalloc(P.kvs[0], q, summ["fine"], w.top_k, w.window, rb, ids, cnt,
                                      out, summ.get("coarse"), w.top_k_coarse)
        torch.cuda.synchronize()
        res.append((ids, cnt, out, summ))
    return res


def check_equal(w, ref, got, what):
    (i0, c0, o0, s0), (i1, c1, o1, s1) = ref, got
    assert torch.equal(c0, c1), what
    assert torch.equal(i0, i1), what
    assert torch.equal(o0, o1), (what, float((o0 - o1).abs().max()))
    for lvl in s0:  # rows past a sequence's block count are never written
        S = s0[lvl].block_size
        for b, T in enumerate(w.seq_lens_array()):
            nb_b = -(-int(T) // S)
            assert torch.equal(s0[lvl].data[b, :, :nb_b], s1[lvl].data[b, :, :nb_b]), (
                what, lvl, b)


def test_noalloc_step_equals_decode_step_twice_then_smaller():
    big = Problem.make(BIG)
    small = Problem.make(SMALL)
    for P, what in ((big, "first call"), (big, "second call"), (small, "smaller input")):
        ref, got = run_both(P)
        check_equal(P.w, ref, got, what)
        log("no-alloc step == hs_decode_step: %s (%s)" % (what, P.w.name))


def test_noalloc_two_level_step():
    P = Problem.make(TWO)
    ref, got = run_both(P)
    check_equal(P.w, ref, got, "two-level")
