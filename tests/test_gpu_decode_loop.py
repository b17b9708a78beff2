"""GPU parity of decode-time cache maintenance: a multi-step decode loop.

Every step appends one token per sequence with hs_append_kv (its K and V row
written into the page slot at position T_b through the page table, T_b
advanced on the device), then runs hs_decode_step with the refresh of the
growing block, so T grows and the window moves. The generator is
counter-based, so the token appended at position t carries exactly the values
the full-length generator gives row t; the oracle is checked on every unit at
every step on K[:T_b], V[:T_b] with the step's drifting query. Rows at or past
each sequence's starting length are poisoned with NaN before the loop, so a
missing or misplaced append shows up in the outputs. One sequence reaches the
cache's capacity mid-loop: from then on its appends must change nothing.
At the end the pools hold the generator's rows and the incrementally
refreshed summary tables equal a full rebuild bit for bit.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
from gpu_helpers import (Problem, check_ids, check_rows, log, magnitudes, oracle_select,
                         unit_inputs)
from synth import device as sdev
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

C = CONFIGS
# (workload, steps): starting lengths cross block and page boundaries during
# the loop; the last sequence starts 10 tokens short of the capacity T
GROW = {
    "c3-grow": (C[3].scaled(batch=3, hq=8, hkv=2, T=4160, top_k=16, window=256,
                            random_pages=True, seq_lens=(4100, 3990, 4150)), 40),
    "c4-grow": (C[4].scaled(batch=2, hq=2, hkv=2, T=16420, top_k=16, top_k_coarse=4,
                            seq_lens=(16370, 16410)), 24),
    "c1-grow": (C[1].scaled(batch=2, T=1100, seq_lens=(1020, 1090)), 30),
}


def poison_tail(w, P):
    """NaN into every cached row at or past each sequence's starting length."""
    pt = w.page_table()
    lens = w.seq_lens_array()
    nan = float("nan")
    for kv in P.kvs:
        for pool in (kv.k_pool, kv.v_pool):
            for b in range(w.batch):
                for t in range(int(lens[b]), w.T):
                    pool[int(pt[b][t // w.page_size]), :, t % w.page_size, :] = nan


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", list(GROW))
def test_decode_loop_with_appends_matches_oracle(name):
    w, steps = GROW[name]
    log("%s: setting up (%d steps)" % (name, steps))
    P = Problem.make(w)
    poison_tail(w, P)
    kv = P.kvs[0]
    lens = [int(x) for x in w.seq_lens_array()]
    summ = P.summaries()
    # full-length rows of every unit (the generator), for the appends and the oracle
    rows = {(b, g): unit_inputs(w, 0, b, g) for b in range(w.batch) for g in range(w.hkv)}
    K_st = {(b, g): w.k_unit(0, b, g) for b in range(w.batch) for g in range(w.hkv)}
    V_st = {(b, g): w.v_unit(0, b, g) for b in range(w.batch) for g in range(w.hkv)}
    tdt = sdev.TORCH_DTYPE[w.dtype]
    ws = None
    ties = 0
    for s in range(steps):
        k_new = torch.zeros((w.batch, w.hkv, w.d), dtype=tdt)
        v_new = torch.zeros_like(k_new)
        for b in range(w.batch):
            if lens[b] < w.T:
                for g in range(w.hkv):
                    k_new[b, g] = sdev.to_torch(K_st[(b, g)][lens[b]], w.dtype)
                    v_new[b, g] = sdev.to_torch(V_st[(b, g)][lens[b]], w.dtype)
        hs.hs_append_kv(kv, k_new.cuda(), v_new.cuda())
        lens = [min(t + 1, w.T) for t in lens]
        refresh = min((t - 1) // w.S for t in lens if t > 0)
        q = P.q(0, s)
        ids_t, cnt_t, out_t, ws = P.decode_step(q, summ, refresh, ws=ws)
        torch.cuda.synchronize()
        assert kv.seq_lens.cpu().tolist() == lens, (s, kv.seq_lens.cpu().tolist(), lens)
        ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
        out = out_t.cpu().double().numpy()
        for (b, g), (_, K, V) in rows.items():
            T = lens[b]
            qo = unit_inputs(w, 0, b, g, s)[0]
            sel = oracle_select(w, qo, K, T)
            gi = ids[b, g, :cnt[b, g]]
            what = "%s step %d unit (%d,%d) T=%d" % (name, s, b, g, T)
            ties += check_ids(w, gi, sel, magnitudes(w, qo, K, T), T, what=what)
            ref = oracle.attend_unit(qo, K, V, T, gi, w.S)
            check_rows(w, out[b, g * w.G:(g + 1) * w.G], ref, what)
        if s % 10 == 0:
            log("%s: step %d ok (T = %s)" % (name, s, lens))
    # the pools hold the generator's rows up to each final length
    pt = w.page_table()
    for (b, g) in rows:
        t = np.arange(lens[b])
        pages = pt[b][t // w.page_size]
        got_k = kv.k_pool[torch.from_numpy(pages).long(), g,
                          torch.from_numpy(t % w.page_size).long()].cpu()
        got_v = kv.v_pool[torch.from_numpy(pages).long(), g,
                          torch.from_numpy(t % w.page_size).long()].cpu()
        assert torch.equal(got_k, sdev.to_torch(K_st[(b, g)][:lens[b]], w.dtype)), (b, g)
        assert torch.equal(got_v, sdev.to_torch(V_st[(b, g)][:lens[b]], w.dtype)), (b, g)
    # incrementally refreshed tables equal a full rebuild (rows of valid blocks)
    for key, tab in summ.items():
        fresh = hs.Summaries(torch.empty_like(tab.data), tab.kind, tab.block_size)
        hs.hs_build_summaries(kv, fresh)
        torch.cuda.synchronize()
        for b in range(w.batch):
            nb = -(-lens[b] // tab.block_size)
            assert torch.equal(tab.data[b, :, :nb].view(torch.int16 if tab.data.dtype ==
                                                        torch.bfloat16 else torch.int32),
                               fresh.data[b, :, :nb].view(torch.int16 if tab.data.dtype ==
                                                          torch.bfloat16 else torch.int32)), \
                (name, key, b)
    log("%s: %d steps, %d tolerated near-tie differences" % (name, steps, ties))


@pytest.mark.timeout(900)
def test_decode_loop_full_size_sampled():
    """The 128K workload at full size, as the benchmark's decode-loop figure
    runs it: 8 steps of hs_append_kv + hs_decode_step from lengths just below
    the cache's 131072 tokens (sequence 1 crosses a 32-token block boundary),
    rows past each starting length poisoned with NaN first. The appended rows
    are the generator's, copied out of the pools before the poisoning. Four
    sampled units are checked against the oracle at every step; at the end the
    refreshed tables equal a full rebuild."""
    base = C[3]
    start = (base.T - 8, base.T - 35, base.T - 3, base.T - 20)
    w = base.scaled(seq_lens=start)
    steps = 8
    log("config 3 decode loop at full size: %d steps from lengths %s" % (steps, start))
    P = Problem.make(w)
    kv = P.kvs[0]
    pt = w.page_table()
    new_rows = {}
    for b in range(w.batch):
        t = np.arange(start[b], w.T)
        pages = torch.from_numpy(pt[b][t // w.page_size].astype(np.int64)).cuda()
        slots = torch.from_numpy(t % w.page_size).cuda()
        new_rows[b] = (kv.k_pool[pages, :, slots].clone(), kv.v_pool[pages, :, slots].clone())
    poison_tail(w, P)
    summ = P.summaries()
    units = [(0, 0), (1, 3), (2, 5), (3, 7)]
    rows = {u: unit_inputs(w, 0, u[0], u[1]) for u in units}
    lens = list(start)
    ws = None
    ties = 0
    for s in range(steps):
        k_new = torch.zeros((w.batch, w.hkv, w.d), dtype=kv.k_pool.dtype, device="cuda")
        v_new = torch.zeros_like(k_new)
        for b in range(w.batch):
            if lens[b] < w.T:
                k_new[b] = new_rows[b][0][lens[b] - start[b]]
                v_new[b] = new_rows[b][1][lens[b] - start[b]]
        hs.hs_append_kv(kv, k_new, v_new)
        lens = [min(t + 1, w.T) for t in lens]
        refresh = min((t - 1) // w.S for t in lens)
        ids_t, cnt_t, out_t, ws = P.decode_step(P.q(0, s), summ, refresh, ws=ws)
        torch.cuda.synchronize()
        assert kv.seq_lens.cpu().tolist() == lens, (s, kv.seq_lens.cpu().tolist(), lens)
        ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
        out = out_t.cpu().double().numpy()
        for (b, g), (_, K, V) in rows.items():
            T = lens[b]
            qo = unit_inputs(w, 0, b, g, s)[0]
            sel = oracle_select(w, qo, K, T)
            gi = ids[b, g, :cnt[b, g]]
            what = "config 3 loop step %d unit (%d,%d) T=%d" % (s, b, g, T)
            ties += check_ids(w, gi, sel, magnitudes(w, qo, K, T), T, what=what)
            check_rows(w, out[b, g * w.G:(g + 1) * w.G], oracle.attend_unit(qo, K, V, T, gi, w.S),
                       what)
    for key, tab in summ.items():
        fresh = hs.Summaries(torch.empty_like(tab.data), tab.kind, tab.block_size)
        hs.hs_build_summaries(kv, fresh)
        torch.cuda.synchronize()
        for b in range(w.batch):
            nb = -(-lens[b] // tab.block_size)
            view = torch.int16 if tab.data.dtype == torch.bfloat16 else torch.int32
            assert torch.equal(tab.data[b, :, :nb].view(view), fresh.data[b, :, :nb].view(view)), \
                (key, b)
    log("config 3 decode loop: %d steps, lengths %s, %d tolerated near-tie differences" % (
        steps, lens, ties))
    del P
    torch.cuda.empty_cache()
