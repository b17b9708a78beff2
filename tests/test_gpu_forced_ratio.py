"""GPU parity of ratio-based k and caller-forced blocks (the reserve set).

k_b = max(1, int(nb_b * ratio)) per unit ("SparDA" section 3.2 / 3.4) and a
seeded random reserve set of 2 % of each unit's blocks, padded with -1 and
salted with a duplicate, an out-of-range id and a window block ("SparDA"
section 3.4: the caller draws it, so both sides see the same ids). Every
top-k path of the library is covered: the register path (single level, up to
4096 candidates), the two-level bitmap path and the general path (more than
4096 candidates). The separate calls (hs_select_blocks + hs_sparse_decode)
and the fused hs_decode_step must agree bit for bit and match the oracle.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
from gpu_helpers import Problem, check_ids, check_rows, log, magnitudes, unit_inputs
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

C = CONFIGS
WORK = {
    "regs": C[3].scaled(batch=2, hq=8, hkv=2, T=8209, seq_lens=(8209, 5000)),
    "two-level": C[4].scaled(batch=2, hq=2, hkv=2, T=16684, top_k=16, top_k_coarse=4,
                             seq_lens=(16684, 9000)),
    "general": C[3].scaled(batch=1, hq=4, hkv=1, T=20000, S=4, page_size=4, top_k=50,
                           window=64, needles=0),
}
_P = {}


def problem(name):
    if name not in _P:
        log("setting up %s" % name)
        _P[name] = Problem.make(WORK[name])
    return _P[name]


def reserve_sets(w, seed, frac=0.02):
    """[B][Hkv][cap] int32 forced ids (the caller's random draw)."""
    rng = np.random.default_rng(seed)
    lens = w.seq_lens_array()
    sets = []
    for b in range(w.batch):
        nb = -(-int(lens[b]) // w.S)
        for g in range(w.hkv):
            r = max(1, int(nb * frac)) if nb else 0
            ids = rng.choice(max(nb, 1), size=min(r, max(nb, 1)), replace=False).tolist()
            extra = [ids[0] if ids else 0, nb + 3, max(nb - 1, 0), -1]
            sets.append(ids + extra)
    cap = max(len(s) for s in sets)
    arr = np.full((w.batch, w.hkv, cap), -1, np.int32)
    for i, s in enumerate(sets):
        arr[i // w.hkv, i % w.hkv, :len(s)] = s
    return arr


@pytest.mark.parametrize("name", list(WORK))
@pytest.mark.parametrize("mode", ["forced", "ratio", "both"])
def test_forced_and_ratio_match_oracle(name, mode):
    w = WORK[name]
    P = problem(name)
    kv = P.kvs[0]
    q = P.q()
    summ = P.summaries()
    ratio = 0.07 if mode in ("ratio", "both") else 0.0
    forced = reserve_sets(w, 7) if mode in ("forced", "both") else None
    fcap = forced.shape[-1] if forced is not None else 0
    forced_t = torch.from_numpy(forced).cuda() if forced is not None else None
    kmax = max(1, int(w.nb * float(np.float32(ratio)))) if ratio > 0 else w.top_k
    cap = min(w.nb, min(kmax, w.nb) + -(-w.window // w.S) + 1 + fcap)
    coarse = summ.get("coarse")
    ids = torch.full((w.batch, w.hkv, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
    n = hs.hs_select_workspace_size(kv, summ["fine"], w.hq, w.top_k, w.window, cap, coarse,
                                    w.top_k_coarse, ratio, forced_t)
    hs.hs_select_blocks(kv, q, summ["fine"], w.top_k, w.window, ids, cnt, hs.workspace(n, "cuda"),
                        coarse, w.top_k_coarse, top_k_ratio=ratio, forced=forced_t)
    out = P.decode(q, ids, cnt)
    # fused step (refresh of the last block: the table does not change)
    ids2 = torch.full_like(ids, -7)
    cnt2 = torch.full_like(cnt, -7)
    out2 = torch.full_like(out, float("nan"))
    n2 = hs.hs_select_decode_workspace_size(kv, summ["fine"], w.hq, w.top_k, w.window, cap,
                                            coarse, w.top_k_coarse, ratio, forced_t)
    hs.hs_decode_step(kv, q, summ["fine"], w.top_k, w.window, (w.T - 1) // w.S, ids2, cnt2, out2,
                      hs.workspace(n2, "cuda"), coarse, w.top_k_coarse, top_k_ratio=ratio,
                      forced=forced_t)
    torch.cuda.synchronize()
    g_ids, g_cnt = ids.cpu().numpy(), cnt.cpu().numpy()
    assert np.array_equal(cnt2.cpu().numpy(), g_cnt)
    i2 = ids2.cpu().numpy()
    for b in range(w.batch):
        for g in range(w.hkv):
            assert np.array_equal(i2[b, g, :g_cnt[b, g]], g_ids[b, g, :g_cnt[b, g]]), (b, g)
    o1, o2 = out.cpu().double().numpy(), out2.cpu().double().numpy()
    assert np.array_equal(o1, o2), float(np.nanmax(np.abs(o1 - o2)))
    lens = w.seq_lens_array()
    ties = 0
    for b in range(w.batch):
        for g in range(w.hkv):
            T = int(lens[b])
            qo, K, V = unit_inputs(w, 0, b, g)
            f = forced[b, g] if forced is not None else None
            sel = oracle.select_unit(qo, K, T, w.kind, w.S, w.top_k, w.window,
                                     coarse_S=w.coarse_S, top_k_coarse=w.top_k_coarse,
                                     top_k_ratio=ratio, forced=f)
            gi = g_ids[b, g, :g_cnt[b, g]]
            what = "%s/%s unit (%d,%d)" % (name, mode, b, g)
            if f is not None:
                nb = -(-T // w.S)
                assert set(int(x) for x in f if 0 <= x < nb) <= set(gi.tolist()), what
            ties += check_ids(w, gi, sel, magnitudes(w, qo, K, T), T, what=what)
            ref = oracle.attend_unit(qo, K, V, T, gi, w.S)
            check_rows(w, o1[b, g * w.G:(g + 1) * w.G], ref, what)
    log("%s/%s: %d tolerated near-tie differences, counts %s" % (name, mode, ties,
                                                                 g_cnt.reshape(-1).tolist()))


def test_whole_coarse_block_loading():
    """Two levels whose fine top-k covers every candidate slice: the GPU keeps
    every fine block of its kept coarse blocks (and the window), as the oracle
    does, through the separate calls and the fused step."""
    w = WORK["two-level"]
    P = problem("two-level")
    kv = P.kvs[0]
    q = P.q()
    summ = P.summaries()
    R = w.coarse_S // w.S
    k = w.top_k_coarse * R
    cap = min(w.nb, k + -(-w.window // w.S) + 1)
    ids = torch.full((w.batch, w.hkv, cap), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
    n = hs.hs_select_workspace_size(kv, summ["fine"], w.hq, k, w.window, cap, summ["coarse"],
                                    w.top_k_coarse)
    hs.hs_select_blocks(kv, q, summ["fine"], k, w.window, ids, cnt, hs.workspace(n, "cuda"),
                        summ["coarse"], w.top_k_coarse)
    out = P.decode(q, ids, cnt)
    torch.cuda.synchronize()
    g_ids, g_cnt = ids.cpu().numpy(), cnt.cpu().numpy()
    o = out.cpu().double().numpy()
    lens = w.seq_lens_array()
    for b in range(w.batch):
        for g in range(w.hkv):
            T = int(lens[b])
            qo, K, V = unit_inputs(w, 0, b, g)
            sel = oracle.select_unit(qo, K, T, w.kind, w.S, k, w.window, coarse_S=w.coarse_S,
                                     top_k_coarse=w.top_k_coarse)
            gi = g_ids[b, g, :g_cnt[b, g]]
            nb = -(-T // w.S)
            full = {c * R + r for c in sel.coarse_ids.tolist() for r in range(R) if c * R + r < nb}
            assert full <= set(gi.tolist()), (b, g)
            check_ids(w, gi, sel, magnitudes(w, qo, K, T), T, what="whole coarse (%d,%d)" % (b, g))
            check_rows(w, o[b, g * w.G:(g + 1) * w.G], oracle.attend_unit(qo, K, V, T, gi, w.S),
                       "whole coarse (%d,%d)" % (b, g))
