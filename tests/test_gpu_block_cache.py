"""GPU parity of the LRU cache of selected blocks (hs_block_cache_update)
against the CPU oracle, bit for bit: slot tables, the slot of every selected
block, the missed blocks and the per-unit counts, at every step.

Inputs: drifting random selections (most of a step's blocks kept from the
previous step, a few swapped), including empty selections, a capacity equal
to max_selected (every miss evicts) and one of several times max_selected;
then the real pipeline: query-drift steps of a small shared-selection
workload selected on the GPU, with the overlap between consecutive steps
reported.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
from gpu_helpers import Problem, log
from oracle.block_cache import cache_step
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu


def drift_selections(rng, units, steps, nb, ms):
    """[steps][units] ascending id lists; sizes vary in [0, ms]."""
    out = []
    cur = [sorted(rng.choice(nb, size=int(rng.integers(0, ms + 1)), replace=False).tolist())
           for _ in range(units)]
    for t in range(steps):
        if t:
            nxt = []
            for c in cur:
                k = int(rng.integers(0, ms + 1))
                keep = [b for b in c if rng.random() < 0.85][:k]
                pool = np.setdiff1d(np.arange(nb), keep)
                add = rng.choice(pool, size=k - len(keep), replace=False).tolist()
                nxt.append(sorted(keep + add))
            cur = nxt
        out.append(cur)
    return out


def run_and_check(sels, units, cap, ms, what):
    cache = hs.BlockCache.empty(units, cap)
    ref = [([-1] * cap, [-1] * cap) for _ in range(units)]
    ids = torch.full((units, ms), -5, dtype=torch.int32, device="cuda")
    cnt = torch.zeros(units, dtype=torch.int32, device="cuda")
    slot_of = torch.full((units, ms), -9, dtype=torch.int32, device="cuda")
    miss = torch.full((units, ms), -9, dtype=torch.int32, device="cuda")
    stats = torch.full((units, 3), -9, dtype=torch.int32, device="cuda")
    overlap = []
    for t, sel in enumerate(sels):
        h_ids = np.full((units, ms), -5, np.int32)
        for u, s in enumerate(sel):
            h_ids[u, :len(s)] = s
        ids.copy_(torch.from_numpy(h_ids))
        cnt.copy_(torch.tensor([len(s) for s in sel], dtype=torch.int32))
        hs.hs_block_cache_update(cache, t, ids, cnt, slot_of, miss, stats)
        torch.cuda.synchronize()
        g_blk, g_st = cache.slot_block.cpu().numpy(), cache.slot_stamp.cpu().numpy()
        g_sof, g_miss, g_stats = slot_of.cpu().numpy(), miss.cpu().numpy(), stats.cpu().numpy()
        for u, s in enumerate(sel):
            blk, st, sof, mb, h, m, d = cache_step(ref[u][0], ref[u][1], s, t)
            ref[u] = (blk, st)
            where = "%s step %d unit %d" % (what, t, u)
            assert g_blk[u].tolist() == blk and g_st[u].tolist() == st, where
            assert g_sof[u, :len(s)].tolist() == sof, where
            assert g_miss[u, :m].tolist() == mb, where
            assert g_stats[u].tolist() == [h, m, d], where
            if t and s:
                overlap.append(1.0 - d / len(s))
    return overlap


@pytest.mark.parametrize("units,cap,ms,nb", [(5, 24, 8, 64), (3, 8, 8, 40), (16, 580, 145, 4096),
                                             (2, 1024, 300, 2048)])
def test_block_cache_matches_oracle_on_drifting_selections(units, cap, ms, nb):
    rng = np.random.default_rng(units * 1000 + cap)
    sels = drift_selections(rng, units, 12, nb, ms)
    run_and_check(sels, units, cap, ms, "cap %d" % cap)


def test_block_cache_on_selections_of_the_pipeline():
    """Query-drift steps of a small shared-selection workload: each step's ids
    come from hs_select_blocks on the GPU; the cache (4 x max_selected) must
    match the oracle, and the overlap of consecutive steps is reported."""
    w = CONFIGS[5].scaled(batch=2, hq=8, hkv=2, T=8192, top_k=24, layers=1, steps=12)
    P = Problem.make(w)
    summ = P.summaries()
    ms = min(w.nb, w.top_k + -(-w.window // w.S) + 1)
    sels = []
    for t in range(w.steps):
        ids, cnt = P.select(P.q(0, t), summ)
        ids, cnt = ids.cpu().numpy(), cnt.cpu().numpy()
        sels.append([ids[b, g, :cnt[b, g]].tolist() for b in range(w.batch)
                     for g in range(w.hkv)])
    ov = run_and_check(sels, w.units, 4 * ms, ms, "pipeline")
    log("pipeline: overlap of consecutive selections min %.2f mean %.2f max %.2f" %
        (min(ov), float(np.mean(ov)), max(ov)))


def test_block_cache_many_stamp_classes():
    """Evictions that span more stamp classes than the kernel takes one by one
    (it sorts the rest): one new block per step fills 32 slots with 32
    distinct stamps, then a step misses 20 blocks at once."""
    units, cap, ms = 2, 32, 24
    sels = []
    for t in range(32):
        sels.append([[t], [100 + t]])          # one new block per step and unit
    sels.append([list(range(200, 220)), list(range(300, 320))])  # 20 misses each
    sels.append([[5] + list(range(200, 210)), list(range(300, 305))])  # ascending, as selected
    run_and_check(sels, units, cap, ms, "many classes")
