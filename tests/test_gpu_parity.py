"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small workloads are compared element by element on every unit; they keep the
five workloads' structure (dtype, head dim, group size, summary kind, block
and page sizes, needles, two levels, random pages, layers) at sizes the
oracle finishes in seconds, with ragged tails and ragged sequence lengths.
The full-size workloads run in the same launch configuration as the
benchmark and are checked on sampled units.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
from gpu_helpers import (Problem, check_ids, check_rows, log, magnitudes, oracle_select,
                         unit_inputs)
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

C = CONFIGS
SMALL = {
    "c1": C[1],
    "c1-ragged": C[1].scaled(batch=3, T=4133, seq_lens=(4133, 4000, 77)),
    "c2s": C[2].scaled(batch=2, hq=4, hkv=4, T=4133, seq_lens=(4133, 2100)),
    "c3s": C[3].scaled(batch=2, hq=8, hkv=2, T=8209, seq_lens=(8209, 5000)),
    "c4s": C[4].scaled(batch=2, hq=2, hkv=2, T=16684, top_k=16, top_k_coarse=4,
                       seq_lens=(16684, 9000)),
    "c5s": C[5].scaled(batch=2, hq=8, hkv=2, T=4160, top_k=6, layers=3),
    # top_k_coarse above the 9 coarse blocks: every coarse block is kept and
    # the fine level ranks every fine block, as a single level would
    "c4s-all-coarse": C[4].scaled(batch=1, hq=2, hkv=2, T=9000, top_k=20, top_k_coarse=12,
                                  needles=0),
    # 274 coarse blocks, more than one scoring chunk: the fused step refreshes
    # both tables and selects the coarse level in three launches instead of
    # its one-launch head
    "c4s-many-coarse": C[4].scaled(batch=1, hq=2, hkv=2, T=70001, coarse_S=256, top_k=40,
                                   top_k_coarse=8, needles=0),
    # two levels over box (min/max) fine summaries, fp32, GQA, d 64
    "c4s-box-f32-g4": C[4].scaled(batch=2, hq=8, hkv=2, d=64, T=9000, dtype="f32", kind="minmax",
                                  S=32, page_size=32, coarse_S=512, top_k=24, top_k_coarse=6,
                                  window=128, needles=0, seq_lens=(9000, 4100)),
    "g8-d64-mean": C[3].scaled(batch=2, hq=16, hkv=2, d=64, T=3001, kind="mean", S=64,
                               page_size=16, top_k=5, window=100, needles=0,
                               seq_lens=(3001, 1500)),
    "g2-f32-d128-box": C[1].scaled(hq=4, hkv=2, d=128, T=2500, kind="minmax", S=32,
                                   page_size=32, top_k=7),
    "g1-f32-d64-box-p8": C[1].scaled(batch=2, T=999, kind="minmax", S=16, page_size=8,
                                     top_k=9, window=40, random_pages=True,
                                     seq_lens=(999, 0)),
}
_PROBLEMS = {}


def problem(name, layers=1):
    key = (name, layers)
    if key not in _PROBLEMS:
        log("setting up %s" % name)
        _PROBLEMS[key] = Problem.make(SMALL[name], layers)
    return _PROBLEMS[key]


def units(w):
    return [(b, g) for b in range(w.batch) for g in range(w.hkv)]


@pytest.mark.parametrize("name", list(SMALL))
def test_summaries_match_oracle(name):
    P = problem(name)
    w = P.w
    summ = P.summaries()
    torch.cuda.synchronize()
    fine = summ["fine"].data.cpu()
    lens = w.seq_lens_array()
    for b, g in units(w):
        T = int(lens[b])
        _, K, _ = unit_inputs(w, 0, b, g)
        nb = -(-T // w.S)
        a, c = oracle.summarize(K[:T], w.S, w.kind)
        if w.kind == "minmax":
            got = fine[b, g, :nb].float().double().numpy()
            assert np.array_equal(got[:, 0], a), (name, b, g)   # exact
            assert np.array_equal(got[:, 1], c), (name, b, g)
        else:
            got = fine[b, g, :nb].double().numpy()
            assert np.all(np.abs(got - a) <= mean_bound(K[:T], w.S, a)), (name, b, g)
    if w.top_k_coarse:
        coarse = summ["coarse"].data.cpu().double().numpy()
        for b, g in units(w):
            T = int(lens[b])
            _, K, _ = unit_inputs(w, 0, b, g)
            mu = oracle.summary_mean(K[:T], w.coarse_S)
            got = coarse[b, g, :len(mu)]
            assert np.all(np.abs(got - mu) <= mean_bound(K[:T], w.coarse_S, mu)), (name, b, g)


def mean_bound(rows, S, mu):
    """fp32 bound for a mean of n stored values: summation error at most
    (n - 1) u sum|x| in any order, plus the rounding of the division and of
    the result (u = 2^-24)."""
    T = rows.shape[0]
    nb = len(mu)
    absum = np.stack([np.abs(rows[b * S:min(b * S + S, T)]).sum(axis=0) for b in range(nb)])
    n = np.minimum(S, T - np.arange(nb) * S)[:, None]
    u = 2.0 ** -24
    return (n - 1) * u * absum / n + 2 * u * np.abs(mu) + 1e-30


@pytest.mark.parametrize("name", list(SMALL))
def test_decode_with_oracle_ids(name):
    """Stage 3 alone: the oracle's selection fed to the GPU decode."""
    P = problem(name)
    w = P.w
    lens = w.seq_lens_array()
    cap = w.max_selected
    ids = np.full((w.batch, w.hkv, cap), -1, np.int32)
    cnt = np.zeros((w.batch, w.hkv), np.int32)
    ref = np.zeros((w.batch, w.hq, w.d))
    for b, g in units(w):
        T = int(lens[b])
        q, K, V = unit_inputs(w, 0, b, g)
        sel = oracle_select(w, q, K, T)
        ids[b, g, :len(sel.ids)] = sel.ids
        cnt[b, g] = len(sel.ids)
        ref[b, g * w.G:(g + 1) * w.G] = oracle.attend_unit(q, K, V, T, sel.ids, w.S)
    ids_t = torch.from_numpy(ids).cuda()
    cnt_t = torch.from_numpy(cnt).cuda()
    out = P.decode(P.q(), ids_t, cnt_t).cpu().double().numpy()
    err = check_rows(w, out, ref, name)
    log("%s decode max row rel err %.3g" % (name, err))


@pytest.mark.parametrize("name", list(SMALL))
def test_select_and_pipeline_match_oracle(name):
    """Stages 1-3 chained on the GPU; ids by the near-tie rule, outputs
    against the oracle's attention over the GPU's ids."""
    P = problem(name)
    w = P.w
    q = P.q()
    summ = P.summaries()
    ids_t, cnt_t = P.select(q, summ)
    out = P.decode(q, ids_t, cnt_t).cpu().double().numpy()
    ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
    lens = w.seq_lens_array()
    ties = 0
    ref = np.zeros_like(out)
    for b, g in units(w):
        T = int(lens[b])
        qo, K, V = unit_inputs(w, 0, b, g)
        sel = oracle_select(w, qo, K, T)
        gi = ids[b, g, :cnt[b, g]]
        ties += check_ids(w, gi, sel, magnitudes(w, qo, K, T), T, what="%s(%d,%d)" % (name, b, g))
        ref[b, g * w.G:(g + 1) * w.G] = oracle.attend_unit(qo, K, V, T, gi, w.S)
    err = check_rows(w, out, ref, name)
    log("%s pipeline: %d tolerated near-tie differences, max row rel err %.3g" % (name, ties, err))


@pytest.mark.parametrize("name", list(SMALL))
def test_fused_select_decode_equals_separate_calls(name):
    """hs_select_decode (selection and attention in one launch) gives the
    same ids, counts and bitwise the same outputs as hs_select_blocks followed
    by hs_sparse_decode; a second and a third call on the same workspace (its
    ready flags and arrival counters back at zero) repeat
    them exactly."""
    P = problem(name)
    q = P.q()
    summ = P.summaries()
    ids_s, cnt_s = P.select(q, summ)
    out_s = P.decode(q, ids_s, cnt_s)
    ws = None
    for call in range(3):
        ids_f, cnt_f, out_f, ws = P.select_decode(q, summ, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(cnt_f, cnt_s), (name, call)
        assert torch.equal(ids_f, ids_s), (name, call)
        assert torch.equal(out_f, out_s), (name, call, float((out_f - out_s).abs().max()))
    # the workspace starts with the control line (status word),
    # then the selection's arrival counters (two levels, one 256-byte line
    # per unit): all zero after a call
    units_n = P.w.batch * P.w.hkv
    end = hs.STEP_SELECT_BYTE + 2 * 256 * units_n
    assert int(ws[:end].view(torch.int32).abs().sum()) == 0, name
    log("%s fused == separate, 3 calls" % name)


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("where", ["last", "many"])
def test_decode_step_equals_refresh_then_select_decode(name, where):
    """hs_decode_step (summary refresh from refresh_begin on, selection and
    attention in one call) leaves the same summary tables, ids and counts
    and bitwise the same outputs as hs_build_summaries from refresh_begin
    (each level) followed by hs_select_decode. The refreshed rows start out
    poisoned in both tables; "many" refreshes 300 blocks (several scoring
    chunks of the fused launch)."""
    P = problem(name)
    w = P.w
    kv = P.kvs[0]
    q = P.q()
    refresh_begin = w.nb - 1 if where == "last" else max(0, w.nb - 300)
    tables = []
    for _ in range(2):
        summ = P.summaries()
        summ["fine"].data[:, :, refresh_begin:] = 7.0
        if "coarse" in summ:
            cb = refresh_begin * w.S // w.coarse_S
            summ["coarse"].data[:, :, cb:] = 7.0
        tables.append(summ)
    ref, got = tables
    hs.hs_build_summaries(kv, ref["fine"], refresh_begin)
    if "coarse" in ref:
        hs.hs_build_summaries(kv, ref["coarse"], refresh_begin * w.S // w.coarse_S)
    ids_r, cnt_r, out_r, _ = P.select_decode(q, ref)
    ws = None
    for call in range(2):  # the second call on the same workspace repeats the first
        ids_g, cnt_g, out_g, ws = P.decode_step(q, got, refresh_begin, ws=ws)
        torch.cuda.synchronize()
        for lvl in ref:  # rows past a unit's block count are never written
            S = ref[lvl].block_size
            for b, T in enumerate(w.seq_lens_array()):
                nb_b = -(-int(T) // S)
                assert torch.equal(ref[lvl].data[b, :, :nb_b], got[lvl].data[b, :, :nb_b]), (
                    name, where, lvl, call, b)
        assert torch.equal(cnt_g, cnt_r) and torch.equal(ids_g, ids_r), (name, where, call)
        assert torch.equal(out_g, out_r), (name, where, call)
    log("%s decode step (refresh from %d) == refresh + select_decode" % (name, refresh_begin))


@pytest.mark.parametrize("top_k,window", [(0, 256), (0, 0), (10 ** 6, 0), (3, 10 ** 6), (64, 1)])
def test_selection_edge_values(top_k, window):
    """k = 0 (window only), nothing selected at all, k >= number of blocks
    (dense), a window longer than the context, a one-token window."""
    P = problem("c1-ragged")
    w = P.w
    q = P.q()
    summ = P.summaries()
    cap = min(w.nb, min(top_k, w.nb) + -(-window // w.S) + 1)
    ids_t, cnt_t = P.select(q, summ, top_k=top_k, window=window, max_selected=cap)
    out = P.decode(q, ids_t, cnt_t).cpu().double().numpy()
    ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
    lens = w.seq_lens_array()
    ref = np.zeros_like(out)
    for b, g in units(w):
        T = int(lens[b])
        qo, K, V = unit_inputs(w, 0, b, g)
        sel = oracle_select(w, qo, K, T, top_k=top_k, window=window)
        check_ids(w, ids[b, g, :cnt[b, g]], sel, magnitudes(w, qo, K, T), T, window=window)
        ref[b, g * w.G:(g + 1) * w.G] = oracle.attend_unit(qo, K, V, T, sel.ids, w.S)
        if top_k >= w.nb:
            assert cnt[b, g] == -(-T // w.S)
    check_rows(w, out, ref, "edge k=%d W=%d" % (top_k, window))
    if top_k == 0 and window == 0:
        assert np.all(cnt == 0) and np.all(out == 0)
    ids_f, cnt_f, out_f, _ = P.select_decode(q, summ, top_k=top_k, window=window,
                                             max_selected=cap)
    assert torch.equal(cnt_f, cnt_t) and torch.equal(ids_f, ids_t)
    assert torch.equal(out_f.cpu().double(), torch.from_numpy(out))


def test_page_permutation_invariance_and_determinism():
    """Identity vs random physical page table: identical ids and bitwise
    identical outputs; a second run is bitwise identical; decode leaves the
    id buffer untouched."""
    P1 = problem("c5s")
    w = P1.w
    P2 = Problem.make(w.scaled(random_pages=False))
    outs = []
    for P in (P1, P2, P1):
        q = P.q()
        summ = P.summaries()
        ids, cnt = P.select(q, summ)
        before = ids.clone()
        out = P.decode(q, ids, cnt)
        torch.cuda.synchronize()
        assert torch.equal(ids, before)
        outs.append((ids.cpu(), cnt.cpu(), out.cpu()))
    for o in outs[1:]:
        assert torch.equal(o[0], outs[0][0]) and torch.equal(o[1], outs[0][1])
        assert torch.equal(o[2], outs[0][2])


def test_shared_selection_across_layers():
    """Selection from layer 0's query and summaries, reused by the decode of
    every layer (each with its own q, K, V); the ids are never modified."""
    P = problem("c5s", layers=3)
    w = P.w
    q0 = P.q(0)
    summ = P.summaries(0)
    ids_t, cnt_t = P.select(q0, summ)
    ids0 = ids_t.clone()
    outs = [P.decode(P.q(layer), ids_t, cnt_t, layer=layer) for layer in range(3)]
    torch.cuda.synchronize()
    assert torch.equal(ids_t, ids0)
    ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
    lens = w.seq_lens_array()
    for b, g in units(w):
        T = int(lens[b])
        qo, K0, _ = unit_inputs(w, 0, b, g)
        sel = oracle_select(w, qo, K0, T)
        check_ids(w, ids[b, g, :cnt[b, g]], sel, magnitudes(w, qo, K0, T), T)
    for layer in range(3):
        out = outs[layer].cpu().double().numpy()
        ref = np.zeros_like(out)
        for b, g in units(w):
            T = int(lens[b])
            ql, K, V = unit_inputs(w, layer, b, g)
            ref[b, g * w.G:(g + 1) * w.G] = oracle.attend_unit(ql, K, V, T, ids[b, g, :cnt[b, g]],
                                                               w.S)
        check_rows(w, out, ref, "layer %d" % layer)


def test_incremental_refresh_of_last_block():
    """After tokens are appended, rebuilding only from the last block on
    equals a full rebuild (the rows before it are untouched)."""
    import hierarchical_sparse_attention_amd as hs
    P = problem("c3s")
    w = P.w
    kv = P.kvs[0]
    short = torch.tensor([8209 - 45, 5000 - 20], dtype=torch.int32, device="cuda")
    kv_short = hs.KVCache(kv.k_pool, kv.v_pool, kv.page_table, short, w.T)
    inc = hs.Summaries.empty(kv, w.kind, w.S)
    inc.data.fill_(0)
    hs.hs_build_summaries(kv_short, inc)
    first_changed = int(min(short.cpu().numpy() // w.S))  # first block holding a new token
    hs.hs_build_summaries(kv, inc, block_begin=first_changed)
    full = hs.Summaries.empty(kv, w.kind, w.S)
    full.data.fill_(0)
    hs.hs_build_summaries(kv, full)
    torch.cuda.synchronize()
    assert torch.equal(inc.data, full.data)


ABSENT = {
    "bf16": C[3].scaled(batch=3, hq=8, hkv=2, T=3001, kind="mean", S=16, page_size=16,
                        top_k=5, window=100, needles=0, seq_lens=(3001, 2000, 1500)),
    "f32": C[1].scaled(batch=3, hq=4, hkv=2, d=128, T=3001, page_size=16,
                       seq_lens=(3001, 2000, 1500)),
}


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("S", [1, 16, 48, 64])
def test_decode_skips_absent_pages(dtype, S):
    """Page-table entries outside [0, num_phys_pages) (-1 and past the pool)
    make their tokens absent: the decode attends over the selected tokens on
    valid pages only, for block sizes that make a 32-token stage straddle
    pages (page size 16) and for token lists. Sequence 2 has no valid page
    at all, so its rows are 0."""
    w = ABSENT[dtype]
    key = ("absent", dtype)
    if key not in _PROBLEMS:
        _PROBLEMS[key] = Problem.make(w)
    P = _PROBLEMS[key]
    kv0 = P.kvs[0]
    pt = w.page_table().copy()
    rng = np.random.default_rng(5)
    bad = rng.random(pt.shape) < 0.3
    pt[bad & (rng.random(pt.shape) < 0.5)] = -1
    pt[bad & (pt >= 0)] = w.num_phys_pages + 5
    pt[2] = -1
    kv = hs.KVCache(kv0.k_pool, kv0.v_pool, torch.from_numpy(pt).cuda(), kv0.seq_lens, w.T)
    lens = w.seq_lens_array()
    n_ids = 24 if S > 1 else 400
    ids = np.full((w.batch, w.hkv, n_ids), -1, np.int32)
    cnt = np.zeros((w.batch, w.hkv), np.int32)
    for b, g in units(w):
        T = int(lens[b])
        nb = -(-T // S)
        pick = np.sort(rng.choice(nb, size=min(n_ids, nb), replace=False)).astype(np.int32)
        ids[b, g, :len(pick)] = pick
        cnt[b, g] = len(pick)
    ws = hs.workspace(hs.hs_decode_workspace_size(kv, w.hq, S, n_ids), "cuda")
    out = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
    hs.hs_sparse_decode(kv, P.q(), S, torch.from_numpy(ids).cuda(), torch.from_numpy(cnt).cuda(),
                        out, ws)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    ref = np.zeros_like(o)
    absent = 0
    for b, g in units(w):
        T = int(lens[b])
        qo, K, V = unit_inputs(w, 0, b, g)
        toks = [t for beta in ids[b, g, :cnt[b, g]] for t in range(beta * S, min(beta * S + S, T))]
        ok = [t for t in toks if 0 <= pt[b, t // w.page_size] < w.num_phys_pages]
        absent += len(toks) - len(ok)
        ref[b, g * w.G:(g + 1) * w.G] = oracle.attend_unit(qo, K, V, T, np.array(ok, np.int32), 1)
    assert np.all(o[2] == 0), "a sequence without valid pages must give zero rows"
    err = check_rows(w, o, ref, "absent pages %s S=%d" % (dtype, S))
    log("absent pages %s S=%d: %d absent tokens skipped, max row rel err %.3g" % (
        dtype, S, absent, err))


@pytest.mark.parametrize("name", ["c3s", "c1-ragged", "c4s"])
def test_split_count_invariance(name):
    """The same ids decoded through id rows of different capacity: the
    capacity sets the number of split tasks per unit (hs_decode_workspace_size
    grows with it), so the tokens are cut into different runs and merged in a
    different order; both outputs match the oracle's attention over the ids."""
    P = problem(name)
    w = P.w
    q = P.q()
    summ = P.summaries()
    ids_t, cnt_t = P.select(q, summ)
    ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
    lens = w.seq_lens_array()
    ref = np.zeros((w.batch, w.hq, w.d))
    for b, g in units(w):
        qo, K, V = unit_inputs(w, 0, b, g)
        ref[b, g * w.G:(g + 1) * w.G] = oracle.attend_unit(qo, K, V, int(lens[b]),
                                                           ids[b, g, :cnt[b, g]], w.S)
    cap0 = ids.shape[-1]
    # splits per unit: min(capacity, ceil(256 / units)), doubled once a split
    # would hold >= 2048 tokens at full capacity; the largest capacity below
    # crosses that threshold, the smallest caps the count at the ids' count
    per = -(-256 // w.units)
    big = max(cap0, -(-2048 * per // w.S)) + 1
    sizes = set()
    for cap in (int(cnt.max()), cap0, big):
        wide = np.full((w.batch, w.hkv, cap), -1, np.int32)
        wide[:, :, :min(cap, cap0)] = ids[:, :, :min(cap, cap0)]
        sizes.add(hs.hs_decode_workspace_size(P.kvs[0], w.hq, w.S, cap))
        out = P.decode(q, torch.from_numpy(wide).cuda(), cnt_t).cpu().double().numpy()
        check_rows(w, out, ref, "%s capacity %d" % (name, cap))
    assert len(sizes) > 1, "%s: capacities did not change the split count" % name
