"""Pins of the CPU oracle against what the pages and mathematics fix.

Each test checks the oracle against something other than itself: a closed
form, a brute-force enumeration, a textbook routine (numpy dense softmax
attention), an invariant, or a structural figure printed on the pages
(tests/golden/pages_structural.json). The mistakes each one is meant to catch
are named in its docstring.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth
from synth.workloads import CONFIGS

GOLD = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(1234)


def dense_attention(q, K, V, scale):
    """Textbook softmax(q K^T * scale) V in float64 (numpy)."""
    lg = (q @ K.T) * scale
    lg = lg - lg.max(axis=-1, keepdims=True)
    p = np.exp(lg)
    return (p / p.sum(axis=-1, keepdims=True)) @ V


# --------------------------------------------------------------- summaries
def test_mean_summary_closed_form_integer_keys():
    """Integer keys k_t,i = t + 1000 i: each block mean is (t0 + t1 - 1)/2 + 1000 i
    exactly, partial last block over its valid tokens only. Catches an
    off-by-one block range, dividing by S instead of the valid count, or a
    transposed [t][i] index."""
    T, d, S = 203, 5, 64
    rows = np.array([[t + 1000.0 * i for i in range(d)] for t in range(T)])
    mu = oracle.summary_mean(rows, S)
    assert mu.shape == (4, d)
    for beta in range(4):
        t0, t1 = beta * S, min(beta * S + S, T)
        want = (t0 + t1 - 1) / 2.0 + 1000.0 * np.arange(d)
        assert np.array_equal(mu[beta], want)


def test_minmax_summary_brute_force():
    """Min/max per block and dimension equals numpy's reduction, bit-exact,
    including a partial last block and a block of a single token."""
    for T, S in ((100, 32), (65, 64), (64, 64), (7, 1)):
        rows = synth.widen(synth.normal(5, 2, 0, T * 16, "bf16"), "bf16").reshape(T, 16)
        mn, mx = oracle.summary_minmax(rows, S)
        for beta in range(-(-T // S)):
            blk = rows[beta * S:min(beta * S + S, T)]
            assert np.array_equal(mn[beta], blk.min(axis=0))
            assert np.array_equal(mx[beta], blk.max(axis=0))


# ------------------------------------------------------------------ scores
def test_scores_reduce_to_dot_product_at_block_size_one():
    """With S = 1 the mean is the key itself and the box is a point, so both
    scores equal sum_j q_j . k_t exactly (closed form). Catches a wrong sign,
    min and max swapped in one term, or heads not summed."""
    G, d, T = 4, 32, 50
    q = synth.widen(synth.normal(9, 1, 0, G * d, "bf16"), "bf16").reshape(G, d)
    K = synth.widen(synth.normal(9, 2, 0, T * d, "bf16"), "bf16").reshape(T, d)
    want = K @ q.sum(axis=0)
    mu = oracle.summary_mean(K, 1)
    mn, mx = oracle.summary_minmax(K, 1)
    assert np.allclose(oracle.scores_mean(q, mu), want, rtol=1e-14, atol=1e-12)
    assert np.allclose(oracle.scores_minmax(q, mn, mx), want, rtol=1e-14, atol=1e-12)


def test_quest_bound_dominates_every_key_in_the_block():
    """Invariant: the box bound is >= max_t q . k_t per head, and the group sum
    of bounds is >= max_t sum_j q_j . k_t; it is tight (equality) for a
    single head when one key holds every per-dimension extreme that the sign
    of q picks. Catches taking min where max is needed, or the
    mean instead of the box."""
    G, d, T, S = 4, 64, 512, 32
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    mn, mx = oracle.summary_minmax(K, S)
    sg = oracle.scores_minmax(q, mn, mx)
    for beta in range(T // S):
        blk = K[beta * S:(beta + 1) * S]
        per_head = [oracle.scores_minmax(q[j:j + 1], mn[beta:beta + 1], mx[beta:beta + 1])[0]
                    for j in range(G)]
        for j in range(G):
            assert per_head[j] >= (blk @ q[j]).max() - 1e-12
        assert sg[beta] >= (blk @ q.sum(axis=0)).max() - 1e-12
        assert abs(sg[beta] - sum(per_head)) < 1e-9
    # tightness: plant the extreme corner as a real key
    q1 = q[:1]
    blk = K[:S].copy()
    blk[3] = np.where(q1[0] > 0, blk.max(axis=0), blk.min(axis=0))
    mn1, mx1 = oracle.summary_minmax(blk, S)
    assert abs(oracle.scores_minmax(q1, mn1, mx1)[0] - (blk @ q1[0]).max()) < 1e-12


def test_mean_score_is_mean_of_token_scores():
    """Linearity: q . mean(k) = mean(q . k) over the block's valid tokens."""
    G, d, T, S = 2, 16, 150, 64
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    s = oracle.scores_mean(q, oracle.summary_mean(K, S))
    tok = K @ q.sum(axis=0)
    for beta in range(3):
        assert abs(s[beta] - tok[beta * S:min(beta * S + S, T)].mean()) < 1e-12


# ------------------------------------------------------------------- top-k
def _brute_topk(s, k, ids=None):
    ids = list(range(len(s))) if ids is None else list(ids)
    order = sorted(range(len(s)), key=lambda c: (-float(np.float32(s[c])), ids[c]))
    return [ids[c] for c in order[:max(0, min(k, len(s)))]]


@pytest.mark.parametrize("n,k", [(1, 1), (7, 3), (64, 8), (64, 64), (64, 100), (33, 0)])
def test_topk_equals_brute_force_sort_with_ties(n, k):
    """Top-k equals a brute-force full sort by (fp32 score desc, id asc) on tiny
    inputs with planted exact duplicates (lowest index wins) and +-0."""
    s = rng.normal(size=n)
    if n >= 7:
        s[[1, 4, 5]] = s[2]          # exact ties
        s[6] = 0.0
        s[0] = -0.0                  # -0 ties with +0
    got = oracle.topk(s, k)
    assert got.tolist() == _brute_topk(s, k)
    # property check independent of any sort: kept >= dropped; equal keys at the
    # boundary are resolved towards lower ids
    keep = set(got.tolist())
    f = s.astype(np.float32)
    for a in keep:
        for b in set(range(n)) - keep:
            assert f[a] > f[b] or (f[a] == f[b] and a < b)


def test_topk_ranks_in_float32_precision():
    """Scores equal after rounding to float32 (the pages' score precision)
    tie, and the lower block index wins; a difference of one float32 ulp
    does decide."""
    base = 1.0
    s = np.array([base + 1e-12, base, base + 2 ** -23])
    assert oracle.topk(s, 1).tolist() == [2]
    assert oracle.topk(s[:2], 1).tolist() == [0]
    s2 = np.array([base, base + 1e-12])
    assert oracle.topk(s2, 1).tolist() == [0]


def test_topk_over_candidate_ids():
    s = np.array([0.5, 2.0, 2.0, -1.0])
    ids = np.array([40, 17, 3, 99], np.int32)
    assert oracle.topk(s, 2, ids).tolist() == [3, 17]


# ------------------------------------------------------------------ window
@pytest.mark.parametrize("T,S,W", [(4096, 64, 256), (4100, 64, 256), (4096, 64, 0),
                                   (100, 32, 1000), (131072, 32, 512), (97, 10, 15)])
def test_window_blocks_brute_force(T, S, W):
    """Window = blocks whose token range meets [T-W, T), by enumerating tokens."""
    want = sorted({t // S for t in range(max(0, T - W), T)}) if W > 0 else []
    assert oracle.window_blocks(T, S, W).tolist() == want


# ------------------------------------------------------------ selection
def test_select_is_topk_union_window_ascending():
    T, S, k, W, G, d = 4096 + 17, 64, 8, 256, 2, 32
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    sel = oracle.select_unit(q, K, T, "minmax", S, k, W)
    mn, mx = oracle.summary_minmax(K, S)
    s = oracle.scores_minmax(q, mn, mx)
    want = sorted(set(_brute_topk(s, k)) | set(oracle.window_blocks(T, S, W).tolist()))
    assert sel.ids.tolist() == want
    assert len(sel.ids) <= k + -(-W // S) + 1
    assert np.all(np.diff(sel.ids) > 0)


def test_two_level_with_all_coarse_blocks_equals_single_level():
    """kc >= number of coarse blocks makes every fine block a candidate, so the
    two-level result equals single-level fine selection."""
    T, S, C, G, d = 8192, 64, 1024, 1, 32
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    one = oracle.select_unit(q, K, T, "mean", S, 20, 512)
    two = oracle.select_unit(q, K, T, "mean", S, 20, 512, coarse_S=C, top_k_coarse=8)
    assert one.ids.tolist() == two.ids.tolist()


def test_two_level_candidates_lie_in_selected_coarse_blocks():
    T, S, C, G, d = 16384, 64, 1024, 1, 32
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    sel = oracle.select_unit(q, K, T, "mean", S, 10, 512, coarse_S=C, top_k_coarse=4)
    coarse = set(sel.coarse_ids.tolist())
    cand = np.nonzero(~np.isnan(sel.fine_scores))[0]
    assert len(coarse) == 4 and len(cand) == 4 * (C // S)
    assert {c * S // C for c in cand} == coarse
    win = set(oracle.window_blocks(T, S, 512).tolist())
    assert all((b * S // C) in coarse or b in win for b in sel.ids)
    # the coarse ranking is the brute-force ranking of the coarse means
    cs = oracle.scores_mean(q, oracle.summary_mean(K, C))
    assert sel.coarse_ids.tolist() == _brute_topk(cs, 4)


def test_pages_structural_counts_two_level_256k():
    """At the two-level 256K workload a unit has 256 coarse blocks (one
    1024-token summary each) and 32 x 16 = 512 fine candidates, as the
    pages count; the attended set is window + top-128 slices. (The counts do
    not depend on the head dim, so a narrow d keeps the test small.)"""
    g = json.load(open(os.path.join(GOLD, "pages_structural.json")))
    w = CONFIGS[4].scaled(batch=1, hq=1, hkv=1, d=8)
    assert w.nc == g["coarse_blocks_256k"]["value"]
    K = synth.widen(w.k_unit(0, 0, 0), "bf16")
    q = synth.widen(w.q(), "bf16")[0, :1]
    sel = oracle.select_unit(q, K, w.T, "mean", w.S, w.top_k, w.window,
                             coarse_S=w.coarse_S, top_k_coarse=w.top_k_coarse)
    assert len(sel.coarse_ids) == g["fine_candidates_256k"]["top_k_coarse"]
    ncand = int((~np.isnan(sel.fine_scores)).sum())
    assert ncand == g["fine_candidates_256k"]["value"]
    assert w.window == g["window_tokens"]["value"]
    assert len(sel.ids) <= w.top_k + w.window // w.S
    # planted needles rank: every needle slice whose coarse block was kept is selected
    kept = set(sel.coarse_ids.tolist())
    for beta in w.needle_blocks(0, 0):
        if beta * w.S // w.coarse_S in kept:
            assert beta in sel.ids


def test_pages_structural_rows_and_ratio():
    g = json.load(open(os.path.join(GOLD, "pages_structural.json")))
    r = g["table_rows_128k_64"]
    assert -(-r["context"] // r["block"]) == r["value"]
    rt = g["ratio_topk"]
    assert max(1, int(rt["n_blocks"] * rt["ratio"])) == rt["value"] == CONFIGS[5].top_k


# --------------------------------------------------------------- attention
@pytest.mark.parametrize("T,S,G,d", [(4096, 64, 4, 64), (1000, 32, 1, 128), (33, 64, 2, 64)])
def test_all_blocks_selected_equals_dense_attention(T, S, G, d):
    """k >= number of blocks: the sparse attention IS dense attention
    (textbook softmax, numpy float64)."""
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    V = rng.normal(size=(T, d))
    ids = np.arange(-(-T // S), dtype=np.int32)
    got = oracle.attend_unit(q, K, V, T, ids, S)
    want = dense_attention(q, K, V, 1 / math.sqrt(d))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
    # and through the full selection with k = nb
    sel = oracle.select_unit(q, K, T, "mean", S, 10 ** 6, 0)
    assert sel.ids.tolist() == ids.tolist()


def test_window_only_equals_sliding_window_attention():
    """k = 0: attention over exactly the window's blocks (sliding-window
    attention on block granularity), textbook dense over those tokens."""
    T, S, W, G, d = 4096 + 40, 64, 256, 2, 64
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(T, d))
    V = rng.normal(size=(T, d))
    sel = oracle.select_unit(q, K, T, "mean", S, 0, W)
    t0 = sel.ids[0] * S
    assert t0 <= T - W and sel.ids[-1] == -(-T // S) - 1
    got = oracle.attend_unit(q, K, V, T, sel.ids, S)
    want = dense_attention(q, K[t0:T], V[t0:T], 1 / math.sqrt(d))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_attention_closed_form_two_tokens():
    """q = (1, 0), k_0 = (1, 0), k_1 = 0, v_0 = e_0, v_1 = e_1, scale s:
    out = (e^s, 1) / (e^s + 1)."""
    q = np.array([[1.0, 0.0]])
    K = np.array([[1.0, 0.0], [0.0, 0.0]])
    V = np.array([[1.0, 0.0], [0.0, 1.0]])
    for s in (0.5, 2.0, 30.0):
        got = oracle.attend_unit(q, K, V, 2, np.array([0], np.int32), 2, scale=s)
        e = math.exp(s)
        assert np.allclose(got[0], [e / (e + 1), 1 / (e + 1)], rtol=1e-15, atol=0)


def test_attention_output_in_hull_of_attended_values():
    T, S, G, d = 2048, 64, 4, 64
    q = rng.normal(size=(G, d)) * 3
    K = rng.normal(size=(T, d))
    V = rng.normal(size=(T, d))
    ids = np.array([1, 5, 9, 31], np.int32)
    out = oracle.attend_unit(q, K, V, T, ids, S)
    toks = np.concatenate([np.arange(b * S, b * S + S) for b in ids])
    assert np.all(out >= V[toks].min(axis=0) - 1e-12)
    assert np.all(out <= V[toks].max(axis=0) + 1e-12)
    # unselected values cannot leak: changing them changes nothing
    V2 = V.copy()
    mask = np.ones(T, bool)
    mask[toks] = False
    V2[mask] += 100.0
    assert np.array_equal(oracle.attend_unit(q, K, V2, T, ids, S), out)


def test_attention_masks_tokens_past_T_and_empty_set():
    T, S, G, d = 100, 64, 1, 8
    q = rng.normal(size=(G, d))
    K = rng.normal(size=(128, d))
    V = rng.normal(size=(128, d))
    got = oracle.attend_unit(q, K, V, T, np.array([1], np.int32), S)
    want = dense_attention(q, K[64:100], V[64:100], 1 / math.sqrt(d))
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)
    assert np.array_equal(oracle.attend_unit(q, K, V, T, np.zeros(0, np.int32), S),
                          np.zeros((G, d)))
    assert np.array_equal(oracle.attend_unit(q, K, V, 0, np.array([0], np.int32), S),
                          np.zeros((G, d)))


def test_paged_gather_is_permutation_invariant():
    """Reading a unit through any physical page permutation gives the same rows."""
    w = CONFIGS[5].scaled(batch=2, hkv=2, hq=8, T=1000)
    kp, _ = w.pools()
    pt = w.page_table()
    ident = w.scaled(random_pages=False)
    kp2, _ = ident.pools()
    for b in range(2):
        for g in range(2):
            a = oracle.gather_unit(kp, oracle.BF16, pt, b, g, 1000)
            c = oracle.gather_unit(kp2, oracle.BF16, ident.page_table(), b, g, 1000)
            assert np.array_equal(a, c)
            assert np.array_equal(a, synth.widen(w.k_unit(0, b, g), "bf16"))


def test_shared_selection_across_layers():
    """Shared mode: selection from layer 0 only; each layer attends over the
    same ids with its own q, K, V (equal to attending that layer with the
    layer-0 ids), and a layer's own selection would differ in general."""
    w = CONFIGS[5].scaled(batch=1, hkv=1, hq=4, T=4096, layers=3, top_k=6)
    K0 = synth.widen(w.k_unit(0, 0, 0), "bf16")
    q0 = synth.widen(w.q(0), "bf16")[0]
    sel = oracle.select_unit(q0, K0, w.T, "mean", w.S, w.top_k, w.window)
    own = []
    for layer in range(3):
        Kl = synth.widen(w.k_unit(layer, 0, 0), "bf16")
        Vl = synth.widen(w.v_unit(layer, 0, 0), "bf16")
        ql = synth.widen(w.q(layer), "bf16")[0]
        out = oracle.attend_unit(ql, Kl, Vl, w.T, sel.ids, w.S)
        toks = np.concatenate([np.arange(b * w.S, b * w.S + w.S) for b in sel.ids])
        want = dense_attention(ql, Kl[toks], Vl[toks], 1 / math.sqrt(w.d))
        assert np.allclose(out, want, rtol=1e-12, atol=1e-13)
        own.append(oracle.select_unit(ql, Kl, w.T, "mean", w.S, w.top_k, w.window).ids.tolist())
    assert own[1] != sel.ids.tolist() or own[2] != sel.ids.tolist()


# ------------------------------------------------ LRU cache of selected blocks
from oracle.block_cache import cache_step  # noqa: E402


def test_block_cache_hand_worked_example():
    """Capacity 4, steps 0-3, worked by hand from the rule (empty slots first,
    then least recently used; ties by slot index)."""
    blk, st = [-1] * 4, [-1] * 4
    # step 0: {5, 9} -> slots 0, 1 (empty, lowest index first); all new
    blk, st, slot_of, miss, h, m, d = cache_step(blk, st, [5, 9], 0)
    assert (blk, st, slot_of, miss, h, m, d) == ([5, 9, -1, -1], [0, 0, -1, -1], [0, 1], [5, 9],
                                                 0, 2, 2)
    # step 1: {2, 9, 11} -> 9 hits (stamp 0 == step - 1), 2 and 11 take the empty 2, 3
    blk, st, slot_of, miss, h, m, d = cache_step(blk, st, [2, 9, 11], 1)
    assert (blk, st, slot_of, miss, h, m, d) == ([5, 9, 2, 11], [0, 1, 1, 1], [2, 1, 3], [2, 11],
                                                 1, 2, 2)
    # step 2: {3, 11} -> 11 hits; 3 evicts block 5 (stamp 0, the oldest)
    blk, st, slot_of, miss, h, m, d = cache_step(blk, st, [3, 11], 2)
    assert (blk, st, slot_of, miss, h, m, d) == ([3, 9, 2, 11], [2, 1, 1, 2], [0, 3], [3],
                                                 1, 1, 1)
    # step 3: {1, 4, 9} -> 9 hits (stamp 1 != 2: new relative to step 2);
    # 1 and 4 take slots 2 (stamp 1) then 0 (stamp 2, tie with 3 broken by index)
    blk, st, slot_of, miss, h, m, d = cache_step(blk, st, [1, 4, 9], 3)
    assert (blk, st, slot_of, miss, h, m, d) == ([4, 9, 1, 11], [3, 3, 3, 2], [2, 0, 1], [1, 4],
                                                 1, 2, 3)


@pytest.mark.parametrize("seed,cap,k,nb", [(1, 8, 4, 20), (2, 12, 6, 40), (3, 64, 16, 100),
                                           (4, 5, 5, 9)])
def test_block_cache_invariants_against_step_history(seed, cap, k, nb):
    """Random drifting selections: after every step the cache holds the whole
    selection once; hits + misses = |S_t|; the step difference equals the set
    difference (when capacity >= 2k); evictions follow LRU against a last-use
    record kept independently from the step history; empty slots go first."""
    rng = np.random.default_rng(seed)
    blk, st = [-1] * cap, [-1] * cap
    last_use = {}
    prev = set()
    cur = set(rng.choice(nb, size=k, replace=False).tolist())
    for t in range(40):
        if t:  # keep most of the previous selection, swap a few blocks
            keep = set(rng.choice(sorted(cur), size=max(0, k - int(rng.integers(0, k // 2 + 2))),
                                  replace=False).tolist())
            pool = [b for b in range(nb) if b not in keep]
            cur = keep | set(rng.choice(pool, size=k - len(keep), replace=False).tolist())
        ids = sorted(cur)
        before = dict((b, s) for s, b in enumerate(blk) if b >= 0)
        empties = sum(1 for b in blk if b < 0)
        nblk, nst, slot_of, miss, h, m, d = cache_step(blk, st, ids, t)
        # the selection is cached, each block once, at the reported slots
        assert sorted(b for b in nblk if b >= 0) == sorted(set(b for b in nblk if b >= 0))
        assert all(nblk[slot_of[j]] == b and nst[slot_of[j]] == t for j, b in enumerate(ids))
        assert h + m == len(ids) and m == len(miss) and miss == sorted(set(ids) - set(before))
        if cap >= 2 * k:
            assert d == len(set(ids) - prev)
        evicted = [b for b in before if b not in nblk]
        if m <= empties:
            assert not evicted
        kept_unused = [b for b in nblk if b >= 0 and b in before and b not in cur]
        for e in evicted:
            for f in kept_unused:
                assert last_use[e] <= last_use[f], (t, e, f)
        for b in ids:
            last_use[b] = t
        prev = set(ids)
        blk, st = nblk, nst


# ------------------------------------ ratio-based k, length schedule, forced set
def test_ratio_k_and_length_schedule_match_the_pages():
    g = json.load(open(os.path.join(GOLD, "pages_structural.json")))
    r = g["ratio_topk"]
    assert oracle.ratio_k(r["n_blocks"], r["ratio"]) == r["value"]
    for T, ratio in g["length_schedule"]["points"]:
        assert oracle.length_ratio(T) == pytest.approx(ratio)
    # below one block's worth the floor of 1 applies; a ratio of 1 keeps every block
    assert oracle.ratio_k(5, 0.1) == 1 and oracle.ratio_k(37, 1.0) == 37
    # the float32 value of the ratio is the one used (0.15 is not exact in binary)
    assert oracle.ratio_k(1000, 0.15) == int(1000 * float(np.float32(0.15)))


def _unit(seed, T=3000, d=64, G=2):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((G, d)), rng.standard_normal((T, d)), T


@pytest.mark.parametrize("kind,two", [("mean", False), ("minmax", False), ("mean", True)])
def test_forced_blocks_are_a_union(kind, two):
    q, K, T = _unit(11)
    S, nb = 32, -(-3000 // 32)
    kw = dict(coarse_S=256, top_k_coarse=3) if two else {}
    plain = oracle.select_unit(q, K, T, kind, S, 7, 100, **kw)
    forced = np.array([-1, 0, 5, 5, nb - 1, nb, 10 ** 6, 40], np.int32)
    got = oracle.select_unit(q, K, T, kind, S, 7, 100, forced=forced, **kw)
    valid = {0, 5, nb - 1, 40}
    assert set(got.ids.tolist()) == set(plain.ids.tolist()) | valid
    assert got.ids.tolist() == sorted(set(got.ids.tolist()))
    # nothing selected but the forced set: exactly its valid distinct ids
    only = oracle.select_unit(q, K, T, kind, S, 0, 0, forced=forced, **kw)
    assert only.ids.tolist() == sorted(valid)
    # forcing every block selects every block
    allb = oracle.select_unit(q, K, T, kind, S, 3, 0, forced=np.arange(nb), **kw)
    assert allb.ids.tolist() == list(range(nb))


def test_ratio_selection_keeps_ratio_k_blocks():
    q, K, T = _unit(12)
    S, nb = 32, -(-3000 // 32)
    for ratio in (0.05, 0.1, 0.3):
        k = oracle.ratio_k(nb, ratio)
        got = oracle.select_unit(q, K, T, "minmax", S, 999, 0, top_k_ratio=ratio)
        assert len(got.ids) == k
        ref = oracle.select_unit(q, K, T, "minmax", S, k, 0)
        assert got.ids.tolist() == ref.ids.tolist()


def test_whole_coarse_block_loading_closed_form():
    """Two levels with top_k at least the number of fine candidates ("8x256K
    ... porting HiSparse to QSA", section 2.2, when the fine level keeps every
    slice): the selection is every fine block inside the kept coarse blocks,
    plus the window."""
    q, K, T = _unit(13, T=5000)
    S, C, kc, W = 64, 512, 3, 200
    R = C // S
    nb = -(-T // S)
    sel = oracle.select_unit(q, K, T, "mean", S, kc * R, W, coarse_S=C, top_k_coarse=kc)
    expect = {g * R + r for g in sel.coarse_ids.tolist() for r in range(R) if g * R + r < nb}
    expect |= set(oracle.window_blocks(T, S, W).tolist())
    assert sel.ids.tolist() == sorted(expect)


# ------------------------------------------- token-level second stage (SparDA 2.3)
def test_token_stage_against_dense_brute_force():
    """Scores from one dense product over every token (a different route than
    the per-candidate dot products), candidates masked, ranked by lexsort."""
    q, K, T = _unit(21, T=700, d=32, G=4)
    S = 16
    blocks = [0, 3, 7, 20, 43]  # 43 holds the partial last block (688..699)
    dense = (K[:T] @ q.T).sum(axis=1)  # [T]: sum over heads
    cand = np.array([t for b in blocks for t in range(b * S, min(b * S + S, T))])
    s32 = dense[cand].astype(np.float32)
    for k in (1, 10, 50, len(cand), len(cand) + 5):
        order = cand[np.lexsort((cand, -s32.astype(np.float64)))][:k]
        ids, sc, kth = oracle.select_tokens_unit(q, K, T, blocks, S, k, 0)
        assert ids.tolist() == sorted(order.tolist()), k
        assert np.allclose(sc[cand], s32, rtol=1e-6)
        assert np.all(np.isnan(np.delete(sc, cand)))


def test_token_stage_window_ties_and_full_set():
    q, K, T = _unit(22, T=500, d=32, G=2)
    S = 32
    K = K.copy()
    qs = q.sum(axis=0)
    K[45] = K[41] = K[40] = 10.0 * qs / np.linalg.norm(qs)  # planted exact ties, the best
    blocks = [1, 5, 15]  # 15 holds tokens 480..499 (the window's)
    for k, expect in ((1, [40]), (2, [40, 41]), (3, [40, 41, 45])):
        ids, _, _ = oracle.select_tokens_unit(q, K, T, blocks, S, k, 0)
        assert ids.tolist() == expect
    # every token of the window is kept, on top of the top-k, candidate or not
    ids, _, _ = oracle.select_tokens_unit(q, K, T, blocks, S, 3, 30)
    assert ids.tolist() == [40, 41, 45] + list(range(470, 500))
    # k >= candidates: every candidate token, and attention over them equals the
    # block-level attention over the same blocks
    ids, _, _ = oracle.select_tokens_unit(q, K, T, blocks, S, 10 ** 6, 0)
    assert ids.tolist() == [t for b in blocks for t in range(b * S, min(b * S + S, T))]
    V = np.random.default_rng(5).standard_normal(K.shape)
    a = oracle.attend_unit(q, K, V, T, ids, 1)
    b = oracle.attend_unit(q, K, V, T, np.array(blocks, np.int32), S)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
