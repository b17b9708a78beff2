"""GPU parity with planted exact score ties: the lowest-index tie-break on
every top-k path, bit-exact against the oracle, with no near-tie allowance.

Ties are made by copying the key rows of one block (or token) over other
blocks (tokens) of the same unit. Identical rows give bit-identical summary
rows and so bit-identical fp32 scores, on the GPU and in the oracle alike.
The copies are placed so that the group of equal scores straddles the k-th
place. Among equal scores the block (token) of lowest index is kept first:
boundary comparisons are exact fp32 comparisons ("8x256K ... porting
HiSparse to QSA", section 5.1), and equal scores go to the lower index.
Before any GPU call, each case checks on the CPU that its group really
straddles the boundary and that no other candidate lies within 1e-5 of the
tied score. Then the exact boundary decides the result on both sides.

Paths covered (select_impl.h):
  * single level, at most 4096 candidates (register path, contiguous
    ownership): a tie group of at most 128 that is ranked directly; a group
    of more than 128 equal keys (all-equal branch); every block identical
    (the key range is one value);
  * single level, more than 4096 candidates: general path with keys in LDS
    (at most 8192) and in the workspace (more), including every block
    identical;
  * two levels: ties at the coarse level (whole coarse blocks copied), more
    than 128 equal fine blocks in the fine level's register path, and the
    general path of a fine level with more than 4096 candidate slots;
  * token level: register path (a group ranked directly and an all-equal
    group) and general path.
Every block case runs through hs_select_blocks, hs_select_decode and
hs_decode_step, and the outputs are checked against the oracle's attention
over the oracle's ids.
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
import synth
from gpu_helpers import Problem, check_ids, check_rows, log, magnitudes
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

C = CONFIGS
SEP_RTOL = 1e-5  # other candidates must differ from the tied score by more than this


def block_scores(q, K, T, S, kind):
    """Oracle scores (float64) of every block of size S."""
    a, b = oracle.summarize(K[:T], S, kind)
    return oracle.scores_mean(q, a) if kind == "mean" else oracle.scores_minmax(q, a, b)


def rank_order(s):
    """Block indices by (score rounded to fp32 descending, index ascending)."""
    s32 = s.astype(np.float32).astype(np.float64)
    return sorted(range(len(s)), key=lambda i: (-s32[i], i))


def window_mask(T, S, W, n):
    win = np.zeros(n, bool)
    win[oracle.window_blocks(T, S, W)] = True
    return win


class Planted:
    """Key rows of layer 0 with edits planted per unit; V and other layers
    come from the generator unchanged."""

    def __init__(self, w, plant_unit):
        self.w = w
        self.k = {}
        for b in range(w.batch):
            kb = np.ascontiguousarray(w.kv_rows("k", 0, b))
            for g in range(w.hkv):
                qo = synth.widen(w.q(), w.dtype)[b, g * w.G:(g + 1) * w.G]
                plant_unit(b, g, qo, kb[g])
            self.k[b] = kb

    def rows_of(self, which, layer, b):
        if which == "k" and layer == 0:
            return self.k[b]
        return self.w.kv_rows(which, layer, b)


def copy_blocks(rows, L, src, dsts):
    """Rows of block src (L tokens) copied over blocks dsts (exact bits)."""
    for d in dsts:
        rows[d * L:(d + 1) * L] = rows[src * L:(src + 1) * L]


def group_copies(w, qo, rows, S, kind, T, W, rank, m, rng):
    """Copies the block of rank `rank` (non-window blocks, oracle order)
    over m blocks ranked below it; returns the group (src and copies)."""
    K = synth.widen(rows, w.dtype)
    s = block_scores(qo, K, T, S, kind)
    win = window_mask(T, S, W, len(s))
    order = [i for i in rank_order(s) if not win[i] and (i + 1) * S <= T]
    src = order[rank]
    below = np.array(order[rank + 1:])
    dsts = rng.choice(below, size=m, replace=False)
    copy_blocks(rows, S, src, dsts)
    return {int(src)} | {int(x) for x in dsts}


def assert_clean_boundary(s, group, kept, mags, what):
    """The tie group straddles the boundary (some, not all, of it kept) and
    every candidate outside it is well away from the tied score."""
    s32 = s.astype(np.float32).astype(np.float64)
    vals = {s32[i] for i in group}
    assert len(vals) == 1, "%s: planted group is not one score: %s" % (what, sorted(vals)[:4])
    tie = vals.pop()
    n_kept = len(set(kept) & group)
    assert 0 < n_kept < len(group), "%s: group of %d, %d kept: not straddling" % (
        what, len(group), n_kept)
    for i in range(len(s)):
        if i in group or np.isnan(s[i]):
            continue
        tol = SEP_RTOL * max(abs(tie), mags[i])
        assert abs(s32[i] - tie) > tol, "%s: block %d within %.3g of the tied score" % (
            what, i, tol)
    return n_kept


def assert_no_near_ties(s, kth, mags, what):
    """No candidate other than those equal to the k-th score lies near it
    (so that the fine boundary of a two-level case is exact on both sides)."""
    s32 = s.astype(np.float32).astype(np.float64)
    for i in range(len(s)):
        if np.isnan(s[i]) or s32[i] == kth:
            continue
        tol = SEP_RTOL * max(abs(kth), mags[i])
        assert abs(s32[i] - kth) > tol, "%s: candidate %d within %.3g of the k-th score" % (
            what, i, tol)


# ------------------------------------------------------------ block cases
# name: (workload, planting, arguments)
BLOCK_CASES = {
    "regs-rank": (C[3].scaled(batch=1, hq=8, hkv=2, T=16384, top_k=64, needles=0),
                  "group", dict(rank=30, m=60)),
    "regs-allequal": (C[3].scaled(batch=1, hq=8, hkv=2, T=16384, top_k=200, needles=0),
                      "group", dict(rank=50, m=300)),
    "regs-identical": (C[2].scaled(batch=1, hq=2, hkv=2, T=8192, top_k=40, needles=0),
                       "identical", {}),
    "general-lds": (C[3].scaled(batch=1, hq=4, hkv=1, d=64, T=20000, kind="mean", S=4,
                                page_size=16, top_k=100, window=64, needles=0),
                    "group", dict(rank=40, m=300)),
    "general-ws": (C[3].scaled(batch=1, hq=4, hkv=1, d=64, T=20000, kind="mean", S=2,
                               page_size=16, top_k=100, window=64, needles=0),
                   "group", dict(rank=40, m=300)),
    "general-ws-identical": (C[3].scaled(batch=1, hq=4, hkv=1, d=64, T=20000, kind="mean",
                                         S=2, page_size=16, top_k=100, window=64, needles=0),
                             "identical", {}),
    "two-level-coarse": (C[4].scaled(batch=1, hq=2, hkv=2, T=32768, coarse_S=256,
                                     top_k_coarse=20, top_k=60, window=256, needles=0),
                         "coarse", dict(rank=8, m=25)),
    "two-level-fine-allequal": (C[4].scaled(batch=1, hq=2, hkv=2, T=65536, coarse_S=512,
                                            top_k_coarse=50, top_k=200, window=256,
                                            needles=0),
                                "fine-tiles", dict(m=40)),
    "two-level-general": (C[4].scaled(batch=1, hq=1, hkv=1, d=64, T=131072, coarse_S=512,
                                      S=16, page_size=16, top_k_coarse=130, top_k=300,
                                      window=256, needles=0),
                          "coarse", dict(rank=10, m=150)),
}
_PROB = {}


def plant_fn(w, how, args, groups):
    """The per-unit planting of a case; records each unit's tie group."""
    rng = np.random.default_rng(7)

    def plant(b, g, qo, rows):
        T = int(w.seq_lens_array()[b])
        if how == "group":
            groups[(b, g)] = group_copies(w, qo, rows, w.S, w.kind, T, w.window, args["rank"],
                                          args["m"], rng)
        elif how == "identical":
            nb = T // w.S
            src = rows[:w.S].copy()
            rows[:nb * w.S] = np.tile(src, (nb, 1))
            groups[(b, g)] = set(range(nb))
        elif how == "coarse":
            # whole coarse blocks copied: a tie group at the coarse level
            groups[(b, g)] = group_copies(w, qo, rows, w.coarse_S, "mean", T, w.window,
                                          args["rank"], args["m"], rng)
        elif how == "fine-tiles":
            # m coarse blocks made of copies of the top fine block: more than
            # 128 equal fine blocks, all inside the kept coarse blocks
            K = synth.widen(rows, w.dtype)
            s = block_scores(qo, K, T, w.S, w.kind)
            R = w.coarse_S // w.S
            nc_full = (T - w.window) // w.coarse_S  # coarse blocks before the window
            src = rank_order(s[:nc_full * R])[0]
            tile = np.tile(rows[src * w.S:(src + 1) * w.S], (R, 1))
            others = [c for c in range(nc_full) if c != src // R]
            cs = [src // R] + [int(c) for c in rng.choice(others, size=args["m"] - 1,
                                                           replace=False)]
            group = set()
            for c in cs:  # the source's own coarse block is tiled too
                rows[c * w.coarse_S:(c + 1) * w.coarse_S] = tile
                group |= set(range(c * R, (c + 1) * R))
            groups[(b, g)] = group
        else:
            raise ValueError(how)

    return plant


def block_problem(name):
    if name not in _PROB:
        w, how, args = BLOCK_CASES[name]
        log("setting up ties case %s" % name)
        groups = {}
        planted = Planted(w, plant_fn(w, how, args, groups))
        P = Problem.make(w, rows_of=planted.rows_of)
        ref = {}
        lens = w.seq_lens_array()
        for b in range(w.batch):
            for g in range(w.hkv):
                T = int(lens[b])
                qo, K, V = P.unit_inputs(0, b, g)
                sel = oracle.select_unit(qo, K, T, w.kind, w.S, w.top_k, w.window,
                                         coarse_S=w.coarse_S, top_k_coarse=w.top_k_coarse)
                what = "%s (%d,%d)" % (name, b, g)
                mags = magnitudes(w, qo, K, T)
                grp = groups[(b, g)]
                if how == "coarse":
                    mu = oracle.summary_mean(K[:T], w.coarse_S)
                    cs = oracle.scores_mean(qo, mu)
                    cmag = np.abs(mu) @ np.abs(qo).sum(axis=0)
                    n = assert_clean_boundary(cs, grp, sel.coarse_ids.tolist(), cmag,
                                              what + " coarse")
                    assert_no_near_ties(sel.fine_scores, sel.kth_score, mags, what + " fine")
                    log("%s: coarse group %d, %d kept" % (what, len(grp), n))
                else:
                    n = assert_clean_boundary(sel.fine_scores, grp, sel.fine_top.tolist(), mags,
                                              what)
                    log("%s: group %d, %d kept by the top-%d" % (what, len(grp), n, w.top_k))
                    if w.top_k_coarse:  # the coarse boundary must be exact too
                        mu = oracle.summary_mean(K[:T], w.coarse_S)
                        cs = oracle.scores_mean(qo, mu)
                        cmag = np.abs(mu) @ np.abs(qo).sum(axis=0)
                        kc = sel.coarse_ids.tolist()
                        if len(kc) < len(cs):
                            assert_no_near_ties(cs, float(np.float32(cs[kc[-1]])), cmag,
                                                what + " coarse")
                ref[(b, g)] = (sel.ids, oracle.attend_unit(qo, K, V, T, sel.ids, w.S))
        _PROB[name] = (P, ref)
    return _PROB[name]


def check_exact(w, ref, ids_t, cnt_t, out_t, what):
    ids, cnt = ids_t.cpu().numpy(), cnt_t.cpu().numpy()
    out = out_t.cpu().double().numpy()
    for (b, g), (rid, rout) in ref.items():
        got = ids[b, g, :cnt[b, g]].tolist()
        assert got == rid.tolist(), "%s (%d,%d): ids differ from the oracle:\n gpu %s\n ref %s" % (
            what, b, g, sorted(set(got) ^ set(rid.tolist()))[:12], len(rid))
        check_rows(w, out[b, g * w.G:(g + 1) * w.G], rout, "%s (%d,%d)" % (what, b, g))


@pytest.mark.parametrize("name", list(BLOCK_CASES))
def test_planted_ties_blocks(name):
    P, ref = block_problem(name)
    w = P.w
    q = P.q()
    summ = P.summaries()
    ids, cnt = P.select(q, summ)
    out = P.decode(q, ids, cnt)
    torch.cuda.synchronize()
    check_exact(w, ref, ids, cnt, out, name + " separate")
    ids2, cnt2, out2, _ = P.select_decode(q, summ)
    torch.cuda.synchronize()
    check_exact(w, ref, ids2, cnt2, out2, name + " select_decode")
    ids3, cnt3, out3, _ = P.decode_step(q, summ, w.nb - 1)
    torch.cuda.synchronize()
    check_exact(w, ref, ids3, cnt3, out3, name + " decode_step")
    log("%s: ids equal to the oracle through all three entry points" % name)


# ------------------------------------------------------------ token cases
# name: (workload, block top_k, token top_k, token window, copy stride)
TOKEN_CASES = {
    "tokens-regs-rank": (C[3].scaled(batch=1, hq=8, hkv=2, T=8192, needles=0), 100, 30, 16, 80),
    "tokens-regs-allequal": (C[3].scaled(batch=1, hq=8, hkv=2, T=8192, needles=0), 100, 150,
                             16, 16),
    "tokens-regs-wide": (C[3].scaled(batch=1, hq=8, hkv=2, T=16384, needles=0), 200, 300, 16,
                         16),
    "tokens-general": (C[3].scaled(batch=1, hq=8, hkv=2, T=32768, needles=0), 300, 400, 16, 16),
}


def token_plant(w, stride, groups):
    def plant(b, g, qo, rows):
        T = int(w.seq_lens_array()[b])
        K = synth.widen(rows, w.dtype)
        lim = T - w.window  # copies stay out of the block window
        sc = K[:lim] @ qo.sum(axis=0)
        src = int(np.argmax(sc))
        dst = [t for t in range(0, lim, stride) if t != src]
        copy_blocks(rows, 1, src, dst)
        groups[(b, g)] = {src} | set(dst)

    return plant


@pytest.mark.parametrize("name", list(TOKEN_CASES))
def test_planted_ties_tokens(name):
    w, kb, kt, wt, stride = TOKEN_CASES[name]
    log("setting up ties case %s" % name)
    groups = {}
    planted = Planted(w, token_plant(w, stride, groups))
    P = Problem.make(w, rows_of=planted.rows_of)
    kv = P.kvs[0]
    q = P.q()
    summ = P.summaries()
    ids, cnt = P.select(q, summ, top_k=kb)
    ms = ids.shape[-1]
    regs = ms * w.S <= 8192 and ms <= 512  # the library's token register path
    assert regs == ("regs" in name), (name, ms, w.S)
    max_tok = min(ms * w.S, kt) + min(wt, w.T)
    tok = torch.full((w.batch, w.hkv, max_tok), -7, dtype=torch.int32, device="cuda")
    tcnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
    n = hs.hs_select_tokens_workspace_size(kv, w.hq, w.S, ms, kt, wt, max_tok)
    ws = hs.workspace(n, "cuda")
    hs.hs_select_tokens(kv, q, w.S, ids, cnt, kt, wt, tok, tcnt, ws)
    out = P.decode(q, tok, tcnt, block_size=1)
    torch.cuda.synchronize()
    b_ids, b_cnt = ids.cpu().numpy(), cnt.cpu().numpy()
    t_ids, t_cnt = tok.cpu().numpy(), tcnt.cpu().numpy()
    o = out.cpu().double().numpy()
    lens = w.seq_lens_array()
    for b in range(w.batch):
        for g in range(w.hkv):
            T = int(lens[b])
            qo, K, V = P.unit_inputs(0, b, g)
            what = "%s (%d,%d)" % (name, b, g)
            sel = oracle.select_unit(qo, K, T, w.kind, w.S, kb, w.window)
            check_ids(w, b_ids[b, g, :b_cnt[b, g]], sel, magnitudes(w, qo, K, T), T, what=what)
            blocks = b_ids[b, g, :b_cnt[b, g]]
            ref, scores, kth = oracle.select_tokens_unit(qo, K, T, blocks, w.S, kt, wt)
            cand = ~np.isnan(scores)
            grp = {t for t in groups[(b, g)] if cand[t]}
            kept_top = [t for t in ref.tolist() if t < T - wt]
            mag = np.abs(K[:T]) @ np.abs(qo).sum(axis=0)
            n_kept = assert_clean_boundary(scores, grp, kept_top, mag, what)
            got = t_ids[b, g, :t_cnt[b, g]].tolist()
            assert got == ref.tolist(), "%s: tokens differ from the oracle: %s" % (
                what, sorted(set(got) ^ set(ref.tolist()))[:12])
            check_rows(w, o[b, g * w.G:(g + 1) * w.G], oracle.attend_unit(qo, K, V, T, ref, 1),
                       what)
            log("%s: %d candidates, tie group %d, %d kept by the top-%d" % (
                what, int(cand.sum()), len(grp), n_kept, kt))
