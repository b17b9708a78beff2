"""GPU parity of the token-level second stage ("SparDA" section 2.3).

The block selection is the GPU's own (hs_select_blocks, tested elsewhere);
given those blocks, hs_select_tokens keeps the top tokens inside them plus the
window's tokens, and hs_sparse_decode with block size 1 attends over exactly
those tokens. The oracle recomputes both from the same blocks. Token sets are
bit-exact except for near ties: a token may differ only if its oracle score
lies within 1e-6 * max(|s_k|, sum_j sum_i |q_j,i k_t,i|) of the k-th kept
score s_k, and never inside the window. Every top-k path of the token level is
covered: the register path (at most 8192 candidate slots and 512 selected
blocks; blocks of 32 tokens or more, and smaller blocks, several per thread),
the general path with keys in LDS (at most 8192 slots but more blocks) and
with keys in the workspace (more slots), and both forms of the general path's
id emission (compacted non-zero bitmap words, and the full scan of a dense
bitmap).
"""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
from gpu_helpers import Problem, check_rows, check_tokens, log, unit_inputs
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

C = CONFIGS
CASES = {
    # name: (workload, block top_k, token top_k, token window)
    "regs": (C[3].scaled(batch=2, hq=8, hkv=2, T=8209, seq_lens=(8209, 5000), top_k=100),
             100, 256, 48),
    "regs-wide": (C[3].scaled(batch=2, hq=8, hkv=2, T=8209, seq_lens=(8209, 5000),
                              top_k=200), 200, 300, 0),
    "regs-s16": (C[3].scaled(batch=2, hq=8, hkv=2, T=6001, seq_lens=(6001, 3100), S=16,
                             page_size=16, top_k=150), 150, 400, 40),
    # more than 4096 kept tokens below the window: the register path stores
    # them directly instead of through its LDS staging
    "regs-many-kept": (C[3].scaled(batch=2, hq=8, hkv=2, T=8209, seq_lens=(8209, 5000),
                                   top_k=240, window=64), 240, 5000, 64),
    "general-lds": (C[3].scaled(batch=1, hq=8, hkv=2, T=8209, S=8, page_size=8, top_k=600,
                                window=64), 600, 700, 30),
    "general-ws": (C[3].scaled(batch=1, hq=8, hkv=2, T=8209, top_k=257), 257, 128, 64),
    "f32-box": (C[1].scaled(hq=4, hkv=2, d=128, T=2500, kind="minmax", S=32, page_size=32,
                            top_k=7), 7, 40, 20),
    "d64-g8-pages": (C[3].scaled(batch=2, hq=16, hkv=2, d=64, T=3001, kind="mean", S=64,
                                 page_size=16, top_k=5, window=100, needles=0,
                                 random_pages=True, seq_lens=(3001, 1500)), 5, 100, 50),
    "mha-g1": (C[2].scaled(batch=2, hq=4, hkv=4, T=4133, seq_lens=(4133, 2100), top_k=20),
               20, 300, 64),
    # every block selected and a fifth of the 66000 tokens kept: nearly every
    # 32-token word of the token bitmap is non-zero, more than the 512 words a
    # wave compacts before emitting, so the emission scans the bitmap in full
    "dense-scan": (C[3].scaled(batch=1, hq=4, hkv=1, T=66000, top_k=2063), 2063, 13200, 64),
}
_P = {}


# the top-k path each case must take
PATHS = {"regs": "regs", "regs-wide": "regs", "regs-s16": "regs", "regs-many-kept": "regs",
         "general-lds": "general",
         "general-ws": "general", "f32-box": "regs", "d64-g8-pages": "regs", "mha-g1": "regs",
         "dense-scan": "general"}


def token_path(max_selected, S):
    """The library's token top-k path for a list capacity and block size."""
    return "regs" if max_selected * S <= 8192 and max_selected <= 512 else "general"


@pytest.mark.parametrize("name", list(CASES))
def test_token_stage_matches_oracle(name):
    w, kb, kt, wt = CASES[name]
    if name not in _P:
        log("setting up %s" % name)
        _P[name] = Problem.make(w)
    P = _P[name]
    kv = P.kvs[0]
    q = P.q()
    summ = P.summaries()
    ids, cnt = P.select(q, summ, top_k=kb)
    ms = ids.shape[-1]
    assert token_path(ms, w.S) == PATHS[name], (name, ms, w.S)
    max_tok = min(ms * w.S, kt) + min(wt, w.T)
    tok = torch.full((w.batch, w.hkv, max_tok), -7, dtype=torch.int32, device="cuda")
    tcnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
    n = hs.hs_select_tokens_workspace_size(kv, w.hq, w.S, ms, kt, wt, max_tok)
    ws = hs.workspace(n, "cuda")
    for rep in range(2):  # the second call reuses the workspace (counters back at zero)
        hs.hs_select_tokens(kv, q, w.S, ids, cnt, kt, wt, tok, tcnt, ws)
    out = P.decode(q, tok, tcnt, block_size=1)
    torch.cuda.synchronize()
    b_ids, b_cnt = ids.cpu().numpy(), cnt.cpu().numpy()
    t_ids, t_cnt = tok.cpu().numpy(), tcnt.cpu().numpy()
    o = out.cpu().double().numpy()
    lens = w.seq_lens_array()
    ties = 0
    for b in range(w.batch):
        for g in range(w.hkv):
            T = int(lens[b])
            qo, K, V = unit_inputs(w, 0, b, g)
            blocks = b_ids[b, g, :b_cnt[b, g]]
            ref, scores, kth = oracle.select_tokens_unit(qo, K, T, blocks, w.S, kt, wt)
            gi = t_ids[b, g, :t_cnt[b, g]]
            what = "%s unit (%d,%d)" % (name, b, g)
            ties += check_tokens(gi, ref, scores, kth, qo, K, T, wt, what)
            check_rows(w, o[b, g * w.G:(g + 1) * w.G], oracle.attend_unit(qo, K, V, T, gi, 1),
                       what)
    log("%s: token counts %s, %d tolerated near-tie differences" % (
        name, t_cnt.reshape(-1).tolist(), ties))


@pytest.mark.parametrize("name", ["regs", "f32-box", "d64-g8-pages", "mha-g1"])
def test_token_list_attention_skips_invalid_ids(name):
    """hs_sparse_decode with block size 1 over caller-made token lists salted
    with -1, ids at or past T_b and huge ids: the invalid entries are skipped,
    so the output is the attention over the valid tokens alone."""
    w = CASES[name][0]
    if name not in _P:
        _P[name] = Problem.make(w)
    P = _P[name]
    q = P.q()
    lens = w.seq_lens_array()
    rng = np.random.default_rng(31)
    n = 300
    lists = np.full((w.batch, w.hkv, n), -1, np.int32)
    cnts = np.zeros((w.batch, w.hkv), np.int32)
    valid = {}
    for b in range(w.batch):
        T = int(lens[b])
        for g in range(w.hkv):
            good = np.sort(rng.choice(T, size=min(200, T), replace=False)).astype(np.int32)
            bad = np.array([-1, T, T + 7, 2 ** 30], np.int32)
            lst = np.concatenate([good[:50], bad[:2], good[50:], bad[2:]])
            lists[b, g, :len(lst)] = lst
            cnts[b, g] = len(lst)
            valid[(b, g)] = good
    tok = torch.from_numpy(lists).cuda()
    tc = torch.from_numpy(cnts).cuda()
    out = P.decode(q, tok, tc, block_size=1)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    for (b, g), good in valid.items():
        T = int(lens[b])
        qo, K, V = unit_inputs(w, 0, b, g)
        ref = oracle.attend_unit(qo, K, V, T, good, 1)
        check_rows(w, o[b, g * w.G:(g + 1) * w.G], ref, "%s invalid ids (%d,%d)" % (name, b, g))


@pytest.mark.parametrize("name", ["regs", "general-ws"])
def test_token_stage_empty_lists_and_sequences(name):
    """Degenerate inputs of the token stage: a unit with no selected blocks
    keeps only its window's tokens (the window is attended whether scored or
    not), a sequence of length 0 keeps nothing and attends to nothing (output
    row 0), and every other unit is unaffected; the token ids match the
    oracle and the attention over them matches the oracle's."""
    w0, kb, kt, wt = CASES[name]
    lens = (w0.T, 0) if w0.batch == 2 else (w0.T,)
    w = w0.scaled(seq_lens=lens) if w0.batch == 2 else w0
    P = Problem.make(w)
    kv = P.kvs[0]
    q = P.q()
    summ = P.summaries()
    ids, cnt = P.select(q, summ, top_k=kb)
    ms = ids.shape[-1]
    cnt[0, 0] = 0  # unit (0, 0): an empty block list
    max_tok = min(ms * w.S, kt) + min(wt, w.T)
    tok = torch.full((w.batch, w.hkv, max_tok), -7, dtype=torch.int32, device="cuda")
    tcnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
    ws = hs.workspace(hs.hs_select_tokens_workspace_size(kv, w.hq, w.S, ms, kt, wt, max_tok),
                      "cuda")
    hs.hs_select_tokens(kv, q, w.S, ids, cnt, kt, wt, tok, tcnt, ws)
    out = P.decode(q, tok, tcnt, block_size=1)
    torch.cuda.synchronize()
    b_ids, b_cnt = ids.cpu().numpy(), cnt.cpu().numpy()
    t_ids, t_cnt = tok.cpu().numpy(), tcnt.cpu().numpy()
    o = out.cpu().double().numpy()
    seq = w.seq_lens_array()
    for b in range(w.batch):
        for g in range(w.hkv):
            T = int(seq[b])
            qo, K, V = unit_inputs(w, 0, b, g)
            blocks = b_ids[b, g, :b_cnt[b, g]]
            ref, scores, kth = oracle.select_tokens_unit(qo, K, T, blocks, w.S, kt, wt)
            gi = t_ids[b, g, :t_cnt[b, g]]
            what = "%s degenerate unit (%d,%d) T=%d, %d blocks" % (name, b, g, T, len(blocks))
            if (b, g) == (0, 0):
                assert np.array_equal(gi, np.arange(max(0, T - wt), T, dtype=np.int32)), what
            if T == 0:
                assert len(gi) == 0, what
                assert np.all(o[b, g * w.G:(g + 1) * w.G] == 0.0), what
                continue
            check_tokens(gi, ref, scores, kth, qo, K, T, wt, what)
            check_rows(w, o[b, g * w.G:(g + 1) * w.G], oracle.attend_unit(qo, K, V, T, gi, 1),
                       what)
    log("%s degenerate lists: token counts %s" % (name, t_cnt.reshape(-1).tolist()))
