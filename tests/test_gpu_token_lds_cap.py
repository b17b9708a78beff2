"""The token stage's general path (more than 8192 candidate slots) at the
largest cache capacity its LDS budget accepts ("SparDA" article, section 2.3:
the token pass inside the chosen blocks). Above the register path the kept
tokens are marked in an LDS bitmap of max_seq_len bits next to the staged id
list, together at most HS_TOKEN_LDS_BYTES; the cache here is declared with
the largest max_seq_len that fits (one token more is refused: see
test_capi_host), its sequences are short, so the oracle's cost follows them,
and the token sets must match the oracle under the near-tie rule."""
import re
import os

import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
from gpu_helpers import Problem, check_tokens, log, unit_inputs
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "hs_attn.h")


def token_lds_bytes():
    m = re.search(r"#define HS_TOKEN_LDS_BYTES \((\d+) << (\d+)\)", open(HEADER).read())
    return int(m.group(1)) << int(m.group(2))


def largest_capacity(max_tokens):
    """Largest max_seq_len whose bitmap words and staged list (max_tokens + 64
    entries) fit the budget."""
    return 32 * (token_lds_bytes() // 4 - max_tokens - 64)


def test_general_path_at_the_lds_cap():
    w = CONFIGS[3].scaled(batch=1, hq=8, hkv=2, T=10000, needles=0)
    kt, wt, ms = 512, 64, 300  # 300 blocks of 32 tokens: 9600 slots, the general path
    max_tok = min(ms * w.S, kt) + wt
    cap = largest_capacity(max_tok)
    log("token stage at max_seq_len %d (bitmap %d KiB)" % (cap, cap // 8 // 1024))
    P = Problem.make(w)
    pages = -(-cap // w.page_size)
    pt = torch.full((w.batch, pages), -1, dtype=torch.int32, device="cuda")
    pt[:, :P.page_table.shape[1]] = P.page_table
    kv = hs.KVCache(P.kvs[0].k_pool, P.kvs[0].v_pool, pt, P.seq_lens, cap)
    rng = np.random.default_rng(7)
    nb = -(-w.T // w.S)
    blocks = np.stack([np.sort(rng.choice(nb, size=ms, replace=False)) for _ in range(w.hkv)])
    ids = torch.from_numpy(blocks.astype(np.int32)[None]).cuda()
    cnt = torch.full((w.batch, w.hkv), ms, dtype=torch.int32, device="cuda")
    q = P.q()
    tok = torch.full((w.batch, w.hkv, max_tok), -7, dtype=torch.int32, device="cuda")
    tcnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
    ws = hs.workspace(hs.hs_select_tokens_workspace_size(kv, w.hq, w.S, ms, kt, wt, max_tok),
                      "cuda")
    for _ in range(2):  # the second call reuses the workspace
        hs.hs_select_tokens(kv, q, w.S, ids, cnt, kt, wt, tok, tcnt, ws)
    torch.cuda.synchronize()
    t_ids, t_cnt = tok.cpu().numpy(), tcnt.cpu().numpy()
    T = int(w.seq_lens_array()[0])
    ties = 0
    for g in range(w.hkv):
        qo, K, _ = unit_inputs(w, 0, 0, g)
        ref, scores, kth = oracle.select_tokens_unit(qo, K, T, blocks[g], w.S, kt, wt)
        ties += check_tokens(t_ids[0, g, :t_cnt[0, g]], ref, scores, kth, qo, K, T, wt,
                             "lds-cap unit (0,%d)" % g)
    log("lds cap: token counts %s, %d tolerated near-tie differences" % (
        t_cnt.reshape(-1).tolist(), ties))
