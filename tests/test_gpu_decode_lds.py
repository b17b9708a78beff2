"""The separate decode launch with a split task's run of the list beyond the
default 64 KiB of LDS ("8x256K long-context sparse attention: porting
HiSparse to QSA", section 3.3: attention over a compact index list; "SparDA"
article, section 2.3: lists of single tokens). 512 units take one split task
each, so a unit's whole token list (up to 9,508 entries of 8-byte row offsets,
about 76 KB) is one task's run; the launch raises the kernel's LDS limit.
Each list holds every token of its sequence in ascending order, salted with
invalid entries; sampled units are checked against the oracle's attention
over the valid tokens, and a list one entry too long for the LDS budget is
refused before any launch."""
import numpy as np
import pytest
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
from gpu_helpers import Problem, check_rows, log, unit_inputs
from synth.workloads import CONFIGS

pytestmark = pytest.mark.gpu


def test_token_list_runs_beyond_64k_of_lds():
    lens = tuple(9500 if b % 2 == 0 else 7000 for b in range(16))
    w = CONFIGS[2].scaled(batch=16, hq=32, hkv=32, d=64, T=9500, seq_lens=lens, needles=0)
    cap = w.T + 8
    assert w.batch * w.hkv == 512 and 8 * cap > 64 << 10  # one split task per unit
    log("decode LDS run: %d units, %d-entry lists (%d KiB of row offsets per task)" % (
        w.batch * w.hkv, cap, 8 * cap // 1024))
    P = Problem.make(w)
    q = P.q()
    lists = np.full((w.batch, w.hkv, cap), -1, np.int32)
    cnts = np.zeros((w.batch, w.hkv), np.int32)
    for b in range(w.batch):
        T = lens[b]
        lst = np.concatenate([np.array([-1], np.int32), np.arange(T, dtype=np.int32),
                              np.array([T, T + 5, 2 ** 30], np.int32)])
        lists[b, :, :len(lst)] = lst
        cnts[b, :] = len(lst)
    tok = torch.from_numpy(lists).cuda()
    tc = torch.from_numpy(cnts).cuda()
    out = P.decode(q, tok, tc, block_size=1)
    torch.cuda.synchronize()
    o = out.cpu().double().numpy()
    for b, g in ((0, 0), (1, 5), (6, 31), (15, 17)):
        T = lens[b]
        qo, K, V = unit_inputs(w, 0, b, g)
        ref = oracle.attend_unit(qo, K, V, T, np.arange(T, dtype=np.int32), 1)
        check_rows(w, o[b, g * w.G:(g + 1) * w.G], ref, "decode LDS run (%d,%d)" % (b, g))
    # the largest run the budget takes (96 KiB of 8-byte offsets) and one more
    kv = P.kvs[0]
    assert hs.hs_decode_workspace_size(kv, w.hq, 1, 12288) > 0
    with pytest.raises(hs.HsError):
        hs.hs_decode_workspace_size(kv, w.hq, 1, 12289)
