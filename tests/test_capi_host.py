"""CPU tests of the C-ABI library: it loads without a GPU, exports every
symbol include/hs_attn.h declares, and rejects invalid arguments on the host
before any HIP call. No call here reaches a kernel launch: every call either
is a pure host function or fails validation."""
import ctypes
import os
import re

import pytest

import hierarchical_sparse_attention_amd as hs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hs_attn.h")
FAKE = 0x7F0000000000  # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(hs_[a-z_]+)\s*\(", src)))


def test_library_loads_and_exports_every_declared_symbol():
    L = hs.lib()
    names = declared_functions()
    assert set(names) == set(hs.EXPORTS)
    for n in names:
        assert hasattr(L, n), n
    assert hs.hs_version() == 4


def test_step_status_rejects_bad_arguments():
    """hs_step_status validates before any HIP call: null pointers and a
    workspace shorter than the status word."""
    L = hs.lib()
    v = ctypes.c_int32(7)
    assert L.hs_step_status(None, 4096, ctypes.byref(v), None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_step_status(FAKE, 4096, None, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_step_status(FAKE, 3, ctypes.byref(v), None) == hs.HS_ERR_WORKSPACE
    assert v.value == 7


def test_status_strings():
    assert hs.status_string(hs.HS_OK) == "HS_OK"
    assert hs.status_string(hs.HS_ERR_WORKSPACE) == "HS_ERR_WORKSPACE"
    assert hs.status_string(99) == "HS_UNKNOWN_STATUS"


def kv_struct(**over):
    f = dict(k_pool=FAKE, v_pool=FAKE + 4096, page_table=FAKE + 8192, seq_lens=FAKE + 12288,
             batch=4, num_kv_heads=8, head_dim=128, page_size=32, max_pages=4096,
             num_phys_pages=4 * 4096, max_seq_len=131072, dtype=hs.HS_BF16)
    f.update(over)
    return hs.hs_kv_cache(**f)


def summ(kind=hs.HS_SUMMARY_MINMAX, S=32, max_blocks=4096, data=FAKE + 65536):
    return hs.hs_summaries(data, kind, S, max_blocks)


def sel_size(p, kv, fine, coarse=None):
    n = ctypes.c_size_t(0)
    st = hs.lib().hs_select_workspace_size(ctypes.byref(p), ctypes.byref(kv), ctypes.byref(fine),
                                           ctypes.byref(coarse) if coarse else None,
                                           ctypes.byref(n))
    return st, n.value


def test_decode_split_count_follows_the_work_per_split():
    """Split tasks per unit, read off the decode workspace (partials o and
    (m, l) per split): about 256 tasks in all, twice that when a split would
    still hold 2048 or more tokens at the full selection."""
    def dsize(kv, block_size, max_selected):
        n = ctypes.c_size_t(0)
        assert hs.lib().hs_decode_workspace_size(ctypes.byref(kv), 32, block_size, max_selected,
                                                 ctypes.byref(n)) == hs.HS_OK
        return n.value

    per_split = 4 * (128 + 2) * 4  # G = 4 heads of (o[128], m, l) floats
    # 16 x 8 = 128 units: 2 splits hold 111 tokens (block 1), 4 hold 111 blocks of 64
    kv = kv_struct(batch=16, page_size=64, max_pages=1024, num_phys_pages=16 * 1024,
                   max_seq_len=65536)
    assert dsize(kv, 64, 111) - dsize(kv, 1, 111) == 128 * 2 * per_split
    # 32 units at 145 blocks of 32 tokens: 8 splits of about 580 tokens stay 8
    # (doubling would give 16 splits)
    kv = kv_struct()
    assert dsize(kv, 32, 145) - dsize(kv, 1, 145) == 0
    # 256 units: one split of 73 x 64 tokens becomes two
    kv = kv_struct(batch=8, num_kv_heads=32, page_size=64, max_pages=512,
                   num_phys_pages=8 * 512, max_seq_len=32768)
    assert dsize(kv, 64, 73) - dsize(kv, 1, 73) == 256 * 1 * (128 + 2) * 4


def test_decode_rejects_runs_beyond_the_lds_of_a_split_task():
    """A split task of hs_sparse_decode holds its run of the list in LDS, at
    most 96 KiB: 4-byte ids, 8-byte row offsets for token lists (S = 1) of a
    bf16 cache. 32 units take 16 splits at these lengths."""
    def st(kv, block_size, max_selected):
        n = ctypes.c_size_t(0)
        return hs.lib().hs_decode_workspace_size(ctypes.byref(kv), 32, block_size, max_selected,
                                                 ctypes.byref(n))
    kv = kv_struct()
    assert st(kv, 1, 16 * 12288) == hs.HS_OK          # 12288 tokens x 8 B per split
    assert st(kv, 1, 16 * 12288 + 1) == hs.HS_ERR_INVALID_ARG
    assert st(kv, 32, 16 * 24576) == hs.HS_OK         # 24576 ids x 4 B per split
    assert st(kv, 32, 16 * 24576 + 1) == hs.HS_ERR_INVALID_ARG
    kv32 = kv_struct(dtype=hs.HS_F32)
    assert st(kv32, 1, 16 * 24576) == hs.HS_OK        # float32 caches keep the ids
    assert st(kv32, 1, 16 * 24576 + 1) == hs.HS_ERR_INVALID_ARG
    # the entry point refuses it before any launch
    assert hs.lib().hs_sparse_decode(ctypes.byref(kv), FAKE, 32, ctypes.c_float(0.0), 1, FAKE,
                                     FAKE, 16 * 12288 + 1, FAKE, FAKE, 1 << 40, None) == \
        hs.HS_ERR_INVALID_ARG


def test_select_workspace_size_layout():
    p = hs.hs_select_params(32, 128, 512, 0, 145)
    st, n = sel_size(p, kv_struct(), summ())
    assert st == hs.HS_OK
    assert n >= 4 * 8 * 4096 * 4          # one fp32 score per block and unit
    assert n % 256 == 0
    # two-level: coarse scores + kept coarse ids + fine candidate scores
    kv4 = kv_struct(num_kv_heads=32, batch=8, max_pages=4096, page_size=64,
                    num_phys_pages=8 * 4096, max_seq_len=262144)
    p2 = hs.hs_select_params(32, 128, 512, 32, 137)
    st, n2 = sel_size(p2, kv4, summ(hs.HS_SUMMARY_MEAN, 64, 4096),
                      summ(hs.HS_SUMMARY_MEAN, 1024, 256))
    assert st == hs.HS_OK
    units = 8 * 32
    assert n2 >= units * (256 * 4 + 32 * 4 + 4 + 512 * 4)


@pytest.mark.parametrize("change,code", [
    (dict(head_dim=96), hs.HS_ERR_UNSUPPORTED),
    (dict(dtype=7), hs.HS_ERR_UNSUPPORTED),
    (dict(batch=0), hs.HS_ERR_INVALID_ARG),
    (dict(page_table=0), hs.HS_ERR_INVALID_ARG),
    (dict(seq_lens=0), hs.HS_ERR_INVALID_ARG),
    (dict(max_seq_len=4096 * 32 + 1), hs.HS_ERR_INVALID_ARG),
    (dict(page_size=0), hs.HS_ERR_INVALID_ARG),
])
def test_select_rejects_bad_cache(change, code):
    p = hs.hs_select_params(32, 128, 512, 0, 145)
    assert sel_size(p, kv_struct(**change), summ())[0] == code


@pytest.mark.parametrize("params,code", [
    ((30, 128, 512, 0, 145), hs.HS_ERR_INVALID_ARG),   # Hq not a multiple of Hkv
    ((24, 128, 512, 0, 145), hs.HS_ERR_UNSUPPORTED),   # G = 3
    ((32, 128, 512, 0, 144), hs.HS_ERR_INVALID_ARG),   # capacity below k + W/S + 1
    ((32, -1, 512, 0, 145), hs.HS_ERR_INVALID_ARG),
    ((32, 128, -5, 0, 145), hs.HS_ERR_INVALID_ARG),
])
def test_select_rejects_bad_params(params, code):
    assert sel_size(hs.hs_select_params(*params), kv_struct(), summ())[0] == code


def test_select_rejects_bad_summaries():
    p = hs.hs_select_params(32, 128, 512, 0, 145)
    assert sel_size(p, kv_struct(), summ(max_blocks=4095))[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(p, kv_struct(), summ(data=FAKE + 1))[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(p, kv_struct(), summ(kind=5))[0] == hs.HS_ERR_INVALID_ARG
    # two-level needs a coarse table whose block size is a multiple of S
    p2 = hs.hs_select_params(32, 128, 512, 8, 145)
    assert sel_size(p2, kv_struct(), summ())[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(p2, kv_struct(), summ(), summ(hs.HS_SUMMARY_MEAN, 48, 4096))[0] == \
        hs.HS_ERR_INVALID_ARG
    assert sel_size(p2, kv_struct(), summ(), summ(hs.HS_SUMMARY_MEAN, 1024, 128))[0] == hs.HS_OK


def test_entry_points_fail_before_launch():
    L = hs.lib()
    kv = kv_struct()
    p = hs.hs_select_params(32, 128, 512, 0, 145)
    fine = summ()
    st, need = sel_size(p, kv, fine)
    assert st == hs.HS_OK
    # workspace too small / missing -> HS_ERR_WORKSPACE, nothing launched
    assert L.hs_select_blocks(ctypes.byref(p), ctypes.byref(kv), FAKE, ctypes.byref(fine), None,
                              FAKE, FAKE, FAKE, need - 1, None) == hs.HS_ERR_WORKSPACE
    assert L.hs_select_blocks(ctypes.byref(p), ctypes.byref(kv), FAKE, ctypes.byref(fine), None,
                              FAKE, FAKE, None, need, None) == hs.HS_ERR_WORKSPACE
    assert L.hs_select_blocks(ctypes.byref(p), ctypes.byref(kv), None, ctypes.byref(fine), None,
                              FAKE, FAKE, FAKE, need, None) == hs.HS_ERR_INVALID_ARG
    n = ctypes.c_size_t(0)
    assert L.hs_decode_workspace_size(ctypes.byref(kv), 32, 32, 145, ctypes.byref(n)) == hs.HS_OK
    dneed = n.value
    # 32 units * 8 splits (about one split task per compute unit of the GPU)
    # * 4 heads * (128 + 2) floats, plus counters
    assert dneed >= 32 * 8 * 4 * 130 * 4 + 32 * 4
    args = (ctypes.byref(kv), FAKE, 32, ctypes.c_float(0.0), 32, FAKE, FAKE, 145, FAKE)
    assert L.hs_sparse_decode(*args, FAKE, dneed - 1, None) == hs.HS_ERR_WORKSPACE
    assert L.hs_sparse_decode(ctypes.byref(kv), FAKE, 32, ctypes.c_float(float("nan")), 32, FAKE,
                              FAKE, 145, FAKE, FAKE, dneed, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_sparse_decode(ctypes.byref(kv), FAKE, 32, ctypes.c_float(0.0), 0, FAKE, FAKE,
                              145, FAKE, FAKE, dneed, None) == hs.HS_ERR_INVALID_ARG
    kv_nov = kv_struct(v_pool=0)
    assert L.hs_sparse_decode(ctypes.byref(kv_nov), FAKE, 32, ctypes.c_float(0.0), 32, FAKE, FAKE,
                              145, FAKE, FAKE, dneed, None) == hs.HS_ERR_INVALID_ARG
    # build: bad block_begin, missing K pool, misaligned pool
    assert L.hs_build_summaries(ctypes.byref(kv), -1, ctypes.byref(fine), None) == \
        hs.HS_ERR_INVALID_ARG
    kv_nok = kv_struct(k_pool=0)
    assert L.hs_build_summaries(ctypes.byref(kv_nok), 0, ctypes.byref(fine), None) == \
        hs.HS_ERR_INVALID_ARG
    kv_mis = kv_struct(k_pool=FAKE + 2)
    assert L.hs_build_summaries(ctypes.byref(kv_mis), 0, ctypes.byref(fine), None) == \
        hs.HS_ERR_INVALID_ARG
    assert L.hs_build_summaries(None, 0, ctypes.byref(fine), None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_select_workspace_size(None, ctypes.byref(kv), ctypes.byref(fine), None,
                                      ctypes.byref(n)) == hs.HS_ERR_INVALID_ARG


def test_append_rejects_bad_arguments_before_launch():
    L = hs.lib()
    kv = kv_struct()
    sl = kv.seq_lens
    # missing or misaligned rows, a length array other than the cache's, no V pool
    assert L.hs_append_kv(ctypes.byref(kv), None, FAKE, sl, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_append_kv(ctypes.byref(kv), FAKE, FAKE + 4, sl, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_append_kv(ctypes.byref(kv), FAKE, FAKE, sl + 64, None) == hs.HS_ERR_INVALID_ARG
    assert L.hs_append_kv(ctypes.byref(kv), FAKE, FAKE, None, None) == hs.HS_ERR_INVALID_ARG
    kv_nov = kv_struct(v_pool=0)
    assert L.hs_append_kv(ctypes.byref(kv_nov), FAKE, FAKE, sl, None) == hs.HS_ERR_INVALID_ARG
    kv_bad = kv_struct(head_dim=96)
    assert L.hs_append_kv(ctypes.byref(kv_bad), FAKE, FAKE, sl, None) == hs.HS_ERR_UNSUPPORTED
    assert L.hs_append_kv(None, FAKE, FAKE, sl, None) == hs.HS_ERR_INVALID_ARG


def test_block_cache_rejects_bad_arguments_before_launch():
    L = hs.lib()
    c = hs.hs_block_cache(FAKE, FAKE + 4096, 580)
    args = lambda **o: [o.get(k, v) for k, v in (  # noqa: E731
        ("cache", ctypes.byref(c)), ("units", 32), ("step", 0), ("ids", FAKE), ("cnt", FAKE),
        ("ms", 145), ("slot_of", FAKE), ("miss", FAKE), ("stats", FAKE), ("stream", None))]
    assert L.hs_block_cache_update(*args(cache=None)) == hs.HS_ERR_INVALID_ARG
    assert L.hs_block_cache_update(*args(units=0)) == hs.HS_ERR_INVALID_ARG
    assert L.hs_block_cache_update(*args(step=-1)) == hs.HS_ERR_INVALID_ARG
    assert L.hs_block_cache_update(*args(step=2 ** 31 - 1)) == hs.HS_ERR_INVALID_ARG
    assert L.hs_block_cache_update(*args(ids=None)) == hs.HS_ERR_INVALID_ARG
    assert L.hs_block_cache_update(*args(stats=None)) == hs.HS_ERR_INVALID_ARG
    assert L.hs_block_cache_update(*args(ms=581)) == hs.HS_ERR_INVALID_ARG  # capacity < max_selected
    big = hs.hs_block_cache(FAKE, FAKE + 4096, 1025)
    assert L.hs_block_cache_update(*args(cache=ctypes.byref(big))) == hs.HS_ERR_UNSUPPORTED
    empty = hs.hs_block_cache(None, FAKE, 580)
    assert L.hs_block_cache_update(*args(cache=ctypes.byref(empty))) == hs.HS_ERR_INVALID_ARG


def test_select_ratio_and_forced_validation():
    kv, fine = kv_struct(), summ()
    base = (32, 128, 512, 0, 145)
    P = lambda ratio=0.0, forced=None, cap=0, ms=145: hs.hs_select_params(  # noqa: E731
        *base[:4], ms, ratio, forced, cap)
    assert sel_size(P(), kv, fine)[0] == hs.HS_OK
    assert sel_size(P(ratio=float("nan")), kv, fine)[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(P(ratio=1.5), kv, fine)[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(P(ratio=-0.1), kv, fine)[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(P(cap=4), kv, fine)[0] == hs.HS_ERR_INVALID_ARG        # cap without ids
    assert sel_size(P(forced=FAKE), kv, fine)[0] == hs.HS_ERR_INVALID_ARG  # ids without cap
    # capacity counts the forced blocks: 128 + 16 + 1 + 4 = 149 rows
    assert sel_size(P(forced=FAKE, cap=4, ms=148), kv, fine)[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(P(forced=FAKE, cap=4, ms=149), kv, fine)[0] == hs.HS_OK
    # with a ratio the k of max_blocks blocks counts: int(4096 * 0.05) = 204 -> 221 rows
    assert sel_size(P(ratio=0.05, ms=220), kv, fine)[0] == hs.HS_ERR_INVALID_ARG
    assert sel_size(P(ratio=0.05, ms=221), kv, fine)[0] == hs.HS_OK


def test_noalloc_step_refuses_before_any_hip_call():
    """hs_decode_step_noalloc checks its arguments and the step's workspace
    size against HS_NOALLOC_SCRATCH_BYTES before any HIP call (this host has
    no GPU): a step too large for the array is refused with HS_ERR_WORKSPACE,
    bad arguments with HS_ERR_INVALID_ARG."""
    L = hs.lib()
    fine = summ()
    nb = ctypes.c_size_t(0)

    def call(p, kv, refresh=4095, q=FAKE + (1 << 20)):
        return L.hs_decode_step_noalloc(ctypes.byref(p), ctypes.byref(kv), q, ctypes.byref(fine),
                                        None, refresh, ctypes.c_float(0.0), FAKE + (2 << 20),
                                        FAKE + (3 << 20), FAKE + (4 << 20), None)

    # 256 sequences x 8 KV heads at 128K: 2048 units of 4096 scores (32 MiB)
    # alone, beyond the 16 MiB array
    kv = kv_struct(batch=256, num_phys_pages=256 * 4096)
    p = hs.hs_select_params(32, 128, 512, 0, 145)
    assert L.hs_select_decode_workspace_size(ctypes.byref(p), ctypes.byref(kv),
                                             ctypes.byref(fine), None,
                                             ctypes.byref(nb)) == hs.HS_OK
    assert nb.value > hs.NOALLOC_SCRATCH_BYTES
    assert call(p, kv) == hs.HS_ERR_WORKSPACE
    small = kv_struct()  # the 128K workload itself fits
    assert L.hs_select_decode_workspace_size(ctypes.byref(p), ctypes.byref(small),
                                             ctypes.byref(fine), None,
                                             ctypes.byref(nb)) == hs.HS_OK
    assert nb.value <= hs.NOALLOC_SCRATCH_BYTES
    assert call(p, small, refresh=-1) == hs.HS_ERR_INVALID_ARG
    assert call(p, small, q=FAKE + 2) == hs.HS_ERR_INVALID_ARG
    assert call(hs.hs_select_params(32, 128, 512, 0, 10), small) == hs.HS_ERR_INVALID_ARG


def test_token_stage_lds_cap():
    """hs_select_tokens sizes its general path's LDS (a bitmap of max_seq_len
    bits and the staged list of max_tokens + 64 entries) against
    HS_TOKEN_LDS_BYTES: the largest capacity that fits is accepted, one token
    more is refused, and the register path (at most 8192 slots and 512
    blocks) needs no per-sequence LDS at any capacity."""
    m = re.search(r"#define HS_TOKEN_LDS_BYTES \((\d+) << (\d+)\)", open(HEADER).read())
    budget = int(m.group(1)) << int(m.group(2))
    L = hs.lib()
    size = ctypes.c_size_t(0)

    def ws(max_seq_len, ms, S=32, kt=512, wt=64):
        kv = kv_struct(batch=1, num_kv_heads=2, max_pages=-(-max_seq_len // 32),
                       max_seq_len=max_seq_len)
        max_tok = min(ms * S, kt) + wt
        return L.hs_select_tokens_workspace_size(ctypes.byref(kv), 8, S, ms, kt, wt, max_tok,
                                                 ctypes.byref(size))

    cap = 32 * (budget // 4 - (512 + 64) - 64)  # 300 blocks: general path, 576 kept at most
    assert ws(cap, 300) == hs.HS_OK
    assert ws(cap + 1, 300) == hs.HS_ERR_UNSUPPORTED
    assert ws(1 << 30, 200) == hs.HS_OK  # register path: 6400 slots, 200 blocks

