"""CPU oracle of query-guided block-sparse decode attention.

TEST INFRASTRUCTURE ONLY. The tests, the smoke check and the benchmark's
CPU-baseline leg may use this package; the library and its Python binding
never do. It shares no code with the GPU path and imports nothing from it.

The arithmetic lives in ``hs_oracle.c`` (plain loops, float64); this module
only marshals numpy arrays through ctypes and loops over units. Inputs are
the stored values (float32 arrays, or bfloat16 bit patterns as uint16), which
are widened to float64 exactly.

Parity status: every function here is pinned by the CPU tests against
closed forms, brute force, textbook dense attention or invariants; none is
"parity unpinned".
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hs_oracle.c")
_LIB = os.path.join(_HERE, "libhs_oracle.so")
_lib = None

F32, BF16 = 0, 1


def build(force: bool = True) -> str:
    """Compile hs_oracle.c into libhs_oracle.so with gcc."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-shared", "-fPIC",
                               "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        vp, i32, i64, dbl = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        L.hso_gather_unit.argtypes = [vp, i32, vp, i32, i32, i32, i32, i32, i32, i32, i32, vp]
        L.hso_gather_unit.restype = i32
        L.hso_summary_mean.argtypes = [vp, i32, i32, i32, vp]
        L.hso_summary_minmax.argtypes = [vp, i32, i32, i32, vp, vp]
        L.hso_scores_mean.argtypes = [vp, i32, i32, vp, vp, i32, vp]
        L.hso_scores_minmax.argtypes = [vp, i32, i32, vp, vp, vp, i32, vp]
        L.hso_topk.argtypes = [vp, vp, i32, i32, vp]
        L.hso_topk.restype = i32
        L.hso_window.argtypes = [i32, i32, i32, vp]
        L.hso_select_unit.argtypes = [vp, i32, i32, i32, i32, vp, vp, i32, i32, i32, vp, vp,
                                      i32, vp, vp, vp, vp]
        L.hso_select_unit.restype = i32
        L.hso_attend_unit.argtypes = [vp, i32, i32, vp, vp, i32, vp, i32, i32, dbl, vp]
        for name in ("hso_summary_mean", "hso_summary_minmax", "hso_scores_mean",
                     "hso_scores_minmax", "hso_window", "hso_attend_unit"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    if a is None:
        return None
    assert a.flags.c_contiguous, "oracle inputs must be C-contiguous"
    return a.ctypes.data


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, np.float64)


def gather_unit(pool: np.ndarray, dtype: int, page_table: np.ndarray, b: int, g: int,
                T: int) -> np.ndarray:
    """Rows [T][d] of unit (b, g) read through the page table."""
    pool = np.ascontiguousarray(pool)
    pt = np.ascontiguousarray(page_table, np.int32)
    nphys, hkv, P, d = pool.shape
    rows = np.empty((T, d), np.float64)
    rc = lib().hso_gather_unit(_p(pool), dtype, _p(pt), pt.shape[1], nphys, hkv, P, d, b, g, T,
                               _p(rows))
    if rc != 0:
        raise ValueError("page table entry out of range")
    return rows


def summary_mean(rows: np.ndarray, S: int) -> np.ndarray:
    rows = _f64(rows)
    T, d = rows.shape
    mu = np.empty((-(-T // S), d), np.float64)
    lib().hso_summary_mean(_p(rows), T, d, S, _p(mu))
    return mu


def summary_minmax(rows: np.ndarray, S: int):
    rows = _f64(rows)
    T, d = rows.shape
    nb = -(-T // S)
    mn = np.empty((nb, d), np.float64)
    mx = np.empty((nb, d), np.float64)
    lib().hso_summary_minmax(_p(rows), T, d, S, _p(mn), _p(mx))
    return mn, mx


def scores_mean(q: np.ndarray, mu: np.ndarray, rows_of: Optional[np.ndarray] = None):
    q, mu = _f64(q), _f64(mu)
    G, d = q.shape
    ro = None if rows_of is None else np.ascontiguousarray(rows_of, np.int32)
    n = mu.shape[0] if ro is None else len(ro)
    s = np.empty(n, np.float64)
    lib().hso_scores_mean(_p(q), G, d, _p(mu), _p(ro), n, _p(s))
    return s


def scores_minmax(q: np.ndarray, mn: np.ndarray, mx: np.ndarray,
                  rows_of: Optional[np.ndarray] = None):
    q, mn, mx = _f64(q), _f64(mn), _f64(mx)
    G, d = q.shape
    ro = None if rows_of is None else np.ascontiguousarray(rows_of, np.int32)
    n = mn.shape[0] if ro is None else len(ro)
    s = np.empty(n, np.float64)
    lib().hso_scores_minmax(_p(q), G, d, _p(mn), _p(mx), _p(ro), n, _p(s))
    return s


def topk(s: np.ndarray, k: int, ids: Optional[np.ndarray] = None) -> np.ndarray:
    s = _f64(s)
    ids_ = None if ids is None else np.ascontiguousarray(ids, np.int32)
    out = np.empty(max(len(s), 1), np.int32)
    m = lib().hso_topk(_p(s), _p(ids_), len(s), k, _p(out))
    return out[:m].copy()


def window_blocks(T: int, S: int, W: int) -> np.ndarray:
    nb = -(-T // S)
    mark = np.zeros(max(nb, 1), np.uint8)
    lib().hso_window(T, S, W, _p(mark))
    return np.nonzero(mark[:nb])[0].astype(np.int32)


@dataclass
class UnitSelection:
    ids: np.ndarray            # ascending selected block ids
    fine_scores: np.ndarray    # [nb] fine score of each candidate, NaN otherwise
    coarse_ids: np.ndarray     # kept coarse blocks (rank order), empty if single level
    kth_score: float           # score of the last block kept by the fine top-k (NaN if none)
    fine_top: np.ndarray       # fine top-k ids in rank order


def summarize(rows: np.ndarray, S: int, kind: str):
    """(a, b) summary pair: ('mean') -> (mu, None); ('minmax') -> (mn, mx)."""
    if kind == "mean":
        return summary_mean(rows, S), None
    return summary_minmax(rows, S)


def ratio_k(nb: int, ratio: float) -> int:
    """k of a fixed-ratio selection over nb blocks: max(1, int(nb * ratio))
    ("SparDA", section 3.2 and its inference listing in section 3.4). The
    ratio is the float32 value a caller passes; nb * ratio is exact in float64."""
    return max(1, int(nb * float(np.float32(ratio))))


def length_ratio(T: int) -> float:
    """The length schedule of "SparDA" section 3.2: no compression up to 8K
    tokens, 15 % up to 16K, 10 % up to 32K, 5 % beyond (the page's example
    points 16K, 32K and 128K; each length takes the ratio of the first point
    at or above it)."""
    if T <= 8192:
        return 1.0
    if T <= 16384:
        return 0.15
    if T <= 32768:
        return 0.10
    return 0.05


def select_unit(q: np.ndarray, rows_k: np.ndarray, T: int, kind: str, S: int, top_k: int,
                window: int, coarse_S: int = 0, top_k_coarse: int = 0,
                coarse_kind: str = "mean", summaries=None, top_k_ratio: float = 0.0,
                forced=None) -> UnitSelection:
    """Full selection of one unit from its key rows [>=T][d] (only t < T used).

    top_k_ratio > 0 replaces top_k by ratio_k(ceil(T / S), top_k_ratio).
    forced: caller-supplied block ids ("SparDA" section 3.4: a small random
    reserve set kept besides the scored top-k) unioned into the selection;
    ids outside [0, ceil(T / S)) are ignored."""
    if top_k_ratio > 0:
        top_k = ratio_k(-(-T // S), top_k_ratio)
    q = _f64(q)
    G, d = q.shape
    rows = _f64(rows_k[:T])
    if summaries is None:
        fa, fb = summarize(rows, S, kind)
        ca = cb = None
        if top_k_coarse > 0:
            ca, cb = summarize(rows, coarse_S, coarse_kind)
    else:
        fa, fb, ca, cb = summaries
    nb = -(-T // S)
    ids = np.empty(max(nb, 1), np.int32)
    fs = np.empty(max(nb, 1), np.float64)
    cids = np.empty(max(top_k_coarse, 1), np.int32)
    ncs = ctypes.c_int(0)
    cnt = lib().hso_select_unit(_p(q), G, d, T, S, _p(fa), _p(fb), top_k, window,
                                max(coarse_S, 1), _p(ca), _p(cb), top_k_coarse, _p(ids),
                                _p(fs), _p(cids), ctypes.addressof(ncs))
    fs = fs[:nb]
    cand = np.nonzero(~np.isnan(fs))[0].astype(np.int32)
    ftop = topk(fs[cand], top_k, cand) if len(cand) else np.zeros(0, np.int32)
    kth = float(np.float32(fs[ftop[-1]])) if len(ftop) else float("nan")
    sel_ids = ids[:cnt].copy()
    if forced is not None and len(forced):
        f = np.asarray(forced, np.int64)
        f = f[(f >= 0) & (f < nb)].astype(np.int32)
        sel_ids = np.union1d(sel_ids, f).astype(np.int32)
    return UnitSelection(ids=sel_ids, fine_scores=fs.copy(),
                         coarse_ids=cids[:ncs.value].copy(), kth_score=kth, fine_top=ftop)


def select_tokens_unit(q: np.ndarray, rows_k: np.ndarray, T: int, block_ids, S: int,
                       top_k_tokens: int, window_tokens: int):
    """Token-level second stage inside the selected blocks ("SparDA", section
    2.3: after the block selection, a finer pass keeps single tokens inside the
    chosen blocks). Candidates: the tokens t < T of blocks `block_ids`. Score
    of token t: the sum over the G query heads of q_j . k_t (the block score
    with the block reduced to one token), computed in float64 and rounded to
    float32 for ranking. Kept: the first min(k, #candidates) candidates by
    (score desc, token asc), plus every token of the window [T - W, T) (as at
    the block level, the local window is always attended). Returns (ascending
    token ids, scores of all T tokens with NaN for non-candidates, the k-th
    kept score)."""
    q = _f64(q)
    K = _f64(rows_k[:T])
    cand = sorted({t for b in np.asarray(block_ids, np.int64).tolist() if 0 <= b
                   for t in range(b * S, min(b * S + S, T))})
    scores = np.full(T, np.nan)
    qs = q.sum(axis=0)
    for t in cand:
        scores[t] = float(np.float32(np.dot(K[t], qs)))
    order = sorted(cand, key=lambda t: (-scores[t], t))
    top = order[:max(0, min(top_k_tokens, len(order)))]
    win = list(range(max(0, T - window_tokens), T)) if window_tokens > 0 else []
    kth = scores[top[-1]] if top else float("nan")
    return np.array(sorted(set(top) | set(win)), np.int32), scores, kth


def attend_unit(q: np.ndarray, K: np.ndarray, V: np.ndarray, T: int, ids: np.ndarray, S: int,
                scale: Optional[float] = None) -> np.ndarray:
    """Exact softmax attention of q [G][d] over the tokens t < T of blocks `ids`."""
    q = _f64(q)
    G, d = q.shape
    K, V = _f64(K[:T]), _f64(V[:T])
    ids = np.ascontiguousarray(ids, np.int32)
    out = np.empty((G, d), np.float64)
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    lib().hso_attend_unit(_p(q), G, d, _p(K), _p(V), T, _p(ids), len(ids), S, sc, _p(out))
    return out


def map_units(fn, n_units: int, threads: int = 1):
    """Run fn(u) for u in range(n_units), optionally on a thread pool (the C
    calls release the GIL)."""
    if threads <= 1:
        return [fn(u) for u in range(n_units)]
    with ThreadPoolExecutor(max_workers=threads) as ex:
        return list(ex.map(fn, range(n_units)))
