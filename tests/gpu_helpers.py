"""Helpers for the GPU parity tests: put a workload on the device, run the
library's three entry points, run the oracle on chosen units and compare.

Comparison rules (stated by the target of the build, with the readings of
the open points):
  * block ids: bit-exact, except blocks whose oracle score lies within
    1e-6 * max(|s_k|, sum_j sum_i |q_j,i x_beta,i|) of the oracle's k-th kept
    score s_k (a near tie that fp32 accumulation order may resolve either
    way); window blocks must always be present;
  * outputs: per output row (b, h), ||o_gpu - o_ref||_inf / ||o_ref||_inf
    <= 2e-3 for bf16 caches and <= 1e-5 for fp32 caches; the GPU path
    accumulates in fp32 on exactly the stored inputs, so it is also held to
    KERNEL_RTOL = 2e-5 (fp32 rounding of a <=10^4-term softmax), which catches
    a dropped or doubled token that the looser bound could let through.
"""
from __future__ import annotations

import math
import sys
import time
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np
import torch

import hierarchical_sparse_attention_amd as hs
import oracle
import synth
from synth import device as sdev
from synth.workloads import Workload

# accepted relative error of an output row per cache dtype (bf16 inputs
# carry 8 significand bits; float32 caches are held to 1e-5)
OUTPUT_RTOL = {"bf16": 2e-3, "f32": 1e-5}
KERNEL_RTOL = 2e-5
TIE_RTOL = 1e-6


def log(msg: str) -> None:
    print("[%s] %s" % (time.strftime("%H:%M:%S"), msg), flush=True)
    sys.stdout.flush()


@dataclass
class Problem:
    w: Workload
    layers: int = 1
    kvs: List[hs.KVCache] = field(default_factory=list)
    page_table: Optional[torch.Tensor] = None
    seq_lens: Optional[torch.Tensor] = None
    rows_of: Optional[Callable] = None  # (which, layer, b) -> [Hkv][T][d], else the generator

    @staticmethod
    def make(w: Workload, layers: int = 1, rows_of: Optional[Callable] = None) -> "Problem":
        p = Problem(w=w, layers=layers, rows_of=rows_of)
        p.page_table = sdev.page_table_tensor(w)
        p.seq_lens = sdev.seq_lens_tensor(w)
        for layer in range(layers):
            kp, vp = sdev.make_pools(w, layer, rows_of=rows_of)
            p.kvs.append(hs.KVCache(kp, vp, p.page_table, p.seq_lens, w.T))
        torch.cuda.synchronize()
        return p

    def unit_inputs(self, layer: int, b: int, g: int, step: int = 0):
        """Oracle-side q [G][d], K and V rows [T][d] (float64) of one unit,
        from the same rows the pools were filled with."""
        if self.rows_of is None:
            return unit_inputs(self.w, layer, b, g, step)
        w = self.w
        q = synth.widen(w.q(layer, step), w.dtype)[b, g * w.G:(g + 1) * w.G]
        K = synth.widen(self.rows_of("k", layer, b)[g], w.dtype)
        V = synth.widen(self.rows_of("v", layer, b)[g], w.dtype)
        return q, K, V

    def q(self, layer=0, step=0) -> torch.Tensor:
        return sdev.q_tensor(self.w, layer, step)

    def summaries(self, layer=0) -> Dict[str, hs.Summaries]:
        w, kv = self.w, self.kvs[layer]
        fine = hs.Summaries.empty(kv, w.kind, w.S)
        hs.hs_build_summaries(kv, fine)
        out = {"fine": fine}
        if w.top_k_coarse:
            coarse = hs.Summaries.empty(kv, "mean", w.coarse_S)
            hs.hs_build_summaries(kv, coarse)
            out["coarse"] = coarse
        return out

    def select(self, q: torch.Tensor, summ: Dict[str, hs.Summaries], top_k=None, window=None,
               max_selected=None):
        w, kv = self.w, self.kvs[0]
        k = w.top_k if top_k is None else top_k
        W = w.window if window is None else window
        cap = max_selected or min(w.nb, min(k, w.nb) + -(-W // w.S) + 1)
        ids = torch.full((w.batch, w.hkv, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
        coarse = summ.get("coarse")
        n = hs.hs_select_workspace_size(kv, summ["fine"], w.hq, k, W, cap, coarse, w.top_k_coarse)
        ws = hs.workspace(n, "cuda")
        hs.hs_select_blocks(kv, q, summ["fine"], k, W, ids, cnt, ws, coarse, w.top_k_coarse)
        return ids, cnt

    def select_decode(self, q: torch.Tensor, summ: Dict[str, hs.Summaries], top_k=None,
                      window=None, max_selected=None, layer=0, ws=None):
        """hs_select_decode (one launch); returns ids, counts, out and the
        workspace (so that a test can call again with the same one)."""
        w, kv = self.w, self.kvs[layer]
        k = w.top_k if top_k is None else top_k
        W = w.window if window is None else window
        cap = max_selected or min(w.nb, min(k, w.nb) + -(-W // w.S) + 1)
        ids = torch.full((w.batch, w.hkv, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
        out = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        coarse = summ.get("coarse")
        if ws is None:
            n = hs.hs_select_decode_workspace_size(kv, summ["fine"], w.hq, k, W, cap, coarse,
                                                   w.top_k_coarse)
            ws = hs.workspace(n, "cuda")
        hs.hs_select_decode(kv, q, summ["fine"], k, W, ids, cnt, out, ws, coarse, w.top_k_coarse)
        return ids, cnt, out, ws

    def decode_step(self, q: torch.Tensor, summ: Dict[str, hs.Summaries], refresh_begin: int,
                    layer=0, ws=None):
        """hs_decode_step (refresh + selection + attention); returns ids,
        counts, out and the workspace."""
        w, kv = self.w, self.kvs[layer]
        cap = min(w.nb, min(w.top_k, w.nb) + -(-w.window // w.S) + 1)  # as select_decode
        ids = torch.full((w.batch, w.hkv, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((w.batch, w.hkv), -7, dtype=torch.int32, device="cuda")
        out = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        coarse = summ.get("coarse")
        if ws is None:
            n = hs.hs_select_decode_workspace_size(kv, summ["fine"], w.hq, w.top_k, w.window, cap,
                                                   coarse, w.top_k_coarse)
            ws = hs.workspace(n, "cuda")
        hs.hs_decode_step(kv, q, summ["fine"], w.top_k, w.window, refresh_begin, ids, cnt, out,
                          ws, coarse, w.top_k_coarse)
        return ids, cnt, out, ws

    def decode(self, q: torch.Tensor, ids: torch.Tensor, cnt: torch.Tensor, layer=0,
               block_size=None):
        w, kv = self.w, self.kvs[layer]
        S = w.S if block_size is None else block_size
        n = hs.hs_decode_workspace_size(kv, w.hq, S, ids.shape[-1])
        ws = hs.workspace(n, "cuda")
        out = torch.full((w.batch, w.hq, w.d), float("nan"), dtype=torch.float32, device="cuda")
        hs.hs_sparse_decode(kv, q, S, ids, cnt, out, ws)
        return out


def unit_inputs(w: Workload, layer: int, b: int, g: int, step: int = 0):
    """Oracle-side inputs of one unit: q [G][d], K and V rows [T][d] (float64)."""
    q = synth.widen(w.q(layer, step), w.dtype)[b, g * w.G:(g + 1) * w.G]
    K = synth.widen(w.k_unit(layer, b, g), w.dtype)
    V = synth.widen(w.v_unit(layer, b, g), w.dtype)
    return q, K, V


def oracle_select(w: Workload, q, K, T, top_k=None, window=None):
    k = w.top_k if top_k is None else top_k
    W = w.window if window is None else window
    return oracle.select_unit(q, K, T, w.kind, w.S, k, W, coarse_S=w.coarse_S,
                              top_k_coarse=w.top_k_coarse)


def magnitudes(w: Workload, q, K, T) -> np.ndarray:
    """sum_j sum_i |q_j,i| * |x_beta,i| for every fine block (the scale of
    the terms that make up a block score)."""
    a, b = oracle.summarize(K[:T], w.S, w.kind)
    x = np.abs(a) if b is None else np.maximum(np.abs(a), np.abs(b))
    return x @ np.abs(q).sum(axis=0)


def paired_differences(got: List[int], ref: List[int], what: str):
    """The GPU list and the oracle's must have the same size; returns the
    pairs (dropped oracle id, extra GPU id), each side in ascending order.
    Every difference is then one oracle id traded for one GPU id, and both
    members of each pair are judged by the near-tie rule."""
    assert len(got) == len(ref), "%s: %d ids, the oracle keeps %d" % (what, len(got), len(ref))
    dropped = sorted(set(ref) - set(got))
    extra = sorted(set(got) - set(ref))
    assert len(dropped) == len(extra), what
    return list(zip(dropped, extra))


def check_ids(w: Workload, gpu_ids: np.ndarray, sel: oracle.UnitSelection, mags: np.ndarray,
              T: int, window=None, what="") -> int:
    """Assert the near-tie rule; returns the number of tolerated differences
    (pairs of one dropped oracle block and one extra GPU block)."""
    W = w.window if window is None else window
    g = gpu_ids.tolist()
    assert g == sorted(set(g)), "%s: ids not strictly ascending: %s" % (what, g[:20])
    pairs = paired_differences(g, sel.ids.tolist(), what)
    if not pairs:
        return 0
    win = set(oracle.window_blocks(T, w.S, W).tolist())
    sk = sel.kth_score
    for pair in pairs:
        for beta in pair:
            assert beta not in win, "%s: window block %d differs" % (what, beta)
            s = sel.fine_scores[beta] if 0 <= beta < len(sel.fine_scores) else float("nan")
            assert not math.isnan(s), "%s: block %d was not a candidate" % (what, beta)
            tol = TIE_RTOL * max(abs(sk), mags[beta])
            assert abs(s - sk) <= tol, (
                "%s: block %d (pair %s) differs, score %.9g vs k-th %.9g (tol %.3g)"
                % (what, beta, pair, s, sk, tol))
    return len(pairs)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per output row ||got - ref||_inf / ||ref||_inf (0 where both are zero)."""
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def check_rows(w: Workload, got: np.ndarray, ref: np.ndarray, what="") -> float:
    assert np.all(np.isfinite(got)), "%s: non-finite output" % what
    err = float(row_rel_err(got, ref).max()) if got.size else 0.0
    tol = OUTPUT_RTOL[w.dtype]
    assert err <= tol, "%s: max row rel err %.3g > %.3g" % (what, err, tol)
    assert err <= KERNEL_RTOL, "%s: max row rel err %.3g > kernel bound %.3g" % (
        what, err, KERNEL_RTOL)
    return err


def check_tokens(gi, ref_ids, scores, kth, qo, K, T, W, what):
    """Equal sizes; each (dropped, extra) pair of differing tokens is judged
    by the near-tie rule on both members. Returns the number of pairs."""
    g = gi.tolist()
    assert g == sorted(set(g)), what
    pairs = paired_differences(g, ref_ids.tolist(), what)
    mag = np.abs(K[:T]) @ np.abs(qo).sum(axis=0)
    for pair in pairs:
        for t in pair:
            assert not (t >= T - W), "%s: window token %d differs" % (what, t)
            s = scores[t] if 0 <= t < T else float("nan")
            assert not np.isnan(s), "%s: token %d was not a candidate" % (what, t)
            tol = 1e-6 * max(abs(kth), mag[t])
            assert abs(s - kth) <= tol, "%s: token %d (pair %s) score %.9g vs k-th %.9g" % (
                what, t, pair, s, kth)
    return len(pairs)
