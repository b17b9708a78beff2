"""The five seeded synthetic decode workloads and their input recipe.

Recipe (random values only; no attention arithmetic here):
  * seed = 1000 * config. Streams: q = 1, K = 2, V = 3, needle positions = 4,
    needle noise = 5, page table = 6, query drift = 7; layer l adds 16 * l.
  * q, K, V ~ N(0, 1), rounded to the cache dtype. Element (b, g, t, i) of a
    layer's K (or V) has counter index ((b * Hkv + g) * T + t) * d + i, so any
    unit can be regenerated alone. q element (b, h, i) has index
    (b * Hq + h) * d + i.
  * Needles stand in for a needle-in-a-haystack workload: a few far-context
    blocks whose keys align with the query. For unit (b, g), q_dir is the
    normalised sum of the unit's G rounded query heads (fp64); `needles`
    blocks are drawn without replacement (partial Fisher-Yates, stream 4)
    among the blocks that end before the window; each key of those blocks is
    RNE(3 * q_dir + N(0, 1)) with the noise from stream 5.
  * Query drift over decode steps: q_t = 0.9 q_{t-1} + 0.44 n_t, n_t ~ N(0, 1)
    from stream 7, kept in fp64 and rounded to the cache dtype for input.
  * Page table: identity (page p of sequence b -> b * max_pages + p), or a
    Fisher-Yates permutation of all B * max_pages physical pages (stream 6),
    shared by every layer and KV head.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass
from typing import Optional, Tuple

import numpy as np

from . import normal, round_to, uniform, widen

STREAM_Q, STREAM_K, STREAM_V = 1, 2, 3
STREAM_NEEDLE_POS, STREAM_NEEDLE_NOISE = 4, 5
STREAM_PAGES, STREAM_DRIFT = 6, 7
LAYER_STRIDE = 16


@dataclass(frozen=True)
class Workload:
    name: str
    config: int
    batch: int
    hq: int
    hkv: int
    d: int
    T: int
    dtype: str            # 'f32' or 'bf16'
    page_size: int
    kind: str             # fine-level summary: 'mean' or 'minmax'
    S: int                # fine block size
    top_k: int
    window: int
    coarse_S: int = 0     # two-level: coarse block size (mean-pooled)
    top_k_coarse: int = 0
    needles: int = 0      # needle blocks per unit (layer 0)
    layers: int = 1
    steps: int = 1        # decode steps with query drift
    random_pages: bool = False
    seq_lens: Optional[Tuple[int, ...]] = None  # ragged T_b; default all T

    # -- derived shapes ---------------------------------------------------
    @property
    def seed(self) -> int:
        return 1000 * self.config

    @property
    def G(self) -> int:
        return self.hq // self.hkv

    @property
    def units(self) -> int:
        return self.batch * self.hkv

    @property
    def nb(self) -> int:
        return -(-self.T // self.S)

    @property
    def nc(self) -> int:
        return -(-self.T // self.coarse_S) if self.coarse_S else 0

    @property
    def max_pages(self) -> int:
        return -(-self.T // self.page_size)

    @property
    def num_phys_pages(self) -> int:
        return self.batch * self.max_pages

    @property
    def max_selected(self) -> int:
        return min(self.nb, min(self.top_k, self.nb) + -(-self.window // self.S) + 1)

    def scaled(self, **changes) -> "Workload":
        return dataclasses.replace(self, **changes)

    def seq_lens_array(self) -> np.ndarray:
        if self.seq_lens is None:
            return np.full(self.batch, self.T, np.int32)
        assert len(self.seq_lens) == self.batch
        return np.asarray(self.seq_lens, np.int32)

    # -- page table -------------------------------------------------------
    def page_table(self) -> np.ndarray:
        n = self.num_phys_pages
        if not self.random_pages:
            perm = np.arange(n, dtype=np.int64)
        else:
            u = uniform(self.seed, STREAM_PAGES, 0, n)
            perm = np.arange(n, dtype=np.int64)
            for i in range(n - 1, 0, -1):
                j = int(u[i] * (i + 1))
                perm[i], perm[j] = perm[j], perm[i]
        return perm.reshape(self.batch, self.max_pages).astype(np.int32)

    # -- queries ----------------------------------------------------------
    def q_master(self, layer: int = 0, step: int = 0) -> np.ndarray:
        """fp64 query state [B][Hq][d] of a layer at a decode step."""
        n = self.batch * self.hq * self.d
        q = normal(self.seed, STREAM_Q + LAYER_STRIDE * layer, 0, n)
        for t in range(1, step + 1):
            z = normal(self.seed, STREAM_DRIFT + LAYER_STRIDE * layer, (t - 1) * n, n)
            q = 0.9 * q + 0.44 * z
        return q.reshape(self.batch, self.hq, self.d)

    def q(self, layer: int = 0, step: int = 0) -> np.ndarray:
        """Query input in the cache dtype (float32, or bf16 bits as uint16)."""
        return round_to(self.q_master(layer, step), self.dtype)

    # -- needles ----------------------------------------------------------
    def needle_blocks(self, b: int, g: int) -> np.ndarray:
        if self.needles <= 0:
            return np.zeros(0, np.int64)
        tb = int(self.seq_lens_array()[b])
        m = max(0, (tb - self.window) // self.S)
        n = min(self.needles, m)
        arr = np.arange(m, dtype=np.int64)
        u = uniform(self.seed, STREAM_NEEDLE_POS, (b * self.hkv + g) * 4096, max(n, 1))
        for i in range(n):
            j = i + int(u[i] * (m - i))
            arr[i], arr[j] = arr[j], arr[i]
        return np.sort(arr[:n])

    def q_dir(self, b: int, g: int) -> np.ndarray:
        qw = widen(self.q(0, 0), self.dtype)[b, g * self.G:(g + 1) * self.G]
        s = qw.sum(axis=0)
        return s / np.linalg.norm(s)

    # -- keys and values --------------------------------------------------
    def _unit_start(self, b: int, g: int) -> int:
        return (b * self.hkv + g) * self.T * self.d

    def plant_needles(self, k: np.ndarray, b: int, g: int) -> None:
        """Overwrite the needle blocks of unit (b, g) in its key rows k [T][d]."""
        blocks = self.needle_blocks(b, g)
        if not len(blocks):
            return
        qd = self.q_dir(b, g)
        unit = b * self.hkv + g
        for ni, beta in enumerate(blocks):
            t0 = int(beta) * self.S
            t1 = min(t0 + self.S, self.T)
            cnt = (t1 - t0) * self.d
            z = normal(self.seed, STREAM_NEEDLE_NOISE,
                       ((unit * self.needles + ni) * self.S) * self.d, cnt)
            rows = 3.0 * qd[None, :] + z.reshape(t1 - t0, self.d)
            k[t0:t1] = round_to(rows, self.dtype)

    def kv_rows(self, which: str, layer: int, b: int, g0: int = 0, g1: Optional[int] = None):
        """Rows of units (b, g0) .. (b, g1 - 1) as [g1 - g0][T][d] in the cache
        dtype ('k' has the needles planted on layer 0)."""
        g1 = self.hkv if g1 is None else g1
        stream = (STREAM_K if which == "k" else STREAM_V) + LAYER_STRIDE * layer
        n = (g1 - g0) * self.T * self.d
        x = normal(self.seed, stream, self._unit_start(b, g0), n, self.dtype)
        x = x.reshape(g1 - g0, self.T, self.d)
        if which == "k" and layer == 0 and self.needles > 0:
            for g in range(g0, g1):
                self.plant_needles(x[g - g0], b, g)
        return x

    def k_unit(self, layer: int, b: int, g: int) -> np.ndarray:
        """Keys of unit (b, g): [T][d] in the cache dtype, needles planted."""
        return self.kv_rows("k", layer, b, g, g + 1)[0]

    def v_unit(self, layer: int, b: int, g: int) -> np.ndarray:
        return self.kv_rows("v", layer, b, g, g + 1)[0]

    # -- whole pools (small workloads only) -------------------------------
    def pools(self, layer: int = 0):
        """(k_pool, v_pool) as numpy [num_phys][Hkv][P][d] in the cache dtype.

        Holds the whole cache on the host: meant for workloads of a few
        hundred MB at most."""
        P, d = self.page_size, self.d
        npg = self.max_pages
        st = np.float32 if self.dtype == "f32" else np.uint16
        kp = np.zeros((self.num_phys_pages, self.hkv, P, d), st)
        vp = np.zeros_like(kp)
        pt = self.page_table()
        pad = npg * P - self.T
        for b in range(self.batch):
            for g in range(self.hkv):
                for src, dst in ((self.k_unit(layer, b, g), kp), (self.v_unit(layer, b, g), vp)):
                    if pad:
                        src = np.concatenate([src, np.zeros((pad, d), st)])
                    dst[pt[b], g] = src.reshape(npg, P, d)
        return kp, vp


def _w(**kw) -> Workload:
    return Workload(**kw)


CONFIGS = {
    1: _w(name="tiny-mha-4k-f32", config=1, batch=1, hq=4, hkv=4, d=64, T=4096,
          dtype="f32", page_size=64, kind="mean", S=64, top_k=8, window=256),
    2: _w(name="mha-32k-bf16-quest", config=2, batch=8, hq=32, hkv=32, d=128, T=32768,
          dtype="bf16", page_size=64, kind="minmax", S=64, top_k=64, window=512, needles=4),
    3: _w(name="gqa-128k-bf16-quest", config=3, batch=4, hq=32, hkv=8, d=128, T=131072,
          dtype="bf16", page_size=32, kind="minmax", S=32, top_k=128, window=512,
          needles=16),
    4: _w(name="two-level-256k-bf16", config=4, batch=8, hq=32, hkv=32, d=128, T=262144,
          dtype="bf16", page_size=64, kind="mean", S=64, top_k=128, window=512,
          coarse_S=1024, top_k_coarse=32, needles=4),
    5: _w(name="shared-selection-64k-bf16", config=5, batch=16, hq=32, hkv=8, d=128,
          T=65536, dtype="bf16", page_size=64, kind="mean", S=64,
          top_k=max(1, int(1024 * 0.1)), window=512, layers=8, steps=16,
          random_pages=True),
}


def storage_bytes(w: Workload) -> int:
    return 4 if w.dtype == "f32" else 2


def summary_row_bytes(w: Workload, kind: str) -> int:
    return w.d * 4 if kind == "mean" else 2 * w.d * storage_bytes(w)
