"""Place generated inputs into device memory (torch), in the paged layout.

Plumbing only: the values come from the generator; this module moves them
into pools [num_phys_pages][Hkv][P][d] through the workload's page table.
"""
from __future__ import annotations

import numpy as np
import torch

from .workloads import Workload

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def to_torch(x: np.ndarray, dtype: str) -> torch.Tensor:
    """Host numpy storage (float32, or bf16 bits as uint16) -> torch CPU tensor."""
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, np.float32))
    return torch.from_numpy(np.ascontiguousarray(x, np.uint16).view(np.int16)).view(torch.bfloat16)


def q_tensor(w: Workload, layer: int = 0, step: int = 0, device="cuda") -> torch.Tensor:
    return to_torch(w.q(layer, step), w.dtype).to(device)


def page_table_tensor(w: Workload, device="cuda") -> torch.Tensor:
    return torch.from_numpy(w.page_table()).to(device)


def seq_lens_tensor(w: Workload, device="cuda") -> torch.Tensor:
    return torch.from_numpy(w.seq_lens_array()).to(device)


def fill_pool(w: Workload, which: str, layer: int, pool: torch.Tensor,
              page_table: np.ndarray, rows_of=None) -> None:
    """Write one layer's K or V of every unit into `pool` (device tensor
    [num_phys][Hkv][P][d]) through `page_table` [B][max_pages]. rows_of:
    optional callable (which, layer, b) -> [Hkv][T][d] storage rows that
    replaces the generator (a test that edits the generated rows)."""
    P, d, npg = w.page_size, w.d, w.max_pages
    pad = npg * P - w.T
    dev = pool.device
    get = rows_of if rows_of is not None else w.kv_rows
    for b in range(w.batch):
        rows = to_torch(get(which, layer, b), w.dtype).to(dev)  # [Hkv][T][d]
        if pad:
            rows = torch.cat([rows, torch.zeros((w.hkv, pad, d), dtype=rows.dtype, device=dev)], 1)
        pages = rows.view(w.hkv, npg, P, d).permute(1, 0, 2, 3)      # [npg][Hkv][P][d]
        idx = torch.from_numpy(page_table[b].astype(np.int64)).to(dev)
        pool.index_copy_(0, idx, pages.contiguous())
        del rows, pages


def make_pools(w: Workload, layer: int = 0, device="cuda", rows_of=None):
    """(k_pool, v_pool) device tensors of one layer (rows_of: see fill_pool)."""
    shape = (w.num_phys_pages, w.hkv, w.page_size, w.d)
    pt = w.page_table()
    kp = torch.zeros(shape, dtype=TORCH_DTYPE[w.dtype], device=device)
    vp = torch.zeros(shape, dtype=TORCH_DTYPE[w.dtype], device=device)
    fill_pool(w, "k", layer, kp, pt, rows_of)
    fill_pool(w, "v", layer, vp, pt, rows_of)
    return kp, vp
