"""Python binding of libhs_attn.so: query-guided block-sparse decode attention
on MI355X (gfx950).

Argument marshalling only: every step runs in the library's HIP kernels. The
functions keep the C names (hs_build_summaries, hs_select_blocks,
hs_sparse_decode, ...) and take torch tensors, which only provide device
memory; the current torch stream is used unless one is passed. There is no
CPU fallback: if the library has not been built, loading fails with an error.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhs_attn.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_UNSUPPORTED, HS_ERR_WORKSPACE, HS_ERR_HIP = range(5)
HS_F32, HS_BF16 = 0, 1
HS_SUMMARY_MEAN, HS_SUMMARY_MINMAX = 0, 1
HS_STEP_WAIT_EXPIRED = 1
# byte offsets in a hs_select_decode / hs_decode_step workspace (hs_attn.h)
STEP_STATUS_BYTE, STEP_SELECT_BYTE = 0, 256
KIND = {"mean": HS_SUMMARY_MEAN, "minmax": HS_SUMMARY_MINMAX}

# Names declared in include/hs_attn.h; the CPU tests check that each is exported.
EXPORTS = ("hs_select_workspace_size", "hs_decode_workspace_size", "hs_build_summaries",
           "hs_select_blocks", "hs_sparse_decode", "hs_select_decode_workspace_size",
           "hs_select_decode", "hs_decode_step", "hs_append_kv", "hs_block_cache_update",
           "hs_select_tokens_workspace_size", "hs_select_tokens", "hs_step_status",
           "hs_decode_step_noalloc", "hs_status_string", "hs_version")


class hs_block_cache(ctypes.Structure):
    _fields_ = [("slot_block", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("capacity", ctypes.c_int32)]


class HsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s" % (fn, status_string(status)))


class hs_kv_cache(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p),
                ("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_phys_pages", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class hs_summaries(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("kind", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("max_blocks", ctypes.c_int32)]


class hs_select_params(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("window_tokens", ctypes.c_int32), ("top_k_coarse", ctypes.c_int32),
                ("max_selected", ctypes.c_int32), ("top_k_ratio", ctypes.c_float),
                ("forced_ids", ctypes.c_void_p), ("forced_cap", ctypes.c_int32)]


def _sel_params(num_q_heads, top_k, window, top_k_coarse, max_selected, top_k_ratio=0.0,
                forced=None) -> hs_select_params:
    """Selection parameters; forced: None or a contiguous int32 device tensor
    [B][Hkv][forced_cap] of block ids (-1 = none)."""
    if forced is not None:
        if forced.dtype != torch.int32 or not forced.is_contiguous():
            raise ValueError("forced ids must be a contiguous int32 tensor")
        return hs_select_params(num_q_heads, top_k, window, top_k_coarse, max_selected,
                                float(top_k_ratio), _ptr(forced), int(forced.shape[-1]))
    return hs_select_params(num_q_heads, top_k, window, top_k_coarse, max_selected,
                            float(top_k_ratio), None, 0)


_lib = None


def lib() -> ctypes.CDLL:
    """Load libhs_attn.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libhs_attn.so is not built; run "
                              "`python -m hierarchical_sparse_attention_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.hs_select_workspace_size.argtypes = [P(hs_select_params), P(hs_kv_cache),
                                               P(hs_summaries), P(hs_summaries), P(sz)]
        L.hs_decode_workspace_size.argtypes = [P(hs_kv_cache), i32, i32, i32, P(sz)]
        L.hs_build_summaries.argtypes = [P(hs_kv_cache), i32, P(hs_summaries), vp]
        L.hs_select_blocks.argtypes = [P(hs_select_params), P(hs_kv_cache), vp, P(hs_summaries),
                                       P(hs_summaries), vp, vp, vp, sz, vp]
        L.hs_sparse_decode.argtypes = [P(hs_kv_cache), vp, i32, ctypes.c_float, i32, vp, vp, i32,
                                       vp, vp, sz, vp]
        L.hs_select_decode_workspace_size.argtypes = [P(hs_select_params), P(hs_kv_cache),
                                                      P(hs_summaries), P(hs_summaries), P(sz)]
        L.hs_select_decode.argtypes = [P(hs_select_params), P(hs_kv_cache), vp,
                                       P(hs_summaries), P(hs_summaries), ctypes.c_float, vp, vp,
                                       vp, vp, sz, vp]
        L.hs_decode_step.argtypes = [P(hs_select_params), P(hs_kv_cache), vp, P(hs_summaries),
                                     P(hs_summaries), i32, ctypes.c_float, vp, vp, vp, vp, sz, vp]
        L.hs_append_kv.argtypes = [P(hs_kv_cache), vp, vp, vp, vp]
        L.hs_select_tokens_workspace_size.argtypes = [P(hs_kv_cache), i32, i32, i32, i32, i32,
                                                      i32, P(sz)]
        L.hs_select_tokens.argtypes = [P(hs_kv_cache), vp, i32, i32, vp, vp, i32, i32, i32, vp,
                                       vp, i32, vp, sz, vp]
        L.hs_block_cache_update.argtypes = [P(hs_block_cache), i32, i32, vp, vp, i32, vp, vp, vp,
                                            vp]
        L.hs_step_status.argtypes = [vp, sz, P(ctypes.c_int32), vp]
        L.hs_decode_step_noalloc.argtypes = [P(hs_select_params), P(hs_kv_cache), vp,
                                             P(hs_summaries), P(hs_summaries), i32,
                                             ctypes.c_float, vp, vp, vp, vp]
        for name in ("hs_select_workspace_size", "hs_decode_workspace_size",
                     "hs_build_summaries", "hs_select_blocks", "hs_sparse_decode",
                     "hs_select_decode_workspace_size", "hs_select_decode", "hs_decode_step",
                     "hs_append_kv", "hs_block_cache_update",
                     "hs_select_tokens_workspace_size", "hs_select_tokens", "hs_step_status",
                     "hs_decode_step_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        L.hs_status_string.argtypes = [ctypes.c_int]
        L.hs_status_string.restype = ctypes.c_char_p
        L.hs_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def status_string(s: int) -> str:
    return lib().hs_status_string(s).decode()


def _check(fn: str, st: int) -> None:
    if st != HS_OK:
        raise HsError(fn, st)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libhs_attn must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return HS_F32
    if t.dtype == torch.bfloat16:
        return HS_BF16
    raise ValueError("unsupported dtype %s (float32 or bfloat16)" % t.dtype)


@dataclass
class KVCache:
    """One layer's paged cache: pools [num_phys][Hkv][P][d], page_table
    int32 [B][max_pages], seq_lens int32 [B] (all on the device)."""
    k_pool: Optional[torch.Tensor]
    v_pool: Optional[torch.Tensor]
    page_table: torch.Tensor
    seq_lens: torch.Tensor
    max_seq_len: int
    dtype: Optional[torch.dtype] = None
    shape: Optional[tuple] = None  # (num_phys, Hkv, P, d) when pools are absent

    def struct(self) -> hs_kv_cache:
        ref = self.k_pool if self.k_pool is not None else self.v_pool
        shape = tuple(ref.shape) if ref is not None else self.shape
        dt = ref.dtype if ref is not None else self.dtype
        if shape is None or dt is None:
            raise ValueError("KVCache needs a pool or an explicit shape and dtype")
        nphys, hkv, P, d = shape
        for t in (self.page_table, self.seq_lens):
            if t.dtype != torch.int32:
                raise ValueError("page_table and seq_lens must be int32")
        B, max_pages = self.page_table.shape
        return hs_kv_cache(_ptr(self.k_pool), _ptr(self.v_pool), _ptr(self.page_table),
                           _ptr(self.seq_lens), B, hkv, d, P, max_pages, nphys,
                           int(self.max_seq_len), HS_F32 if dt == torch.float32 else HS_BF16)


@dataclass
class Summaries:
    """A summary table: mean -> float32 [B][Hkv][max_blocks][d];
    minmax -> cache dtype [B][Hkv][max_blocks][2][d]."""
    data: torch.Tensor
    kind: str
    block_size: int

    @property
    def max_blocks(self) -> int:
        return self.data.shape[2]

    def struct(self) -> hs_summaries:
        return hs_summaries(_ptr(self.data), KIND[self.kind], self.block_size, self.max_blocks)

    @staticmethod
    def empty(kv: KVCache, kind: str, block_size: int, device=None) -> "Summaries":
        s = kv.struct()
        nb = -(-kv.max_seq_len // block_size)
        dev = device or kv.page_table.device
        dt = kv.k_pool.dtype if kv.k_pool is not None else kv.dtype
        if kind == "mean":
            t = torch.empty((s.batch, s.num_kv_heads, nb, s.head_dim), dtype=torch.float32,
                            device=dev)
        else:
            t = torch.empty((s.batch, s.num_kv_heads, nb, 2, s.head_dim), dtype=dt, device=dev)
        return Summaries(t, kind, block_size)


# ------------------------------------------------------------ entry points
def hs_select_workspace_size(kv: KVCache, fine: Summaries, num_q_heads: int, top_k: int,
                             window: int, max_selected: int, coarse: Optional[Summaries] = None,
                             top_k_coarse: int = 0, top_k_ratio: float = 0.0,
                             forced: Optional[torch.Tensor] = None) -> int:
    p = _sel_params(num_q_heads, top_k, window, top_k_coarse, max_selected, top_k_ratio, forced)
    n = ctypes.c_size_t(0)
    ks, fs = kv.struct(), fine.struct()
    cs = coarse.struct() if coarse is not None else None
    _check("hs_select_workspace_size",
           lib().hs_select_workspace_size(ctypes.byref(p), ctypes.byref(ks), ctypes.byref(fs),
                                          ctypes.byref(cs) if cs is not None else None,
                                          ctypes.byref(n)))
    return n.value


def hs_decode_workspace_size(kv: KVCache, num_q_heads: int, block_size: int,
                             max_selected: int) -> int:
    n = ctypes.c_size_t(0)
    ks = kv.struct()
    _check("hs_decode_workspace_size",
           lib().hs_decode_workspace_size(ctypes.byref(ks), num_q_heads, block_size, max_selected,
                                          ctypes.byref(n)))
    return n.value


def hs_build_summaries(kv: KVCache, out: Summaries, block_begin: int = 0, stream=None) -> None:
    ks, os_ = kv.struct(), out.struct()
    _check("hs_build_summaries",
           lib().hs_build_summaries(ctypes.byref(ks), block_begin, ctypes.byref(os_),
                                    _stream(stream)))


def hs_append_kv(kv: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, stream=None) -> None:
    """Write one token per sequence (k_new, v_new [B][Hkv][d] in the cache
    dtype) at position seq_lens[b] and advance kv.seq_lens on the device."""
    for t in (k_new, v_new):
        if t.dtype != kv.k_pool.dtype or not t.is_contiguous():
            raise ValueError("k_new / v_new must be contiguous and in the cache dtype")
    ks = kv.struct()
    _check("hs_append_kv", lib().hs_append_kv(ctypes.byref(ks), _ptr(k_new), _ptr(v_new),
                                              _ptr(kv.seq_lens), _stream(stream)))


def hs_select_tokens_workspace_size(kv: KVCache, num_q_heads: int, block_size: int,
                                    max_selected: int, top_k_tokens: int, window: int,
                                    max_tokens: int) -> int:
    n = ctypes.c_size_t(0)
    ks = kv.struct()
    _check("hs_select_tokens_workspace_size",
           lib().hs_select_tokens_workspace_size(ctypes.byref(ks), num_q_heads, block_size,
                                                 max_selected, top_k_tokens, window, max_tokens,
                                                 ctypes.byref(n)))
    return n.value


def hs_select_tokens(kv: KVCache, q: torch.Tensor, block_size: int, block_ids: torch.Tensor,
                     num_selected: torch.Tensor, top_k_tokens: int, window: int,
                     token_ids: torch.Tensor, num_tokens: torch.Tensor, workspace: torch.Tensor,
                     stream=None) -> None:
    """Token-level second stage: block_ids int32 [B][Hkv][max_selected] from
    hs_select_blocks; token_ids int32 [B][Hkv][max_tokens]; num_tokens int32
    [B][Hkv]. Attend with hs_sparse_decode(kv, q, 1, token_ids, num_tokens, ...)."""
    for t in (block_ids, num_selected, token_ids, num_tokens):
        if t.dtype != torch.int32:
            raise ValueError("ids and counts must be int32")
    ks = kv.struct()
    _check("hs_select_tokens",
           lib().hs_select_tokens(ctypes.byref(ks), _ptr(q), q.shape[1], block_size,
                                  _ptr(block_ids), _ptr(num_selected), block_ids.shape[-1],
                                  top_k_tokens, window, _ptr(token_ids), _ptr(num_tokens),
                                  token_ids.shape[-1], _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


@dataclass
class BlockCache:
    """LRU index of selected blocks: slot_block and slot_stamp int32
    [units][capacity], both -1 when empty."""
    slot_block: torch.Tensor
    slot_stamp: torch.Tensor

    @staticmethod
    def empty(units: int, capacity: int, device="cuda") -> "BlockCache":
        return BlockCache(torch.full((units, capacity), -1, dtype=torch.int32, device=device),
                          torch.full((units, capacity), -1, dtype=torch.int32, device=device))

    def struct(self) -> hs_block_cache:
        return hs_block_cache(_ptr(self.slot_block), _ptr(self.slot_stamp),
                              int(self.slot_block.shape[-1]))


def hs_block_cache_update(cache: BlockCache, step: int, block_ids: torch.Tensor,
                          num_selected: torch.Tensor, slot_of: torch.Tensor,
                          miss_blocks: torch.Tensor, stats: torch.Tensor, stream=None) -> None:
    """block_ids / slot_of / miss_blocks int32 [..][max_selected] with
    units rows; num_selected int32 [units]; stats int32 [units][3]."""
    for t in (cache.slot_block, cache.slot_stamp, block_ids, num_selected, slot_of, miss_blocks,
              stats):
        if t.dtype != torch.int32 or not t.is_contiguous():
            raise ValueError("block cache arrays must be contiguous int32")
    units = num_selected.numel()
    ms = block_ids.shape[-1]
    if cache.slot_block.numel() != units * cache.slot_block.shape[-1] or \
            block_ids.numel() != units * ms or slot_of.numel() != units * ms or \
            miss_blocks.numel() != units * ms or stats.numel() != units * 3:
        raise ValueError("block cache arrays do not match the number of units")
    cs = cache.struct()
    _check("hs_block_cache_update",
           lib().hs_block_cache_update(ctypes.byref(cs), units, step, _ptr(block_ids),
                                       _ptr(num_selected), ms, _ptr(slot_of), _ptr(miss_blocks),
                                       _ptr(stats), _stream(stream)))


def hs_select_blocks(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int, window: int,
                     block_ids: torch.Tensor, num_selected: torch.Tensor,
                     workspace: torch.Tensor, coarse: Optional[Summaries] = None,
                     top_k_coarse: int = 0, stream=None, top_k_ratio: float = 0.0,
                     forced: Optional[torch.Tensor] = None) -> None:
    """q [B][Hq][d] in the cache dtype; block_ids int32 [B][Hkv][max_selected];
    num_selected int32 [B][Hkv]; workspace a uint8 device tensor;
    top_k_ratio > 0 replaces top_k by max(1, int(nb_b * ratio)) per unit;
    forced: int32 [B][Hkv][cap] block ids unioned into the selection."""
    if block_ids.dtype != torch.int32 or num_selected.dtype != torch.int32:
        raise ValueError("block_ids and num_selected must be int32")
    p = _sel_params(q.shape[1], top_k, window, top_k_coarse, block_ids.shape[-1], top_k_ratio,
                    forced)
    ks, fs = kv.struct(), fine.struct()
    cs = coarse.struct() if coarse is not None else None
    _check("hs_select_blocks",
           lib().hs_select_blocks(ctypes.byref(p), ctypes.byref(ks), _ptr(q), ctypes.byref(fs),
                                  ctypes.byref(cs) if cs is not None else None, _ptr(block_ids),
                                  _ptr(num_selected), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


def hs_sparse_decode(kv: KVCache, q: torch.Tensor, block_size: int, block_ids: torch.Tensor,
                     num_selected: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                     scale: float = 0.0, stream=None) -> None:
    """out float32 [B][Hq][d]; scale 0 means 1/sqrt(d)."""
    if out.dtype != torch.float32:
        raise ValueError("out must be float32")
    ks = kv.struct()
    _check("hs_sparse_decode",
           lib().hs_sparse_decode(ctypes.byref(ks), _ptr(q), q.shape[1], float(scale), block_size,
                                  _ptr(block_ids), _ptr(num_selected), block_ids.shape[-1],
                                  _ptr(out), _ptr(workspace), workspace.numel(),
                                  _stream(stream)))


def hs_select_decode_workspace_size(kv: KVCache, fine: Summaries, num_q_heads: int, top_k: int,
                                    window: int, max_selected: int,
                                    coarse: Optional[Summaries] = None,
                                    top_k_coarse: int = 0, top_k_ratio: float = 0.0,
                                    forced: Optional[torch.Tensor] = None) -> int:
    p = _sel_params(num_q_heads, top_k, window, top_k_coarse, max_selected, top_k_ratio, forced)
    n = ctypes.c_size_t(0)
    ks, fs = kv.struct(), fine.struct()
    cs = coarse.struct() if coarse is not None else None
    _check("hs_select_decode_workspace_size",
           lib().hs_select_decode_workspace_size(ctypes.byref(p), ctypes.byref(ks),
                                                 ctypes.byref(fs),
                                                 ctypes.byref(cs) if cs is not None else None,
                                                 ctypes.byref(n)))
    return n.value


def _select_decode_args(kv, q, fine, top_k, window, block_ids, num_selected, out, workspace,
                        coarse, top_k_coarse, scale, stream, top_k_ratio=0.0, forced=None):
    if block_ids.dtype != torch.int32 or num_selected.dtype != torch.int32:
        raise ValueError("block_ids and num_selected must be int32")
    if out.dtype != torch.float32:
        raise ValueError("out must be float32")
    p = _sel_params(q.shape[1], top_k, window, top_k_coarse, block_ids.shape[-1], top_k_ratio,
                    forced)
    ks, fs = kv.struct(), fine.struct()
    cs = coarse.struct() if coarse is not None else None
    args = (ctypes.byref(p), ctypes.byref(ks), _ptr(q), ctypes.byref(fs),
            ctypes.byref(cs) if cs is not None else None, ctypes.c_float(scale),
            _ptr(block_ids), _ptr(num_selected), _ptr(out), _ptr(workspace), workspace.numel(),
            _stream(stream))
    keep = (p, ks, fs, cs, kv, q, fine, coarse, block_ids, num_selected, out, workspace, forced)
    return args, keep


def hs_select_decode(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int, window: int,
                     block_ids: torch.Tensor, num_selected: torch.Tensor, out: torch.Tensor,
                     workspace: torch.Tensor, coarse: Optional[Summaries] = None,
                     top_k_coarse: int = 0, scale: float = 0.0, stream=None,
                     top_k_ratio: float = 0.0, forced: Optional[torch.Tensor] = None) -> None:
    """hs_select_blocks then hs_sparse_decode (block size fine.block_size) in
    one launch; same arguments and outputs as those two calls."""
    args, _ = _select_decode_args(kv, q, fine, top_k, window, block_ids, num_selected, out,
                                  workspace, coarse, top_k_coarse, scale, stream, top_k_ratio,
                                  forced)
    _check("hs_select_decode", lib().hs_select_decode(*args))


def _decode_step_args(kv, q, fine, top_k, window, refresh_begin, block_ids, num_selected, out,
                      workspace, coarse, top_k_coarse, scale, stream, top_k_ratio=0.0,
                      forced=None):
    args, keep = _select_decode_args(kv, q, fine, top_k, window, block_ids, num_selected, out,
                                     workspace, coarse, top_k_coarse, scale, stream, top_k_ratio,
                                     forced)
    return args[:5] + (int(refresh_begin),) + args[5:], keep


def hs_decode_step(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int, window: int,
                   refresh_begin: int, block_ids: torch.Tensor, num_selected: torch.Tensor,
                   out: torch.Tensor, workspace: torch.Tensor, coarse: Optional[Summaries] = None,
                   top_k_coarse: int = 0, scale: float = 0.0, stream=None,
                   top_k_ratio: float = 0.0, forced: Optional[torch.Tensor] = None) -> None:
    """hs_build_summaries from refresh_begin on (each level), then
    hs_select_decode, in one launch for a single level; the workspace is
    that of hs_select_decode."""
    args, _ = _decode_step_args(kv, q, fine, top_k, window, refresh_begin, block_ids,
                                num_selected, out, workspace, coarse, top_k_coarse, scale, stream,
                                top_k_ratio, forced)
    _check("hs_decode_step", lib().hs_decode_step(*args))


def hs_step_status(workspace: torch.Tensor, stream=None) -> int:
    """Status word of a hs_select_decode / hs_decode_step workspace: 0, or
    HS_STEP_WAIT_EXPIRED (synchronises the stream)."""
    v = ctypes.c_int32(0)
    _check("hs_step_status", lib().hs_step_status(_ptr(workspace), workspace.numel(),
                                                  ctypes.byref(v), _stream(stream)))
    return v.value


NOALLOC_SCRATCH_BYTES = 16 << 20  # HS_NOALLOC_SCRATCH_BYTES


def hs_decode_step_noalloc(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int,
                           window: int, refresh_begin: int, block_ids: torch.Tensor,
                           num_selected: torch.Tensor, out: torch.Tensor,
                           coarse: Optional[Summaries] = None, top_k_coarse: int = 0,
                           scale: float = 0.0, stream=None, top_k_ratio: float = 0.0,
                           forced: Optional[torch.Tensor] = None) -> None:
    """hs_decode_step with the library's own device array as its workspace
    (no allocation by the library or here); calls that overlap on one GPU race."""
    if block_ids.dtype != torch.int32 or num_selected.dtype != torch.int32:
        raise ValueError("block_ids and num_selected must be int32")
    if out.dtype != torch.float32:
        raise ValueError("out must be float32")
    p = _sel_params(q.shape[1], top_k, window, top_k_coarse, block_ids.shape[-1], top_k_ratio,
                    forced)
    ks, fs = kv.struct(), fine.struct()
    cs = coarse.struct() if coarse is not None else None
    _check("hs_decode_step_noalloc",
           lib().hs_decode_step_noalloc(ctypes.byref(p), ctypes.byref(ks), _ptr(q),
                                        ctypes.byref(fs),
                                        ctypes.byref(cs) if cs is not None else None,
                                        int(refresh_begin), ctypes.c_float(scale),
                                        _ptr(block_ids), _ptr(num_selected), _ptr(out),
                                        _stream(stream)))


def hs_version() -> int:
    return lib().hs_version()


def workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled uint8 device buffer of at least nbytes (256-byte aligned
    by torch). Workspaces must be zero before their first use (they hold
    arrival counters that every call leaves at zero)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


class Prepared:
    """An entry point with its arguments marshalled once; calling it issues
    the C call on the given stream (for tight loops and graph capture). The
    tensors it points to must stay alive and in place."""

    def __init__(self, name: str, fn, args: tuple, keep: tuple):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != HS_OK:
            raise HsError(self.name, st)


def prepare_build_summaries(kv: KVCache, out: Summaries, block_begin: int, stream) -> Prepared:
    ks, os_ = kv.struct(), out.struct()
    return Prepared("hs_build_summaries", lib().hs_build_summaries,
                    (ctypes.byref(ks), block_begin, ctypes.byref(os_), _stream(stream)),
                    (ks, os_, kv, out))


def prepare_select_blocks(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int, window: int,
                          block_ids: torch.Tensor, num_selected: torch.Tensor,
                          workspace: torch.Tensor, stream, coarse: Optional[Summaries] = None,
                          top_k_coarse: int = 0) -> Prepared:
    p = _sel_params(q.shape[1], top_k, window, top_k_coarse, block_ids.shape[-1])
    ks, fs = kv.struct(), fine.struct()
    cs = coarse.struct() if coarse is not None else None
    args = (ctypes.byref(p), ctypes.byref(ks), _ptr(q), ctypes.byref(fs),
            ctypes.byref(cs) if cs is not None else None, _ptr(block_ids), _ptr(num_selected),
            _ptr(workspace), workspace.numel(), _stream(stream))
    return Prepared("hs_select_blocks", lib().hs_select_blocks, args,
                    (p, ks, fs, cs, kv, q, fine, coarse, block_ids, num_selected, workspace))


def prepare_sparse_decode(kv: KVCache, q: torch.Tensor, block_size: int, block_ids: torch.Tensor,
                          num_selected: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                          stream, scale: float = 0.0) -> Prepared:
    ks = kv.struct()
    args = (ctypes.byref(ks), _ptr(q), q.shape[1], ctypes.c_float(scale), block_size,
            _ptr(block_ids), _ptr(num_selected), block_ids.shape[-1], _ptr(out), _ptr(workspace),
            workspace.numel(), _stream(stream))
    return Prepared("hs_sparse_decode", lib().hs_sparse_decode, args,
                    (ks, kv, q, block_ids, num_selected, out, workspace))


def prepare_select_decode(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int, window: int,
                          block_ids: torch.Tensor, num_selected: torch.Tensor, out: torch.Tensor,
                          workspace: torch.Tensor, stream, coarse: Optional[Summaries] = None,
                          top_k_coarse: int = 0, scale: float = 0.0) -> Prepared:
    args, keep = _select_decode_args(kv, q, fine, top_k, window, block_ids, num_selected, out,
                                     workspace, coarse, top_k_coarse, scale, stream)
    return Prepared("hs_select_decode", lib().hs_select_decode, args, keep)


def prepare_decode_step(kv: KVCache, q: torch.Tensor, fine: Summaries, top_k: int, window: int,
                        refresh_begin: int, block_ids: torch.Tensor, num_selected: torch.Tensor,
                        out: torch.Tensor, workspace: torch.Tensor, stream,
                        coarse: Optional[Summaries] = None, top_k_coarse: int = 0,
                        scale: float = 0.0) -> Prepared:
    args, keep = _decode_step_args(kv, q, fine, top_k, window, refresh_begin, block_ids,
                                   num_selected, out, workspace, coarse, top_k_coarse, scale,
                                   stream)
    return Prepared("hs_decode_step", lib().hs_decode_step, args, keep)
