"""ctypes marshalling for libmsa (see include/msa.h for the meaning of every
argument).  Tensors must already live on the current HIP device in the dtype
and layout the C ABI states; outputs are allocated with torch when not given.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch  # loads the HIP runtime libmsa binds to (same soname), before libmsa

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK = 0
BLK = 128


class MSAError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func} failed with status {status}: {detail}")


class Dims(ctypes.Structure):
    _fields_ = [("G", ctypes.c_int32), ("Hg", ctypes.c_int32), ("D", ctypes.c_int32),
                ("n_idx", ctypes.c_int32), ("d_idx", ctypes.c_int32), ("blk", ctypes.c_int32)]

    @classmethod
    def make(cls, G, Hg, D=128, n_idx=4, d_idx=128, blk=BLK):
        return cls(G, Hg, D, n_idx, d_idx, blk)


class View(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("page_stride", ctypes.c_int64),
                ("group_stride", ctypes.c_int64), ("token_stride", ctypes.c_int64)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_DIMS = ctypes.POINTER(Dims)

_SIGS = {
    "msa_index_score": [_DIMS, _I32, _P, View, _P, _I32, _P, _P, _P, _I32, _P, _I32, _P],
    "msa_topk_blocks": [_DIMS, _I32, _P, _I32, _P, _I32, _P, _P],
    "msa_topk_blocks_paged": [_DIMS, _I32, _P, _I32, _P, _I32, _P, _P, _I32, _P, _P, _P],
    "msa_build_page_table": [_DIMS, _I32, _P, _I32, _P, _P, _I32, _P, _P],
    "msa_sparse_attn_decode": [_DIMS, _I32, _P, View, View, _P, _P, _I32, _P, ctypes.c_float,
                               _P, _P, _P],
    "msa_sparse_attn_decode_select": [_DIMS, _I32, _P, _I32, _I32, _P, _P, _I32, _P, View, View,
                                      _P, ctypes.c_float, _P, _P, _P, _P, _P],
    "msa_decode_step": [_DIMS, _I32, _P, View, _P, _I32, _P, _P, _P, _I32, _I32, _I32, _P, View,
                        View, ctypes.c_float, _P, _P, _P, _P, _P, _P, _P, _P, _I32, _P],
    "msa_prefill_workspace_size": [_DIMS, _I32, _I32, _I32, ctypes.POINTER(ctypes.c_size_t)],
    "msa_prefill_merged_workspace_size": [_DIMS, _I32, _I32, _I32, _I32,
                                          ctypes.POINTER(ctypes.c_size_t)],
    "msa_sparse_attn_prefill_merged": [_DIMS, _I32, _P, View, View, _P, _P, _I32, _P, _I32,
                                       ctypes.c_float, _I32, _P, ctypes.c_size_t, _P, _P, _P],
    "msa_sparse_attn_prefill": [_DIMS, _I32, _P, View, View, _P, _P, _I32, _P, _I32,
                                ctypes.c_float, _P, ctypes.c_size_t, _P, _P, _P],
    "msa_sparse_attn_prefill_noalloc": [_DIMS, _I32, _P, View, View, _P, _P, _I32, _P, _I32,
                                        ctypes.c_float, _P, _P, _P],
    "msa_lse_merge": [_I32, _I32, _I32, _I32, _P, _P, _P, _P, _P],
    "msa_gather_pages": [_DIMS, _I32, _P, _I32, View, View, _P, _P, _P, _P],
    "msa_peak_stream_read": [_P, ctypes.c_size_t, _P, _P],
    "msa_peak_stream_write": [_P, ctypes.c_size_t, ctypes.c_uint32, _P],
    "msa_peak_row_copy": [_P, _P, _P, _P, ctypes.c_int64, _I32, _I32, _P],
    "msa_peak_mfma_bf16": [_I32, _P, ctypes.POINTER(ctypes.c_double), _P],
    "msa_peak_mfma_bf16_random": [_I32, _P, ctypes.POINTER(ctypes.c_double), _P],
}

_lib = None


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libmsa.so (built in-tree); raises when it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_09_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(lib, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        for name in ("msa_version", "msa_last_error"):
            getattr(lib, name).argtypes = []
            getattr(lib, name).restype = ctypes.c_char_p
        lib.msa_status_string.argtypes = [ctypes.c_int]
        lib.msa_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def msa_version() -> str:
    return load().msa_version().decode()


def _check(status: int, func: str):
    if status != MSA_OK:
        raise MSAError(status, func, load().msa_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _need(t: torch.Tensor, dtype, name, contiguous=False):
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise TypeError(f"{name}: must be a device tensor")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def view_of(cache: torch.Tensor, host_ok: bool = False) -> View:
    """C view of a 4-d bf16 cache tensor indexed [page][group][token][dim]
    (any strides, dim stride 1).  With host_ok, a pinned host tensor is accepted
    as well: pinned host memory is mapped into the device's address space, so
    the attention kernels read the selected pages from it directly."""
    if host_ok and not cache.is_cuda:
        if cache.dtype != torch.bfloat16:
            raise TypeError(f"cache: expected torch.bfloat16, got {cache.dtype}")
        if not cache.is_pinned():
            raise TypeError("cache: a host cache must be pinned (pin_memory) to be device-mapped")
    else:
        _need(cache, torch.bfloat16, "cache")
    if cache.dim() != 4 or cache.stride(3) != 1:
        raise ValueError("cache must be 4-d [page][group][token][dim] with unit dim stride")
    return View(cache.data_ptr(), cache.stride(0), cache.stride(1), cache.stride(2))


def _i32(t, name):
    if t is None:
        return None
    _need(t, torch.int32, name)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def msa_index_score(dims: Dims, q_idx, k_idx, block_table, row_pos, score_stride,
                    row_req=None, blk_lo=None, num_reqs=None, scores=None, stream=None):
    _need(q_idx, torch.bfloat16, "q_idx", True)
    rows = q_idx.shape[0]
    _i32(block_table, "block_table"), _i32(row_pos, "row_pos")
    _i32(row_req, "row_req"), _i32(blk_lo, "blk_lo")
    if scores is None:
        scores = torch.empty((rows, dims.G, score_stride), dtype=torch.float32,
                             device=q_idx.device)
    nreq = int(num_reqs if num_reqs is not None else block_table.shape[0])
    _check(load().msa_index_score(ctypes.byref(dims), rows, _ptr(q_idx),
                                  view_of(k_idx), _ptr(block_table), block_table.shape[1],
                                  _ptr(row_req), _ptr(row_pos), _ptr(blk_lo), nreq,
                                  _ptr(scores), score_stride, _stream(stream)),
           "msa_index_score")
    return scores


def msa_topk_blocks(dims: Dims, scores, row_pos, k, sel=None, stream=None):
    _need(scores, torch.float32, "scores", True)
    rows, _, score_stride = scores.shape
    _i32(row_pos, "row_pos")
    if sel is None:
        sel = torch.empty((rows, dims.G, k + 1), dtype=torch.int32, device=scores.device)
    _check(load().msa_topk_blocks(ctypes.byref(dims), rows, _ptr(scores), score_stride,
                                  _ptr(row_pos), k, _ptr(sel), _stream(stream)),
           "msa_topk_blocks")
    return sel


def msa_topk_blocks_paged(dims: Dims, scores, row_pos, k, block_table, row_req=None, sel=None,
                          page_table=None, stream=None):
    """msa_topk_blocks and msa_build_page_table in one launch; returns (sel, page_table)."""
    _need(scores, torch.float32, "scores", True)
    _i32(row_pos, "row_pos"), _i32(block_table, "block_table"), _i32(row_req, "row_req")
    rows, _, score_stride = scores.shape
    if sel is None:
        sel = torch.empty((rows, dims.G, k + 1), dtype=torch.int32, device=scores.device)
    if page_table is None:
        page_table = torch.empty_like(sel)
    _check(load().msa_topk_blocks_paged(ctypes.byref(dims), rows, _ptr(scores), score_stride,
                                        _ptr(row_pos), k, _ptr(row_req), _ptr(block_table),
                                        block_table.shape[1], _ptr(sel), _ptr(page_table),
                                        _stream(stream)),
           "msa_topk_blocks_paged")
    return sel, page_table


def msa_build_page_table(dims: Dims, sel, block_table, row_req=None, page_table=None,
                         stream=None):
    _i32(sel, "sel"), _i32(block_table, "block_table"), _i32(row_req, "row_req")
    rows, _, nslot = sel.shape
    if page_table is None:
        page_table = torch.empty_like(sel)
    _check(load().msa_build_page_table(ctypes.byref(dims), rows, _ptr(sel), nslot,
                                       _ptr(row_req), _ptr(block_table), block_table.shape[1],
                                       _ptr(page_table), _stream(stream)),
           "msa_build_page_table")
    return page_table


def empty_lse_part(rows, H, nslot, device) -> torch.Tensor:
    """Partial LSEs as the C ABI lays them out, [rows][nslot][H] in memory,
    returned as the view indexed [row][head][slot] (the order of o_part)."""
    return torch.empty((rows, nslot, H), dtype=torch.float32, device=device).permute(0, 2, 1)


def _need_lse(lse_part, shape=None):
    """lse_part must be a float32 device view [rows][H][nslot] over memory laid
    out [rows][nslot][H] (as empty_lse_part makes it)."""
    if lse_part.dtype != torch.float32 or not lse_part.is_cuda:
        raise TypeError("lse_part: expected a float32 device tensor")
    if lse_part.dim() != 3 or not lse_part.permute(0, 2, 1).is_contiguous():
        raise ValueError("lse_part must be a [rows][H][nslot] view of [rows][nslot][H] memory "
                         "(see empty_lse_part)")
    if shape is not None and tuple(lse_part.shape) != tuple(shape):
        raise ValueError(f"lse_part: shape {tuple(lse_part.shape)}, expected {tuple(shape)}")


def _attn_out(q, nslot, o_part, lse_part):
    rows, H, D = q.shape
    if o_part is None:
        o_part = torch.empty((rows, H, nslot, D), dtype=torch.bfloat16, device=q.device)
    if lse_part is None:
        lse_part = empty_lse_part(rows, H, nslot, q.device)
    _need_lse(lse_part, (rows, H, nslot))
    return o_part, lse_part


def msa_sparse_attn_decode(dims: Dims, q, k_cache, v_cache, sel, page_table, row_pos,
                           sm_scale=None, o_part=None, lse_part=None, stream=None):
    _need(q, torch.bfloat16, "q", True)
    _i32(sel, "sel"), _i32(page_table, "page_table"), _i32(row_pos, "row_pos")
    nslot = sel.shape[2]
    o_part, lse_part = _attn_out(q, nslot, o_part, lse_part)
    scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dims.D))
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_sparse_attn_decode(ctypes.byref(dims), q.shape[0], _ptr(q), kv[0], kv[1],
                                         _ptr(sel), _ptr(page_table), nslot, _ptr(row_pos), scale,
                                         _ptr(o_part), _ptr(lse_part), _stream(stream)),
           "msa_sparse_attn_decode")
    return o_part, lse_part


def msa_sparse_attn_decode_select(dims: Dims, scores, k, block_table, q, k_cache, v_cache,
                                  row_pos, row_req=None, sm_scale=None, sel=None,
                                  page_table=None, o_part=None, lse_part=None, stream=None):
    """msa_topk_blocks_paged and msa_sparse_attn_decode in one launch; returns
    (sel, page_table, o_part, lse_part)."""
    _need(scores, torch.float32, "scores", True)
    _need(q, torch.bfloat16, "q", True)
    _i32(row_pos, "row_pos"), _i32(block_table, "block_table"), _i32(row_req, "row_req")
    rows, _, score_stride = scores.shape
    if sel is None:
        sel = torch.empty((rows, dims.G, k + 1), dtype=torch.int32, device=scores.device)
    if page_table is None:
        page_table = torch.empty_like(sel)
    _i32(sel, "sel"), _i32(page_table, "page_table")
    o_part, lse_part = _attn_out(q, k + 1, o_part, lse_part)
    scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dims.D))
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_sparse_attn_decode_select(
        ctypes.byref(dims), rows, _ptr(scores), score_stride, k, _ptr(row_req),
        _ptr(block_table), block_table.shape[1], _ptr(q), kv[0], kv[1], _ptr(row_pos), scale,
        _ptr(sel), _ptr(page_table), _ptr(o_part), _ptr(lse_part), _stream(stream)),
        "msa_sparse_attn_decode_select")
    return sel, page_table, o_part, lse_part


MSA_STEP_AUTO, MSA_STEP_ONE_LAUNCH, MSA_STEP_SEPARATE = 0, 1, 2


def decode_step_sync_words(rows, G) -> int:
    """Length of msa_decode_step's int32 sync array (MSA_DECODE_STEP_SYNC_WORDS)."""
    return 4 + 2 * rows * G


def msa_decode_step(dims: Dims, q_idx, k_idx, block_table, row_pos, score_stride, k, q,
                    k_cache, v_cache, row_req=None, blk_lo=None, num_reqs=None, sm_scale=None,
                    mode=MSA_STEP_AUTO, sync=None, scores=None, sel=None, page_table=None,
                    o_part=None, lse_part=None, o=None, lse=None, stream=None):
    """The whole decode step (scores, selection, page table, slot partials and
    their merge); returns (scores, sel, page_table, o_part, lse_part, o, lse).
    sync: int32 device tensor of decode_step_sync_words(rows, G) zeros (left zero
    by every call), used by MSA_STEP_ONE_LAUNCH; when None in that mode a zeroed
    one is allocated for the call (pass a persistent one to avoid that)."""
    _need(q_idx, torch.bfloat16, "q_idx", True)
    _need(q, torch.bfloat16, "q", True)
    _i32(block_table, "block_table"), _i32(row_pos, "row_pos")
    _i32(row_req, "row_req"), _i32(blk_lo, "blk_lo")
    rows, H, D = q.shape
    dev = q.device
    if scores is None:
        scores = torch.empty((rows, dims.G, score_stride), dtype=torch.float32, device=dev)
    if sel is None:
        sel = torch.empty((rows, dims.G, k + 1), dtype=torch.int32, device=dev)
    if page_table is None:
        page_table = torch.empty_like(sel)
    _need(scores, torch.float32, "scores", True)
    _i32(sel, "sel"), _i32(page_table, "page_table")
    o_part, lse_part = _attn_out(q, k + 1, o_part, lse_part)
    if o is None:
        o = torch.empty((rows, H, D), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((rows, H), dtype=torch.float32, device=dev)
    _need(o, torch.bfloat16, "o", True)
    _need(lse, torch.float32, "lse", True)
    if sync is None and mode == MSA_STEP_ONE_LAUNCH:
        sync = torch.zeros(decode_step_sync_words(rows, dims.G), dtype=torch.int32, device=dev)
    if sync is not None:
        _i32(sync, "sync")
        if sync.numel() < decode_step_sync_words(rows, dims.G):
            raise ValueError("sync: too short (decode_step_sync_words)")
    nreq = int(num_reqs if num_reqs is not None else block_table.shape[0])
    scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dims.D))
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_decode_step(
        ctypes.byref(dims), rows, _ptr(q_idx), view_of(k_idx), _ptr(block_table),
        block_table.shape[1], _ptr(row_req), _ptr(row_pos), _ptr(blk_lo), nreq, score_stride, k,
        _ptr(q), kv[0], kv[1], scale, _ptr(scores), _ptr(sel), _ptr(page_table), _ptr(o_part),
        _ptr(lse_part), _ptr(o), _ptr(lse), _ptr(sync), int(mode), _stream(stream)),
        "msa_decode_step")
    return scores, sel, page_table, o_part, lse_part, o, lse


def msa_prefill_merged_workspace_size(dims: Dims, rows, nslot, num_pages, slab_rows=0) -> int:
    n = ctypes.c_size_t(0)
    _check(load().msa_prefill_merged_workspace_size(ctypes.byref(dims), rows, nslot, num_pages,
                                                    slab_rows, ctypes.byref(n)),
           "msa_prefill_merged_workspace_size")
    return n.value


def msa_sparse_attn_prefill_merged(dims: Dims, q, k_cache, v_cache, sel, page_table, row_pos,
                                   num_pages, sm_scale=None, slab_rows=0, workspace=None, o=None,
                                   lse=None, stream=None):
    """Block-major prefill attention and its merge by query slabs; returns (o, lse)."""
    _need(q, torch.bfloat16, "q", True)
    _i32(sel, "sel"), _i32(page_table, "page_table"), _i32(row_pos, "row_pos")
    rows, H, D = q.shape
    nslot = sel.shape[2]
    need = msa_prefill_merged_workspace_size(dims, rows, nslot, num_pages, slab_rows)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if o is None:
        o = torch.empty((rows, H, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((rows, H), dtype=torch.float32, device=q.device)
    scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dims.D))
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_sparse_attn_prefill_merged(
        ctypes.byref(dims), rows, _ptr(q), kv[0], kv[1], _ptr(sel), _ptr(page_table), nslot,
        _ptr(row_pos), num_pages, scale, int(slab_rows), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(o), _ptr(lse), _stream(stream)),
        "msa_sparse_attn_prefill_merged")
    return o, lse


def msa_prefill_workspace_size(dims: Dims, rows, nslot, num_pages) -> int:
    n = ctypes.c_size_t(0)
    _check(load().msa_prefill_workspace_size(ctypes.byref(dims), rows, nslot, num_pages,
                                             ctypes.byref(n)), "msa_prefill_workspace_size")
    return n.value


def msa_sparse_attn_prefill(dims: Dims, q, k_cache, v_cache, sel, page_table, row_pos,
                            num_pages, sm_scale=None, workspace=None, o_part=None,
                            lse_part=None, stream=None):
    _need(q, torch.bfloat16, "q", True)
    _i32(sel, "sel"), _i32(page_table, "page_table"), _i32(row_pos, "row_pos")
    rows, nslot = q.shape[0], sel.shape[2]
    o_part, lse_part = _attn_out(q, nslot, o_part, lse_part)
    need = msa_prefill_workspace_size(dims, rows, nslot, num_pages)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dims.D))
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_sparse_attn_prefill(ctypes.byref(dims), rows, _ptr(q), kv[0], kv[1],
                                          _ptr(sel), _ptr(page_table), nslot, _ptr(row_pos),
                                          num_pages,
                                          scale, _ptr(workspace), workspace.numel(),
                                          _ptr(o_part), _ptr(lse_part), _stream(stream)),
           "msa_sparse_attn_prefill")
    return o_part, lse_part


def msa_sparse_attn_prefill_noalloc(dims: Dims, q, k_cache, v_cache, sel, page_table, row_pos,
                                    num_pages, sm_scale=None, o_part=None, lse_part=None,
                                    stream=None):
    """msa_sparse_attn_prefill without a workspace: the library's static device
    scratch serves instead (for callers that cannot allocate; pass o_part and
    lse_part to allocate nothing on this side either)."""
    _need(q, torch.bfloat16, "q", True)
    _i32(sel, "sel"), _i32(page_table, "page_table"), _i32(row_pos, "row_pos")
    rows, nslot = q.shape[0], sel.shape[2]
    o_part, lse_part = _attn_out(q, nslot, o_part, lse_part)
    scale = float(sm_scale if sm_scale is not None else 1.0 / math.sqrt(dims.D))
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_sparse_attn_prefill_noalloc(ctypes.byref(dims), rows, _ptr(q), kv[0],
                                                  kv[1], _ptr(sel), _ptr(page_table), nslot,
                                                  _ptr(row_pos), num_pages, scale, _ptr(o_part),
                                                  _ptr(lse_part), _stream(stream)),
           "msa_sparse_attn_prefill_noalloc")
    return o_part, lse_part


def msa_gather_pages(dims: Dims, page_table, k_cache, v_cache, dst_k=None, dst_v=None,
                     dst_page_table=None, stream=None):
    """Copy the pages a page table names (K and V, from device or pinned host
    caches) into a compact device pool; returns (k_pool, v_pool, pool_page_table)
    shaped so that msa_sparse_attn_decode can take them as its caches."""
    _i32(page_table, "page_table")
    rows, G, nslot = page_table.shape
    units = rows * G * nslot
    dev = page_table.device
    if dst_k is None:
        dst_k = torch.empty((units, 128, dims.D), dtype=torch.bfloat16, device=dev)
    if dst_v is None:
        dst_v = torch.empty((units, 128, dims.D), dtype=torch.bfloat16, device=dev)
    if dst_page_table is None:
        dst_page_table = torch.empty_like(page_table)
    _need(dst_k, torch.bfloat16, "dst_k", True)
    _need(dst_v, torch.bfloat16, "dst_v", True)
    kv = view_of(k_cache, host_ok=True), view_of(v_cache, host_ok=True)
    _check(load().msa_gather_pages(ctypes.byref(dims), rows, _ptr(page_table), nslot, kv[0], kv[1],
                                   _ptr(dst_k), _ptr(dst_v), _ptr(dst_page_table),
                                   _stream(stream)), "msa_gather_pages")
    # one 128-token page per slot; the group is part of the slot, hence stride 0
    k_pool = dst_k.view(units, 1, 128, dims.D).expand(units, G, 128, dims.D)
    v_pool = dst_v.view(units, 1, 128, dims.D).expand(units, G, 128, dims.D)
    return k_pool, v_pool, dst_page_table


def msa_lse_merge(o_part, lse_part, o=None, lse=None, stream=None):
    _need(o_part, torch.bfloat16, "o_part", True)
    rows, H, nslot, D = o_part.shape
    _need_lse(lse_part, (rows, H, nslot))
    if o is None:
        o = torch.empty((rows, H, D), dtype=torch.bfloat16, device=o_part.device)
    if lse is None:
        lse = torch.empty((rows, H), dtype=torch.float32, device=o_part.device)
    _check(load().msa_lse_merge(rows, H, nslot, D, _ptr(o_part), _ptr(lse_part), _ptr(o),
                                _ptr(lse), _stream(stream)), "msa_lse_merge")
    return o, lse


def msa_peak_stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None):
    """Launch the streaming-read probe over every byte of `buf` (include/msa_peaks.h)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _need(sink, torch.float32, "sink")
    _check(load().msa_peak_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                       _stream(stream)), "msa_peak_stream_read")


def msa_peak_stream_write(buf: torch.Tensor, tag: int = 0, stream=None):
    """Launch the streaming-write probe over every byte of `buf` (include/msa_peaks.h)."""
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous device tensor")
    _check(load().msa_peak_stream_write(_ptr(buf), buf.numel() * buf.element_size(),
                                        int(tag) & 0xffffffff, _stream(stream)),
           "msa_peak_stream_write")


def msa_peak_row_copy(src: torch.Tensor, dst: torch.Tensor, load_idx: torch.Tensor,
                      store_idx: torch.Tensor, tiles_per_wg: int = 64, load_layout: int = 1,
                      stream=None):
    """Launch the row gather-scatter probe (include/msa_peaks.h): destination row
    store_idx[i] of dst gets source row load_idx[i] of src, rows of 256 bytes."""
    for t, name in ((src, "src"), (dst, "dst")):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if (t.numel() * t.element_size()) % 256:
            raise ValueError(f"{name} must hold whole 256-byte rows")
    _i32(load_idx, "load_idx"), _i32(store_idx, "store_idx")
    if load_idx.numel() != store_idx.numel():
        raise ValueError("load_idx and store_idx must have the same length")
    _check(load().msa_peak_row_copy(_ptr(src), _ptr(dst), _ptr(load_idx), _ptr(store_idx),
                                    ctypes.c_int64(load_idx.numel()), int(tiles_per_wg),
                                    int(load_layout), _stream(stream)), "msa_peak_row_copy")


def msa_peak_mfma_bf16(iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the bf16 matrix-core loop probe; returns the FLOPs it performs."""
    _need(sink, torch.float32, "sink")
    flops = ctypes.c_double(0.0)
    _check(load().msa_peak_mfma_bf16(iters, _ptr(sink), ctypes.byref(flops), _stream(stream)),
           "msa_peak_mfma_bf16")
    return flops.value


def msa_peak_mfma_bf16_random(iters: int, sink: torch.Tensor, stream=None) -> float:
    """Launch the bf16 matrix-core loop probe on pseudo-random operands; returns its FLOPs."""
    _need(sink, torch.float32, "sink")
    flops = ctypes.c_double(0.0)
    _check(load().msa_peak_mfma_bf16_random(iters, _ptr(sink), ctypes.byref(flops),
                                            _stream(stream)), "msa_peak_mfma_bf16_random")
    return flops.value
