"""CPU oracle for the MiniMax Sparse Attention (MSA) hot path.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only code allowed to import this package.  It shares
nothing with the GPU library and never imports it.

The arithmetic lives in ``msa_oracle.c`` (plain C, fp64 accumulation, loops in
the order of the definition); this module only builds it with gcc, loads it with
ctypes and marshals NumPy arrays.  bf16 tensors travel as their uint16 bit
patterns.  Each wrapper names the passage of the pages that defines the step in
the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_LIB = os.path.join(_HERE, "libmsa_oracle.so")
BLK = 128

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64


_FLAGS = ["-O3", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
          # strict IEEE: no fast-math, no contraction into FMAs, so every
          # build (portable or host-tuned) computes bit-identical results
          "-ffp-contract=off", "-fno-fast-math"]


def _compile(out: str, extra=()) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", *_FLAGS, *extra, _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile the portable oracle with gcc (-O3, OpenMP, strict IEEE)."""
    if force or not os.path.exists(_LIB):
        _compile(_LIB)
    return _LIB


def build_native(out_dir: str) -> str:
    """Compile a copy tuned for the host it runs on (-march=native) into
    out_dir, for timing the oracle as a CPU baseline on that host; it computes
    exactly what the portable build does.  Built where it runs, because a
    -march=native binary may not execute on another CPU."""
    os.makedirs(out_dir, exist_ok=True)
    return _compile(os.path.join(out_dir, "libmsa_oracle_native.so"), ["-march=native"])


_lib_handle = None


def use_library(path: str) -> None:
    """Route every oracle call through the library at path (e.g. build_native's)."""
    global _lib_handle
    _lib_handle = _bind(ctypes.CDLL(path))


def _bind(lib):
    lib.orc_index_score.argtypes = [_i32, _i32, _i32, _i32, _u16p, _u16p, _i64, _i64, _i64,
                                    _i32p, _i32, _i32p, _i32p, _i32p, _i32, _f64p]
    lib.orc_topk.argtypes = [_i32, _i32, _f32p, _i32, _i32p, _i32, _i32p]
    lib.orc_page_table.argtypes = [_i32, _i32, _i32, _i32p, _i32p, _i32p, _i32, _i32p]
    attn_args = [_i32, _i32, _i32, _i32, _u16p, _u16p, _i64, _i64, _i64,
                 _u16p, _i64, _i64, _i64, _i32p, _i32p, _i32, _i32p, ctypes.c_double,
                 _f64p, _f64p]
    lib.orc_attn.argtypes = attn_args
    lib.orc_attn_partials.argtypes = attn_args
    lib.orc_lse_merge.argtypes = [_i32, _i32, _i32, _i32, _f64p, _f64p, _f64p, _f64p]
    for f in (lib.orc_index_score, lib.orc_topk, lib.orc_page_table, lib.orc_attn,
              lib.orc_attn_partials, lib.orc_lse_merge):
        f.restype = None
    return lib


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib_handle = _bind(ctypes.CDLL(_LIB))
    return _lib_handle


def num_threads() -> int:
    """Threads the OpenMP runtime of the oracle uses (honours OMP_NUM_THREADS)."""
    v = os.environ.get("OMP_NUM_THREADS")
    if v:
        return int(v)
    return len(os.sched_getaffinity(0))


# ----------------------------------------------------------------------------- marshalling
def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _c_i32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _view(pool: np.ndarray):
    """A 4-d [page][group][token][dim] uint16 array (any strides, dim stride 1)."""
    assert pool.dtype == np.uint16 and pool.ndim == 4
    st = [s // 2 for s in pool.strides]
    assert pool.strides[3] == 2, "innermost dimension must be contiguous"
    return pool.ctypes.data_as(_u16p), st[0], st[1], st[2]


# ----------------------------------------------------------------------------- steps
def index_score(q_idx, k_idx_pool, block_table, row_pos, nb, row_req=None, blk_lo=None):
    """Block scores, fp64 [rows][G][nb] (see orc_index_score)."""
    q_idx = np.ascontiguousarray(q_idx, dtype=np.uint16)
    rows, G, n_idx, d_idx = q_idx.shape
    bt = _c_i32(block_table)
    rp, rr, lo = _c_i32(row_pos), _c_i32(row_req), _c_i32(blk_lo)
    out = np.empty((rows, G, nb), dtype=np.float64)
    kp, ps, gs, ts = _view(k_idx_pool)
    _lib().orc_index_score(rows, G, n_idx, d_idx, _ptr(q_idx, _u16p), kp, ps, gs, ts,
                           _ptr(bt, _i32p), bt.shape[1], _ptr(rr, _i32p), _ptr(rp, _i32p),
                           _ptr(lo, _i32p), nb, _ptr(out, _f64p))
    return out


def topk(scores_f32, row_pos, k):
    """Selected blocks int32 [rows][G][k+1] from fp32 scores (see orc_topk)."""
    s = np.ascontiguousarray(scores_f32, dtype=np.float32)
    rows, G, stride = s.shape
    rp = _c_i32(row_pos)
    sel = np.empty((rows, G, k + 1), dtype=np.int32)
    _lib().orc_topk(rows, G, _ptr(s, _f32p), stride, _ptr(rp, _i32p), k, _ptr(sel, _i32p))
    return sel


def page_table(sel, block_table, row_req=None):
    sel = _c_i32(sel)
    rows, G, nslot = sel.shape
    bt, rr = _c_i32(block_table), _c_i32(row_req)
    pt = np.empty_like(sel)
    _lib().orc_page_table(rows, G, nslot, _ptr(sel, _i32p), _ptr(rr, _i32p), _ptr(bt, _i32p),
                          bt.shape[1], _ptr(pt, _i32p))
    return pt


def _attn_common(fn, q, k_pool, v_pool, sel, pt, row_pos, sm_scale, partial):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    rows, H, D = q.shape
    sel, pt, rp = _c_i32(sel), _c_i32(pt), _c_i32(row_pos)
    G, nslot = sel.shape[1], sel.shape[2]
    Hg = H // G
    kp, kps, kgs, kts = _view(k_pool)
    vp, vps, vgs, vts = _view(v_pool)
    if partial:
        o = np.empty((rows, H, nslot, D), dtype=np.float64)
        lse = np.empty((rows, H, nslot), dtype=np.float64)
    else:
        o = np.empty((rows, H, D), dtype=np.float64)
        lse = np.empty((rows, H), dtype=np.float64)
    fn(rows, G, Hg, D, _ptr(q, _u16p), kp, kps, kgs, kts, vp, vps, vgs, vts,
       _ptr(sel, _i32p), _ptr(pt, _i32p), nslot, _ptr(rp, _i32p), float(sm_scale),
       _ptr(o, _f64p), _ptr(lse, _f64p))
    return o, lse


def attn(q, k_pool, v_pool, sel, pt, row_pos, sm_scale):
    """Direct softmax attention over the union of selected tokens: (o, lse) fp64."""
    return _attn_common(_lib().orc_attn, q, k_pool, v_pool, sel, pt, row_pos, sm_scale, False)


def attn_partials(q, k_pool, v_pool, sel, pt, row_pos, sm_scale):
    """Per-(row, head, slot) normalised partials: (o_part, lse_part) fp64."""
    return _attn_common(_lib().orc_attn_partials, q, k_pool, v_pool, sel, pt, row_pos,
                        sm_scale, True)


def lse_merge(o_part, lse_part):
    o_part = np.ascontiguousarray(o_part, dtype=np.float64)
    lse_part = np.ascontiguousarray(lse_part, dtype=np.float64)
    rows, H, nslot, D = o_part.shape
    o = np.empty((rows, H, D), dtype=np.float64)
    lse = np.empty((rows, H), dtype=np.float64)
    _lib().orc_lse_merge(rows, H, nslot, D, _ptr(o_part, _f64p), _ptr(lse_part, _f64p),
                         _ptr(o, _f64p), _ptr(lse, _f64p))
    return o, lse


# ----------------------------------------------------------------------------- whole path
def decode_path(q_idx, k_idx_pool, q, k_pool, v_pool, block_table, row_pos, k, nb,
                sm_scale, row_req=None, blk_lo=None):
    """Scores -> fp32 -> top-k -> page table -> attention, as one oracle pass."""
    scores = index_score(q_idx, k_idx_pool, block_table, row_pos, nb, row_req, blk_lo)
    s32 = scores.astype(np.float32)
    sel = topk(s32, row_pos, k)
    pt = page_table(sel, block_table, row_req)
    o, lse = attn(q, k_pool, v_pool, sel, pt, row_pos, sm_scale)
    return dict(scores=scores, scores_f32=s32, sel=sel, pt=pt, o=o, lse=lse)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(
        np.float64)
