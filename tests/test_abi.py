"""CPU checks of the C boundary: libmsa loads, exports every entry point that
include/msa.h declares, and rejects bad arguments with the right status before
launching anything (all cases below fail validation, so no GPU is touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")
HEADERS = [os.path.join(ROOT, "include", f) for f in sorted(os.listdir(os.path.join(ROOT, "include")))
           if f.endswith(".h")]

MSA_OK, MSA_ERR_NULL, MSA_ERR_INVALID, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE = 0, 1, 2, 3, 4


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_09_amd import binding
    if not os.path.exists(binding.lib_path()):
        from block_sparse_attention_09_amd import build
        build.build()
    return binding.load()


def declared_functions(headers=None):
    text = "".join(open(h).read() for h in (headers or HEADERS))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z_]+)\s*\(", text)))


def test_header_declares_the_six_calls():
    names = declared_functions([HEADER])
    for f in ("msa_index_score", "msa_topk_blocks", "msa_build_page_table",
              "msa_sparse_attn_decode", "msa_sparse_attn_prefill", "msa_lse_merge"):
        assert f in names


def test_every_declared_symbol_is_exported(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_version_and_status_strings(lib):
    from block_sparse_attention_09_amd import binding
    assert "libmsa" in binding.msa_version()
    for s in range(6):
        assert lib.msa_status_string(s)
    assert lib.msa_status_string(99) == b"unknown msa_status_t"


def _dims(**kw):
    from block_sparse_attention_09_amd.binding import Dims
    d = dict(G=8, Hg=8, D=128, n_idx=4, d_idx=128, blk=128)
    d.update(kw)
    return Dims(**d)


FAKE = ctypes.c_void_p(0x10000)      # aligned, never dereferenced: every case fails validation
MISALIGNED = ctypes.c_void_p(0x10002)


def _view(base=FAKE, ps=8 * 128 * 128, gs=128 * 128, ts=128):
    from block_sparse_attention_09_amd.binding import View
    return View(base.value, ps, gs, ts)


def _score(lib, dims, **kw):
    a = dict(rows=1, q=FAKE, kv=_view(), bt=FAKE, bts=4, rr=None, rp=FAKE, lo=None, nreq=1,
             out=FAKE, ss=4)
    a.update(kw)
    st = lib.msa_index_score(ctypes.byref(dims) if dims is not None else None, a["rows"], a["q"],
                             a["kv"], a["bt"], a["bts"], a["rr"], a["rp"], a["lo"], a["nreq"],
                             a["out"], a["ss"], None)
    return st


def test_index_score_validation(lib):
    assert _score(lib, None) == MSA_ERR_NULL
    assert _score(lib, _dims(d_idx=96)) == MSA_ERR_UNSUPPORTED
    assert b"d_idx" in lib.msa_last_error()
    assert _score(lib, _dims(n_idx=17)) == MSA_ERR_UNSUPPORTED
    assert _score(lib, _dims(blk=64)) == MSA_ERR_UNSUPPORTED
    assert _score(lib, _dims(G=0)) == MSA_ERR_INVALID
    assert _score(lib, _dims(), rows=-1) == MSA_ERR_INVALID
    assert _score(lib, _dims(), ss=0) == MSA_ERR_INVALID
    assert _score(lib, _dims(), q=None) == MSA_ERR_NULL
    assert _score(lib, _dims(), q=MISALIGNED) == MSA_ERR_INVALID
    assert _score(lib, _dims(), kv=_view(base=MISALIGNED)) == MSA_ERR_INVALID
    assert _score(lib, _dims(), kv=_view(ts=100)) == MSA_ERR_INVALID
    assert _score(lib, _dims(), rows=0) == MSA_OK          # nothing to do, nothing launched


def test_topk_and_page_table_validation(lib):
    d = _dims()
    assert lib.msa_topk_blocks(ctypes.byref(d), 1, FAKE, 4, FAKE, -1, FAKE, None) == MSA_ERR_INVALID
    assert lib.msa_topk_blocks(ctypes.byref(d), 1, None, 4, FAKE, 2, FAKE, None) == MSA_ERR_NULL
    assert lib.msa_topk_blocks(ctypes.byref(d), 0, None, 4, None, 2, None, None) == MSA_OK
    assert lib.msa_build_page_table(ctypes.byref(d), 1, FAKE, 0, None, FAKE, 4, FAKE,
                                    None) == MSA_ERR_INVALID
    assert lib.msa_build_page_table(ctypes.byref(d), 1, None, 3, None, FAKE, 4, FAKE,
                                    None) == MSA_ERR_NULL
    paged = lib.msa_topk_blocks_paged
    assert paged(ctypes.byref(d), 1, FAKE, 4, FAKE, -1, None, FAKE, 4, FAKE, FAKE,
                 None) == MSA_ERR_INVALID
    assert paged(ctypes.byref(d), 1, FAKE, 4, FAKE, 2, None, FAKE, 0, FAKE, FAKE,
                 None) == MSA_ERR_INVALID
    assert paged(ctypes.byref(d), 1, FAKE, 4, FAKE, 2, None, None, 4, FAKE, FAKE,
                 None) == MSA_ERR_NULL
    assert paged(ctypes.byref(d), 1, FAKE, 4, FAKE, 2, None, FAKE, 4, FAKE, None,
                 None) == MSA_ERR_NULL
    assert paged(ctypes.byref(d), 0, None, 4, None, 2, None, None, 4, None, None,
                 None) == MSA_OK


@pytest.mark.parametrize("k,rows", [(2 ** 31 - 1, 1), (2 ** 30, 1), (2 ** 28, 8)])
def test_topk_rejects_huge_k(lib, k, rows):
    """k near INT32_MAX (k + 1 would overflow the kernels' slot loops) and
    selections beyond an int32 element count are refused before any launch,
    by every call that selects."""
    d = _dims()
    assert lib.msa_topk_blocks(ctypes.byref(d), rows, FAKE, 4, FAKE, k, FAKE,
                               None) == MSA_ERR_INVALID
    assert b"k" in lib.msa_last_error()
    assert lib.msa_topk_blocks_paged(ctypes.byref(d), rows, FAKE, 4, FAKE, k, None, FAKE, 4,
                                     FAKE, FAKE, None) == MSA_ERR_INVALID
    assert lib.msa_sparse_attn_decode_select(
        ctypes.byref(d), rows, FAKE, 4, k, None, FAKE, 4, FAKE, _view(), _view(), FAKE,
        ctypes.c_float(0.088), FAKE, FAKE, FAKE, FAKE, None) == MSA_ERR_INVALID


def _decode(lib, dims, **kw):
    a = dict(rows=1, q=FAKE, k=_view(), v=_view(), sel=FAKE, pt=FAKE, nslot=3, rp=FAKE,
             scale=0.088, o=FAKE, lse=FAKE)
    a.update(kw)
    return lib.msa_sparse_attn_decode(ctypes.byref(dims), a["rows"], a["q"], a["k"], a["v"],
                                      a["sel"], a["pt"], a["nslot"], a["rp"], a["scale"],
                                      a["o"], a["lse"], None)


def test_attention_validation(lib):
    assert _decode(lib, _dims(D=64)) == MSA_ERR_UNSUPPORTED
    assert _decode(lib, _dims(Hg=3)) == MSA_ERR_UNSUPPORTED
    assert _decode(lib, _dims(), scale=0.0) == MSA_ERR_INVALID
    assert _decode(lib, _dims(), scale=float("nan")) == MSA_ERR_INVALID
    assert _decode(lib, _dims(), nslot=0) == MSA_ERR_INVALID
    assert _decode(lib, _dims(), o=MISALIGNED) == MSA_ERR_INVALID
    assert _decode(lib, _dims(), v=_view(base=ctypes.c_void_p(0))) == MSA_ERR_NULL
    assert _decode(lib, _dims(), rows=0) == MSA_OK


def _decode_select(lib, dims, **kw):
    a = dict(rows=1, scores=FAKE, ss=4, k=2, rr=None, bt=FAKE, bts=4, q=FAKE, kc=_view(),
             vc=_view(), rp=FAKE, scale=0.088, sel=FAKE, pt=FAKE, o=FAKE, lse=FAKE)
    a.update(kw)
    return lib.msa_sparse_attn_decode_select(
        ctypes.byref(dims), a["rows"], a["scores"], a["ss"], a["k"], a["rr"], a["bt"], a["bts"],
        a["q"], a["kc"], a["vc"], a["rp"], a["scale"], a["sel"], a["pt"], a["o"], a["lse"], None)


def test_decode_select_validation(lib):
    assert _decode_select(lib, _dims(D=64)) == MSA_ERR_UNSUPPORTED
    assert _decode_select(lib, _dims(), k=-1) == MSA_ERR_INVALID
    assert _decode_select(lib, _dims(), ss=0) == MSA_ERR_INVALID
    assert _decode_select(lib, _dims(), bts=0) == MSA_ERR_INVALID
    assert _decode_select(lib, _dims(), scale=0.0) == MSA_ERR_INVALID
    assert _decode_select(lib, _dims(), o=MISALIGNED) == MSA_ERR_INVALID
    assert _decode_select(lib, _dims(), scores=None) == MSA_ERR_NULL
    assert _decode_select(lib, _dims(), bt=None) == MSA_ERR_NULL
    assert _decode_select(lib, _dims(), sel=None) == MSA_ERR_NULL
    assert _decode_select(lib, _dims(), pt=None) == MSA_ERR_NULL
    assert _decode_select(lib, _dims(), rows=0, scores=None, bt=None, q=None, sel=None, pt=None,
                          rp=None, o=None, lse=None) == MSA_OK


def _decode_step(lib, dims, **kw):
    a = dict(rows=1, qi=FAKE, ki=_view(), bt=FAKE, bts=4, rr=None, rp=FAKE, lo=None, nreq=1,
             ss=4, k=2, q=FAKE, kc=_view(), vc=_view(), scale=0.088, scores=FAKE, sel=FAKE,
             pt=FAKE, op=FAKE, lp=FAKE, o=FAKE, lse=None, sync=FAKE, mode=0)
    a.update(kw)
    return lib.msa_decode_step(
        ctypes.byref(dims), a["rows"], a["qi"], a["ki"], a["bt"], a["bts"], a["rr"], a["rp"],
        a["lo"], a["nreq"], a["ss"], a["k"], a["q"], a["kc"], a["vc"], a["scale"], a["scores"],
        a["sel"], a["pt"], a["op"], a["lp"], a["o"], a["lse"], a["sync"], a["mode"], None)


def test_decode_step_validation(lib):
    assert _decode_step(lib, _dims(d_idx=96)) == MSA_ERR_UNSUPPORTED
    assert _decode_step(lib, _dims(D=64)) == MSA_ERR_UNSUPPORTED
    assert _decode_step(lib, _dims(), mode=3) == MSA_ERR_INVALID
    assert b"mode" in lib.msa_last_error()
    assert _decode_step(lib, _dims(), k=-1) == MSA_ERR_INVALID
    assert _decode_step(lib, _dims(), ss=0) == MSA_ERR_INVALID
    assert _decode_step(lib, _dims(), nreq=0) == MSA_ERR_INVALID
    assert _decode_step(lib, _dims(), scale=0.0) == MSA_ERR_INVALID
    assert _decode_step(lib, _dims(), qi=None) == MSA_ERR_NULL
    assert _decode_step(lib, _dims(), scores=None) == MSA_ERR_NULL
    assert _decode_step(lib, _dims(), o=None) == MSA_ERR_NULL
    assert _decode_step(lib, _dims(), o=MISALIGNED) == MSA_ERR_INVALID
    assert _decode_step(lib, _dims(), ki=_view(ts=100)) == MSA_ERR_INVALID
    # the single launch: score rows of at most 1,024 blocks, and the sync words
    assert _decode_step(lib, _dims(), ss=1025, mode=1) == MSA_ERR_UNSUPPORTED
    assert _decode_step(lib, _dims(), sync=None, mode=1) == MSA_ERR_NULL
    assert _decode_step(lib, _dims(), sync=MISALIGNED) == MSA_ERR_INVALID
    assert _decode_step(lib, _dims(), rows=0, qi=None, bt=None, rp=None, q=None, scores=None,
                        sel=None, pt=None, op=None, lp=None, o=None, sync=None) == MSA_OK


def test_prefill_merged_validation(lib):
    d = _dims()
    n = ctypes.c_size_t(0)
    sizes = []
    for slab in (0, 8192, 4096, 1024, 1):
        assert lib.msa_prefill_merged_workspace_size(ctypes.byref(d), 8192, 17, 544, slab,
                                                     ctypes.byref(n)) == MSA_OK
        sizes.append(n.value)
    # one slab of all rows holds every partial; smaller slabs need less
    assert sizes[0] == sizes[1] > sizes[2] > sizes[3] > sizes[4]
    assert sizes[0] >= 8192 * 64 * 17 * (128 * 2 + 4)
    assert lib.msa_prefill_merged_workspace_size(ctypes.byref(d), 8192, 17, 544, -1,
                                                 ctypes.byref(n)) == MSA_ERR_INVALID
    need = sizes[2]

    def call(**kw):
        a = dict(rows=8192, slab=4096, ws=FAKE, wsb=need, o=FAKE, q=FAKE)
        a.update(kw)
        return lib.msa_sparse_attn_prefill_merged(
            ctypes.byref(d), a["rows"], a["q"], _view(), _view(), FAKE, FAKE, 17, FAKE, 544,
            0.088, a["slab"], a["ws"], a["wsb"], a["o"], None, None)
    assert call(wsb=need - 1) == MSA_ERR_WORKSPACE
    assert call(slab=-1) == MSA_ERR_INVALID
    assert call(o=None) == MSA_ERR_NULL
    assert call(o=MISALIGNED) == MSA_ERR_INVALID
    assert call(ws=ctypes.c_void_p(0x10010)) == MSA_ERR_INVALID      # not 256-byte aligned
    assert call(ws=None) == MSA_ERR_NULL
    assert call(rows=0, ws=None, o=None, q=None) == MSA_OK


def test_prefill_workspace(lib):
    d = _dims()
    n = ctypes.c_size_t(0)
    assert lib.msa_prefill_workspace_size(ctypes.byref(d), 8192, 17, 544, ctypes.byref(n)) == MSA_OK
    need = n.value
    units, entries = 8 * 544, 8192 * 8 * 17
    # at least counts + offsets per (group, page) unit and one list entry per
    # (row, group, slot); at most that plus the counting sort's per-workgroup
    # counts (<= 256 workgroups) and alignment padding
    assert need >= 4 * (2 * units + 1 + entries)
    assert need <= 4 * (258 * units + 1 + entries) + 1024
    st = lib.msa_sparse_attn_prefill(ctypes.byref(d), 8192, FAKE, _view(), _view(), FAKE, FAKE,
                                     17, FAKE, 544, 0.088, FAKE, need - 1, FAKE, FAKE, None)
    assert st == MSA_ERR_WORKSPACE
    assert b"workspace" in lib.msa_last_error()
    st = lib.msa_sparse_attn_prefill(ctypes.byref(d), 8192, FAKE, _view(), _view(), FAKE, FAKE,
                                     17, FAKE, 0, 0.088, FAKE, need, FAKE, FAKE, None)
    assert st == MSA_ERR_INVALID


def test_merge_validation(lib):
    assert lib.msa_lse_merge(1, 8, 3, 64, FAKE, FAKE, FAKE, None, None) == MSA_ERR_UNSUPPORTED
    assert lib.msa_lse_merge(1, 0, 3, 128, FAKE, FAKE, FAKE, None, None) == MSA_ERR_INVALID
    assert lib.msa_lse_merge(1, 8, 3, 128, None, FAKE, FAKE, None, None) == MSA_ERR_NULL
    assert lib.msa_lse_merge(0, 8, 3, 128, None, None, None, None, None) == MSA_OK


def test_gather_pages_validation(lib):
    d = _dims()
    assert lib.msa_gather_pages(ctypes.byref(d), 0, None, 17, _view(), _view(), None, None, None,
                                None) == MSA_OK
    assert lib.msa_gather_pages(ctypes.byref(d), 4, None, 17, _view(), _view(), FAKE, FAKE, FAKE,
                                None) == MSA_ERR_NULL
    assert lib.msa_gather_pages(ctypes.byref(d), 4, FAKE, 0, _view(), _view(), FAKE, FAKE, FAKE,
                                None) == MSA_ERR_INVALID
    assert lib.msa_gather_pages(ctypes.byref(d), 4, FAKE, 17, _view(), _view(), MISALIGNED, FAKE,
                                FAKE, None) == MSA_ERR_INVALID
    d64 = _dims(D=64)
    assert lib.msa_gather_pages(ctypes.byref(d64), 4, FAKE, 17, _view(), _view(), FAKE, FAKE,
                                FAKE, None) == MSA_ERR_UNSUPPORTED


def test_peak_probe_validation(lib):
    flops = ctypes.c_double(0.0)
    assert lib.msa_peak_stream_read(FAKE, 24, FAKE, None) == MSA_ERR_INVALID
    assert lib.msa_peak_stream_read(MISALIGNED, 32, FAKE, None) == MSA_ERR_INVALID
    assert lib.msa_peak_stream_read(None, 32, FAKE, None) == MSA_ERR_NULL
    assert lib.msa_peak_stream_read(None, 0, None, None) == MSA_OK
    assert lib.msa_peak_mfma_bf16(0, FAKE, ctypes.byref(flops), None) == MSA_ERR_INVALID
    assert lib.msa_peak_mfma_bf16(8, None, ctypes.byref(flops), None) == MSA_ERR_NULL
    assert lib.msa_peak_mfma_bf16(8, FAKE, None, None) == MSA_ERR_NULL
    assert lib.msa_peak_stream_write(FAKE, 24, 0, None) == MSA_ERR_INVALID
    assert lib.msa_peak_stream_write(MISALIGNED, 32, 0, None) == MSA_ERR_INVALID
    assert lib.msa_peak_stream_write(None, 32, 0, None) == MSA_ERR_NULL
    assert lib.msa_peak_stream_write(None, 0, 0, None) == MSA_OK
    assert lib.msa_peak_mfma_bf16_random(0, FAKE, ctypes.byref(flops), None) == MSA_ERR_INVALID
    assert lib.msa_peak_mfma_bf16_random(8, None, ctypes.byref(flops), None) == MSA_ERR_NULL
    # row gather-scatter: every call below fails validation (or has n = 0) before any launch
    assert lib.msa_peak_row_copy(FAKE, FAKE, FAKE, FAKE, 33, 64, 0, None) == MSA_ERR_INVALID
    assert lib.msa_peak_row_copy(FAKE, FAKE, FAKE, FAKE, -32, 64, 0, None) == MSA_ERR_INVALID
    assert lib.msa_peak_row_copy(FAKE, FAKE, FAKE, FAKE, 64, 0, 0, None) == MSA_ERR_INVALID
    assert lib.msa_peak_row_copy(FAKE, FAKE, FAKE, FAKE, 64, 65, 1, None) == MSA_ERR_INVALID
    assert lib.msa_peak_row_copy(FAKE, FAKE, FAKE, FAKE, 64, 64, 2, None) == MSA_ERR_INVALID
    assert lib.msa_peak_row_copy(None, FAKE, FAKE, FAKE, 64, 64, 0, None) == MSA_ERR_NULL
    assert lib.msa_peak_row_copy(FAKE, FAKE, None, FAKE, 64, 64, 0, None) == MSA_ERR_NULL
    assert lib.msa_peak_row_copy(MISALIGNED, FAKE, FAKE, FAKE, 64, 64, 0, None) == MSA_ERR_INVALID
    assert lib.msa_peak_row_copy(None, None, None, None, 0, 64, 0, None) == MSA_OK


def test_binding_refuses_host_tensors():
    import torch
    from block_sparse_attention_09_amd import binding
    d = _dims()
    with pytest.raises(TypeError):
        binding.msa_topk_blocks(d, torch.zeros((1, 8, 4)), torch.zeros(1, dtype=torch.int32), 2)
