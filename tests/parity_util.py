"""Helpers for GPU-vs-oracle parity: run the HIP path through the binding, run
the oracle on host copies of the same inputs, and compare with the stated
tolerances.

Tolerances (fixed by the method's accuracy targets):
  scores     |S_gpu - S_ref| <= 1e-3 |S_ref| for finite S_ref (guard 1e-3 max|S_ref|
             per row near 0); -inf exactly where the oracle has -inf
  selection  bit-exact, except near-tie rows (k-th and (k+1)-th oracle scores
             closer than 1e-3 relative), which must still pick a valid top set
  attention  max |o_gpu - o_ref| <= 1e-2 on the same selection; partial LSEs within
             1e-3 max(1, |lse|); empty slots exactly o = 0, lse = -inf
"""
from __future__ import annotations

import math

import numpy as np
import torch

import msa_synth
import oracle

BLK = 128
SCORE_RTOL = 1e-3
ATTN_ATOL = 1e-2
LSE_RTOL = 1e-3


def dims_of(case):
    from block_sparse_attention_09_amd import Dims
    return Dims(G=case.G, Hg=case.Hg, D=case.D, n_idx=case.n_idx, d_idx=case.d_idx, blk=BLK)


def gpu_path(case, prefill=None, sel=None, pt=None, sm_scale=None):
    """Run the whole HIP path on a device case; returns host tensors."""
    import block_sparse_attention_09_amd as msa
    d = dims_of(case)
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(case.D)
    scores = msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos,
                                 case.nb, row_req=case.row_req, blk_lo=case.blk_lo,
                                 num_reqs=case.num_reqs)
    sel_gpu = msa.msa_topk_blocks(d, scores, case.row_pos, case.k)
    pt_gpu = msa.msa_build_page_table(d, sel_gpu, case.block_table, row_req=case.row_req)
    # the fused selection + page-table call writes the same two arrays, bit for bit
    sel_f, pt_f = msa.msa_topk_blocks_paged(d, scores, case.row_pos, case.k, case.block_table,
                                            row_req=case.row_req)
    assert torch.equal(sel_f, sel_gpu), "msa_topk_blocks_paged: sel differs"
    assert torch.equal(pt_f, pt_gpu), "msa_topk_blocks_paged: page table differs"
    use_sel = sel_gpu if sel is None else sel
    use_pt = pt_gpu if pt is None else pt
    if prefill is None:
        prefill = case.prefill
    if prefill:
        o_part, lse_part = msa.msa_sparse_attn_prefill(d, case.q, case.k_cache, case.v_cache,
                                                       use_sel, use_pt, case.row_pos,
                                                       case.num_pages, scale)
    else:
        o_part, lse_part = msa.msa_sparse_attn_decode(d, case.q, case.k_cache, case.v_cache,
                                                      use_sel, use_pt, case.row_pos, scale)
        if sel is None and pt is None:
            # the fused selection + page table + decode attention call writes the
            # same four arrays, bit for bit
            sel_d, pt_d, o_d, lse_d = msa.msa_sparse_attn_decode_select(
                d, scores, case.k, case.block_table, case.q, case.k_cache, case.v_cache,
                case.row_pos, row_req=case.row_req, sm_scale=scale)
            assert torch.equal(sel_d, sel_gpu), "msa_sparse_attn_decode_select: sel differs"
            assert torch.equal(pt_d, pt_gpu), "msa_sparse_attn_decode_select: page table differs"
            assert torch.equal(o_d.view(torch.int16), o_part.view(torch.int16)), \
                "msa_sparse_attn_decode_select: o_part differs"
            assert torch.equal(lse_d.view(torch.int32), lse_part.view(torch.int32)), \
                "msa_sparse_attn_decode_select: lse_part differs"
    o, lse = msa.msa_lse_merge(o_part, lse_part)
    torch.cuda.synchronize()
    return {k: v.cpu() for k, v in dict(scores=scores, sel=sel_gpu, pt=pt_gpu, o_part=o_part,
                                        lse_part=lse_part, o=o, lse=lse).items()}


def host_rows(case, rows):
    """Host (oracle) inputs for a subset of rows: index and query tensors of those
    rows, the key-index pages of their requests in a compact pool, and a block
    table remapped onto it."""
    rows = list(rows)
    rr = case.row_req.cpu().numpy()[rows]
    reqs = sorted(set(rr.tolist()))
    bt_full = case.block_table.cpu().numpy()
    ctx = case.ctx_len.cpu().numpy()
    pages, bt = [], np.zeros((len(reqs), bt_full.shape[1]), np.int32)
    for i, r in enumerate(reqs):
        nblk = (int(ctx[r]) + BLK - 1) // BLK
        bt[i, :nblk] = len(pages) + np.arange(nblk)
        pages.extend(bt_full[r, :nblk].tolist())
    pidx = torch.tensor(pages, dtype=torch.long, device=case.k_idx.device)
    remap = {r: i for i, r in enumerate(reqs)}
    lo = None
    if case.blk_lo is not None:
        lo = case.blk_lo.cpu().numpy()[reqs]
    ridx = torch.tensor(rows, dtype=torch.long, device=case.q.device)
    return dict(
        q_idx=msa_synth.bits(case.q_idx.index_select(0, ridx)),
        q=msa_synth.bits(case.q.index_select(0, ridx)),
        k_idx=msa_synth.bits(case.k_idx.index_select(0, pidx)),
        bt=bt, row_req=np.array([remap[int(r)] for r in rr], np.int32),
        row_pos=case.row_pos.cpu().numpy()[rows], blk_lo=lo)


def host_kv_pages(case, pt_rows: np.ndarray):
    """Compact host K/V pools holding only the pages a page table references,
    plus that page table remapped onto them."""
    used = sorted(set(int(p) for p in pt_rows.ravel() if p >= 0))
    remap = np.full(max(used) + 1 if used else 1, -1, np.int64)
    remap[used] = np.arange(len(used))
    pt_c = np.where(pt_rows >= 0, remap[np.maximum(pt_rows, 0)], -1).astype(np.int32)
    pidx = torch.tensor(used, dtype=torch.long, device=case.k_cache.device)
    return (msa_synth.bits(case.k_cache.index_select(0, pidx)),
            msa_synth.bits(case.v_cache.index_select(0, pidx)), pt_c)


def oracle_scores(case, rows):
    h = host_rows(case, rows)
    return oracle.index_score(h["q_idx"], h["k_idx"], h["bt"], h["row_pos"], case.nb,
                              row_req=h["row_req"], blk_lo=h["blk_lo"])


def oracle_attn(case, rows, sel_rows, pt_rows, sm_scale=None):
    """Oracle partials and direct attention for rows on a given selection."""
    scale = sm_scale if sm_scale is not None else 1.0 / math.sqrt(case.D)
    ridx = torch.tensor(list(rows), dtype=torch.long, device=case.q.device)
    q = msa_synth.bits(case.q.index_select(0, ridx))
    kp, vp, pt_c = host_kv_pages(case, pt_rows)
    pos = case.row_pos.cpu().numpy()[list(rows)]
    op, lp = oracle.attn_partials(q, kp, vp, sel_rows, pt_c, pos, scale)
    o, lse = oracle.attn(q, kp, vp, sel_rows, pt_c, pos, scale)
    return op, lp, o, lse


# ----------------------------------------------------------------------------- comparisons
def check_scores(s_gpu: np.ndarray, s_ref: np.ndarray):
    s_gpu = np.asarray(s_gpu, np.float64)
    ninf_ref = np.isneginf(s_ref)
    assert np.array_equal(np.isneginf(s_gpu), ninf_ref), "-inf pattern differs"
    fin = ~ninf_ref
    guard = SCORE_RTOL * np.max(np.where(fin, np.abs(s_ref), 0), axis=-1, keepdims=True)
    tol = np.maximum(SCORE_RTOL * np.abs(s_ref), guard)
    err = np.where(fin, np.abs(s_gpu - np.where(fin, s_ref, 0)), 0)
    bad = err > tol
    assert not bad.any(), f"{bad.sum()} scores out of tolerance, worst rel " \
                          f"{np.max(err / np.maximum(np.abs(s_ref), 1e-30)):.3g}"
    return float(np.max(np.where(fin, err / np.maximum(np.abs(s_ref), 1e-30), 0)))


def check_selection(sel_gpu, sel_ref, s_ref, row_pos, k):
    """Bit-exact selection, with the near-tie exemption.  Returns the number of
    (row, group) pairs that differed but were accepted as near ties."""
    sel_gpu, sel_ref = np.asarray(sel_gpu), np.asarray(sel_ref)
    exempt = 0
    for r, g in zip(*np.nonzero((sel_gpu != sel_ref).any(axis=-1))):
        own = int(row_pos[r]) // BLK
        sc = np.asarray(s_ref[r, g, :own], np.float64)
        cand = np.nonzero(~np.isneginf(sc))[0]
        order = cand[np.lexsort((cand, -sc[cand]))]
        keff = min(k, len(order))
        assert keff < len(order), f"row {r} group {g}: selection differs with no ranking"
        ck, ck1 = sc[order[keff - 1]], sc[order[keff]]
        tau = 1e-3 * abs(ck)
        assert ck - ck1 < tau, f"row {r} group {g}: selection differs off a near tie"
        got = [b for b in sel_gpu[r, g] if b >= 0]
        want = [b for b in sel_ref[r, g] if b >= 0]
        assert len(got) == len(want) and own in got, f"row {r} group {g}: bad size/own"
        must = set(int(b) for b in cand if sc[b] > ck + tau)
        assert must <= set(got), f"row {r} group {g}: a clear winner is missing"
        assert all(sc[b] >= ck - tau for b in got if b != own), \
            f"row {r} group {g}: a clear loser is selected"
        exempt += 1
    return exempt


def check_partials(o_part_gpu, lse_part_gpu, op_ref, lp_ref):
    o = o_part_gpu.float().numpy()
    lp = lse_part_gpu.numpy().astype(np.float64)
    empty = np.isneginf(lp_ref)
    assert np.array_equal(np.isneginf(lp), empty), "empty-slot pattern differs"
    assert np.all(o[empty] == 0), "empty slots must hold zeros"
    err = np.max(np.abs(o - op_ref)) if o.size else 0.0
    assert err <= ATTN_ATOL, f"partial o error {err}"
    fin = ~empty
    lerr = np.abs(lp[fin] - lp_ref[fin]) / np.maximum(1.0, np.abs(lp_ref[fin]))
    assert (lerr <= LSE_RTOL).all(), f"partial lse error {lerr.max()}"
    return float(err)


def check_output(o_gpu, lse_gpu, o_ref, lse_ref):
    o = o_gpu.float().numpy()
    err = float(np.max(np.abs(o - o_ref)))
    assert err <= ATTN_ATOL, f"output error {err}"
    l = lse_gpu.numpy().astype(np.float64)
    lerr = np.abs(l - lse_ref) / np.maximum(1.0, np.abs(lse_ref))
    assert (lerr <= LSE_RTOL).all(), f"lse error {lerr.max()}"
    return err
