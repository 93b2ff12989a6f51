"""Host copies of a case's inputs for the oracle (marshalling only).

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by the test
suite and by the benchmark's CPU-baseline leg.  Nothing here computes any step
of the method: it copies the bf16 bit patterns of the rows and cache pages the
oracle needs from wherever the case lives (device or host) into compact host
arrays, and renumbers block and page indices onto those compact pools.
"""
from __future__ import annotations

import numpy as np
import torch

BLK = 128


def bits(t: torch.Tensor) -> np.ndarray:
    """bf16 tensor -> NumPy uint16 bit patterns on the host."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")


def host_rows(case, rows):
    """Host inputs of the index score for a subset of rows: index and query
    vectors of those rows, the key-index pages of their requests in a compact
    pool, and a block table renumbered onto that pool."""
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
        q_idx=bits(case.q_idx.index_select(0, ridx)),
        q=bits(case.q.index_select(0, ridx)),
        k_idx=bits(case.k_idx.index_select(0, pidx)),
        bt=bt, row_req=np.array([remap[int(r)] for r in rr], np.int32),
        row_pos=case.row_pos.cpu().numpy()[rows], blk_lo=lo)


def host_kv_pages(case, pt_rows: np.ndarray):
    """Compact host K/V pools holding only the pages a page table references,
    plus that page table renumbered onto them."""
    used = sorted(set(int(p) for p in np.asarray(pt_rows).ravel() if p >= 0))
    remap = np.full(max(used) + 1 if used else 1, -1, np.int64)
    remap[used] = np.arange(len(used))
    pt_c = np.where(pt_rows >= 0, remap[np.maximum(pt_rows, 0)], -1).astype(np.int32)
    pidx = torch.tensor(used, dtype=torch.long, device=case.k_cache.device)
    return (bits(case.k_cache.index_select(0, pidx)),
            bits(case.v_cache.index_select(0, pidx)), pt_c)
