"""Seeded synthetic inputs for the MSA hot path (shared by tests, smoke and bench).

This module holds no arithmetic of the method: it only draws iid N(0, 1) values,
rounds them to bf16 (round-to-nearest-even, torch's conversion), lays them out in
paged caches and builds block tables, positions and request maps.  Both the GPU
library and the CPU oracle consume what it produces; neither is imported here.

Workload recipe (the pages' own traffic, agentic requests on a 60K prefix cache at
concurrency 8, is not available, so seeded synthetic tensors of the same shapes
stand in for it):

* every value of q, q_idx, K, V and k_idx is iid N(0, 1), drawn in fp32 by a torch
  generator seeded from (case seed, tensor id) and rounded to bf16; the generator
  runs on the device the case is built on, so CPU and GPU builds of one seed hold
  different (equally distributed) values;
* caches are paged with 128 tokens per page, laid out [page][group][token][dim];
  "paged" cases place logical block b of request r at a seeded random permutation
  of the page pool, "contiguous" cases use the identity;
* decode rows sit at position L - 1 (the new token is already in the cache);
  prefill rows are the chunk tokens p0 .. p0 + Tq - 1 of one request;
* ``poison`` fills every cache slot after a request's last token with a large
  constant (or, with ``poison="nan"``, with NaN), so a kernel that forgets a
  causal mask, or lets a masked slot's value through, produces visibly wrong
  results.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

BLK = 128

# tensor ids mixed into the seed
T_Q, T_QIDX, T_K, T_V, T_KIDX, T_PERM, T_LEN, T_LO = 1, 2, 3, 4, 5, 6, 7, 8


@dataclasses.dataclass
class Case:
    name: str
    G: int
    Hg: int
    D: int
    n_idx: int
    d_idx: int
    k: int
    rows: int
    num_reqs: int
    num_pages: int
    nb: int                       # score stride = max blocks per request
    q_idx: torch.Tensor           # bf16 [rows][G][n_idx][d_idx]
    q: torch.Tensor               # bf16 [rows][G*Hg][D]
    k_idx: torch.Tensor           # bf16 [P][G][128][d_idx]
    k_cache: torch.Tensor         # bf16 [P][G][128][D]
    v_cache: torch.Tensor         # bf16 [P][G][128][D]
    block_table: torch.Tensor     # int32 [num_reqs][nb]
    row_req: torch.Tensor         # int32 [rows]
    row_pos: torch.Tensor         # int32 [rows]
    ctx_len: torch.Tensor         # int32 [num_reqs] tokens in cache per request
    blk_lo: Optional[torch.Tensor] = None  # int32 [num_reqs][G] or None
    prefill: bool = False

    @property
    def H(self):
        return self.G * self.Hg

    @property
    def nslot(self):
        return self.k + 1

    def to(self, device):
        kw = {}
        for f in dataclasses.fields(self):
            v = getattr(self, f.name)
            kw[f.name] = v.to(device) if isinstance(v, torch.Tensor) else v
        return Case(**kw)


def _gen(seed: int, tensor: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1000 + tensor)
    return g


def bf16_normal(shape, seed: int, tensor: int, device, chunk_elems: int = 1 << 28) -> torch.Tensor:
    """iid N(0,1) drawn in fp32 and rounded to bf16, in chunks to bound temporaries."""
    out = torch.empty(shape, dtype=torch.bfloat16, device=device)
    flat = out.view(-1)
    g = _gen(seed, tensor, device)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=g, dtype=torch.float32, device=device).to(
            torch.bfloat16)
    return out


def build_case(name, *, seed, ctx_lens, G, Hg, d_idx, k, D=128, n_idx=4, paged=True,
               pool_pages=None, prefill_rows=0, lo_frac=0.0, poison=False,
               device="cpu") -> Case:
    """Build one case.

    ctx_lens      : tokens in the cache per request (decode rows sit at len-1)
    prefill_rows  : if > 0 (or a list, one entry per request), the last
                    prefill_rows tokens of each request are query rows (positions
                    len-n .. len-1), rows of one request contiguous
    lo_frac       : if > 0, per-(request, group) lower candidate bound drawn
                    uniformly in [0, lo_frac * n_blocks]
    """
    ctx_lens = [int(x) for x in ctx_lens]
    R = len(ctx_lens)
    nblk = [(L + BLK - 1) // BLK for L in ctx_lens]
    nb = max(nblk)
    need = sum(nblk)
    P = max(need, pool_pages or 0)
    if paged:
        perm = torch.randperm(P, generator=_gen(seed, T_PERM, "cpu"))
    else:
        perm = torch.arange(P)
    bt = torch.zeros((R, nb), dtype=torch.int32)
    off = 0
    for r in range(R):
        bt[r, :nblk[r]] = perm[off:off + nblk[r]].to(torch.int32)
        off += nblk[r]
    if prefill_rows:
        per = list(prefill_rows) if isinstance(prefill_rows, (list, tuple)) else [prefill_rows]
        assert len(per) == R
        row_req = torch.cat([torch.full((n,), r, dtype=torch.int32) for r, n in enumerate(per)])
        row_pos = torch.cat([torch.arange(ctx_lens[r] - n, ctx_lens[r], dtype=torch.int32)
                             for r, n in enumerate(per)])
        rows = int(row_req.numel())
    else:
        rows = R
        row_req = torch.arange(R, dtype=torch.int32)
        row_pos = torch.tensor([L - 1 for L in ctx_lens], dtype=torch.int32)
    blk_lo = None
    if lo_frac > 0:
        g = _gen(seed, T_LO, "cpu")
        blk_lo = torch.zeros((R, G), dtype=torch.int32)
        for r in range(R):
            hi = int(lo_frac * nblk[r])
            blk_lo[r] = torch.randint(0, hi + 1, (G,), generator=g, dtype=torch.int32)
    H = G * Hg
    case = Case(
        name=name, G=G, Hg=Hg, D=D, n_idx=n_idx, d_idx=d_idx, k=k, rows=rows, num_reqs=R,
        num_pages=P, nb=nb,
        q_idx=bf16_normal((rows, G, n_idx, d_idx), seed, T_QIDX, device),
        q=bf16_normal((rows, H, D), seed, T_Q, device),
        k_idx=bf16_normal((P, G, BLK, d_idx), seed, T_KIDX, device),
        k_cache=bf16_normal((P, G, BLK, D), seed, T_K, device),
        v_cache=bf16_normal((P, G, BLK, D), seed, T_V, device),
        block_table=bt.to(device), row_req=row_req.to(device), row_pos=row_pos.to(device),
        ctx_len=torch.tensor(ctx_lens, dtype=torch.int32, device=device),
        blk_lo=None if blk_lo is None else blk_lo.to(device), prefill=bool(prefill_rows))
    if poison:
        nan = poison == "nan"
        for r in range(R):
            L = ctx_lens[r]
            if L % BLK:
                page = int(bt[r, nblk[r] - 1])
                t0 = L % BLK
                case.k_idx[page, :, t0:, :] = float("nan") if nan else 8.0
                case.k_cache[page, :, t0:, :] = float("nan") if nan else 8.0
                case.v_cache[page, :, t0:, :] = float("nan") if nan else 64.0
    return case


# ----------------------------------------------------------------------------- the five workloads
CONFIGS = {
    1: dict(name="decode-4k-b1", seed=1001, G=2, Hg=4, d_idx=64, k=4, paged=False),
    2: dict(name="decode-64k-b8", seed=1002, G=8, Hg=8, d_idx=128, k=16, paged=True),
    3: dict(name="decode-ragged-b32", seed=1003, G=8, Hg=8, d_idx=128, k=32, paged=True),
    4: dict(name="prefill-8k-on-60k", seed=1004, G=8, Hg=8, d_idx=128, k=16, paged=False),
    5: dict(name="decode-1m-b4", seed=1005, G=8, Hg=8, d_idx=128, k=32, paged=True),
}


def ragged_lengths(seed: int, n: int = 32, lo_blocks: int = 64, hi_blocks: int = 2048):
    g = _gen(seed, T_LEN, "cpu")
    nblk = torch.randint(lo_blocks, hi_blocks + 1, (n,), generator=g)
    return [int(b) * BLK for b in nblk]


def config_case(cfg: int, device="cpu", lo_frac: float = 0.0) -> Case:
    """The five seeded workloads at their full sizes."""
    c = dict(CONFIGS[cfg])
    name, seed = c.pop("name"), c.pop("seed")
    if cfg == 1:
        return build_case(name, seed=seed, ctx_lens=[4096], device=device, **c)
    if cfg == 2:
        return build_case(name, seed=seed, ctx_lens=[65536] * 8, pool_pages=4096, device=device,
                          **c)
    if cfg == 3:
        return build_case(name, seed=seed, ctx_lens=ragged_lengths(seed), device=device,
                          lo_frac=lo_frac, **c)
    if cfg == 4:
        return build_case(name, seed=seed, ctx_lens=[61440 + 8192], prefill_rows=8192,
                          device=device, **c)
    if cfg == 5:
        return build_case(name, seed=seed, ctx_lens=[1 << 20] * 4, pool_pages=32768,
                          device=device, **c)
    raise ValueError(cfg)


def bits(t: torch.Tensor):
    """bf16 tensor -> NumPy uint16 bit patterns on the host (a view when possible)."""
    return t.detach().to("cpu").contiguous().view(torch.int16).numpy().view("uint16")
