"""GPU parity: every libmsa call against the CPU oracle, element by element, on
seeded inputs that span several tiles and ragged tails, plus the invariants
that must hold bit for bit (determinism, page placement, cache layout, decode
vs block-major prefill)."""
import math

import numpy as np
import pytest
import torch

import msa_synth
import oracle
import parity_util as pu

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _build(**kw):
    kw.setdefault("device", DEV)
    kw.setdefault("poison", True)
    return msa_synth.build_case("t", **kw)


SMALL = {
    # ragged contexts, partial last blocks, lower bounds, 2 groups x 4 heads, d_idx 64
    "ragged-g2": dict(seed=101, ctx_lens=[700, 1000, 128, 300, 2049], G=2, Hg=4, d_idx=64, k=3,
                      lo_frac=0.3),
    # 8 groups x 8 heads, d_idx 128, more blocks than the top-k
    "g8-d128": dict(seed=102, ctx_lens=[5000, 129, 4096], G=8, Hg=8, d_idx=128, k=4),
    "hg1-nidx1": dict(seed=103, ctx_lens=[1500, 777], G=3, Hg=1, d_idx=128, k=2, n_idx=1),
    "hg2-nidx16": dict(seed=104, ctx_lens=[999, 2600], G=2, Hg=2, d_idx=64, k=5, n_idx=16),
    "hg16": dict(seed=105, ctx_lens=[1300, 64], G=1, Hg=16, d_idx=128, k=3),
    # k larger than every candidate list: selection = all blocks
    "k-all": dict(seed=106, ctx_lens=[900, 400], G=2, Hg=4, d_idx=64, k=40),
    "k-zero": dict(seed=107, ctx_lens=[900, 1], G=2, Hg=4, d_idx=64, k=0),
    # cache slots past each request's last token hold NaN: nothing may leak
    "nan-tail": dict(seed=108, ctx_lens=[700, 1000, 2049, 33], G=2, Hg=8, d_idx=128, k=3,
                     poison="nan"),
    # lower bounds drawn up to 1.5x the block count: some groups score only their own block
    "lo-above-own": dict(seed=109, ctx_lens=[900, 1400, 2000], G=2, Hg=4, d_idx=64, k=3,
                         lo_frac=1.5),
    # long score rows in a small batch: 782 blocks per row (the one-kernel selection +
    # decode attention, its 256 threads holding 4 scores each), 1,954 (past its
    # 1,024-block limit: two kernels)
    "long-782": dict(seed=111, ctx_lens=[100_000, 65_000], G=2, Hg=4, d_idx=64, k=8),
    "long-1954": dict(seed=112, ctx_lens=[250_000, 131_073], G=2, Hg=4, d_idx=64, k=16),
    # either side of the select call's one-round rule (8 groups x 17 slots: 9 rows =
    # 1,224 workgroups run as one kernel, 10 rows = 1,360 as two on a 256-CU part)
    "one-round-9": dict(seed=113, ctx_lens=[3000 + 97 * i for i in range(9)], G=8, Hg=8,
                        d_idx=128, k=16),
    "one-round-10": dict(seed=114, ctx_lens=[3000 + 97 * i for i in range(10)], G=8, Hg=8,
                         d_idx=128, k=16),
    # 3,000 (row, group) pairs of 3 blocks: more pairs than the scan has waves, so
    # waves fill several pairs' -inf ranges and slices cross many pair boundaries
    "many-pairs": dict(seed=110, ctx_lens=[300 + (i % 7) * 13 for i in range(1000)], G=3, Hg=2,
                       d_idx=64, k=2),
}


def _full_compare(case, res, rows=None):
    rows = list(range(case.rows)) if rows is None else list(rows)
    s_ref = pu.oracle_scores(case, rows)
    rel = pu.check_scores(res["scores"].numpy()[rows], s_ref, pu.score_floor(case, rows))
    sel_ref = oracle.topk(s_ref.astype(np.float32), case.row_pos.cpu().numpy()[rows], case.k)
    ntie = pu.check_selection(res["sel"].numpy()[rows], sel_ref, s_ref,
                              case.row_pos.cpu().numpy()[rows], case.k)
    # page table of the GPU selection: exact gather
    pt_ref = oracle.page_table(res["sel"].numpy()[rows], case.block_table.cpu().numpy(),
                               case.row_req.cpu().numpy()[rows])
    assert np.array_equal(res["pt"].numpy()[rows], pt_ref)
    return rel, ntie


@pytest.mark.parametrize("name", list(SMALL))
def test_small_decode_path(name):
    print(f"[case] small decode {name}", flush=True)
    case = _build(**SMALL[name])
    res = pu.gpu_path(case)
    _full_compare(case, res)
    # attention on the GPU's own (validated) selection against the oracle
    rows = list(range(case.rows))
    op, lp, o, lse = pu.oracle_attn(case, rows, res["sel"].numpy(), res["pt"].numpy())
    pu.check_partials(res["o_part"], res["lse_part"], op, lp)
    pu.check_output(res["o"], res["lse"], o, lse)


@pytest.mark.parametrize("nb", [512, 560, 600, 700, 1500, 3000, 5000, 9000, 17000])
def test_topk_exact_on_oracle_scores(nb):
    """Given identical fp32 scores the selection is integer work: bit-exact,
    including exact ties (scores drawn from a few levels) and -inf holes.  The
    block counts cover every kernel variant (one wave with 8, 9, 10, 12 or 16 keys
    per lane, 1,024 threads with 2, 4, 8 or 16 keys each, and the global-memory
    fallback)."""
    import block_sparse_attention_09_amd as msa
    print(f"[case] topk exact nb={nb}", flush=True)
    rng = np.random.default_rng(9 + nb)
    rows, G = (37, 3) if nb <= 3000 else (5, 2)
    levels = np.array([-2.0, -0.5, 0.0, 0.0, 0.25, 1.0, 3.0], np.float32)
    sc = rng.choice(levels, size=(rows, G, nb)).astype(np.float32)
    sc[::3] = rng.standard_normal((len(range(0, rows, 3)), G, nb)).astype(np.float32)
    sc[1, 1, :50] = -np.inf
    if rows > 5:
        sc[5, :, :] = -0.0
    pos = rng.integers(0, nb * 128, size=rows).astype(np.int32)
    pos[0], pos[2] = 5, 130
    pos[3] = nb * 128 - 1
    d = msa.Dims(G=G, Hg=1, D=128, n_idx=4, d_idx=128, blk=128)
    # a random block table (one request per row) for the fused page-table output
    bt = rng.integers(0, 1 << 20, size=(rows, nb)).astype(np.int32)
    sc_d, pos_d, bt_d = (torch.tensor(x, device=DEV) for x in (sc, pos, bt))
    for k in (0, 1, 7, 16, 33, 300, nb + 5):
        want = oracle.topk(sc, pos, k)
        got = msa.msa_topk_blocks(d, sc_d, pos_d, k).cpu().numpy()
        assert np.array_equal(got, want), f"k={k}"
        sel_f, pt_f = msa.msa_topk_blocks_paged(d, sc_d, pos_d, k, bt_d)
        assert np.array_equal(sel_f.cpu().numpy(), want), f"paged k={k}"
        assert np.array_equal(pt_f.cpu().numpy(),
                              oracle.page_table(want, bt, np.arange(rows, dtype=np.int32))), \
            f"paged page table k={k}"


def test_prefill_and_decode_agree_with_oracle():
    """Block-major prefill over many rows of one request and the per-row decode
    kernel on the same selection: both within tolerance of the oracle, with the
    same empty-slot pattern."""
    print("[case] prefill small", flush=True)
    case = _build(seed=201, ctx_lens=[3000], G=2, Hg=8, d_idx=64, k=4, prefill_rows=700,
                  paged=True)
    res_p = pu.gpu_path(case, prefill=True)
    sel = res_p["sel"].to(DEV)
    pt = res_p["pt"].to(DEV)
    res_d = pu.gpu_path(case, prefill=False, sel=sel, pt=pt)
    assert torch.equal(torch.isneginf(res_p["lse_part"]), torch.isneginf(res_d["lse_part"]))
    rows = list(range(0, case.rows, 7)) + [case.rows - 1]
    _full_compare(case, res_p, rows)
    op, lp, o, lse = pu.oracle_attn(case, rows, res_p["sel"].numpy()[rows],
                                    res_p["pt"].numpy()[rows])
    for res in (res_p, res_d):
        pu.check_partials(res["o_part"][rows], res["lse_part"][rows], op, lp)
        pu.check_output(res["o"][rows], res["lse"][rows], o, lse)


def test_prefill_hg4_ragged_tiles():
    print("[case] prefill hg4", flush=True)
    case = _build(seed=202, ctx_lens=[1000], G=2, Hg=4, d_idx=128, k=2, prefill_rows=333)
    res = pu.gpu_path(case, prefill=True)
    rows = list(range(case.rows))
    _full_compare(case, res, rows)
    op, lp, o, lse = pu.oracle_attn(case, rows, res["sel"].numpy(), res["pt"].numpy())
    pu.check_partials(res["o_part"], res["lse_part"], op, lp)
    pu.check_output(res["o"], res["lse"], o, lse)


def test_prefill_nan_tail():
    """Prefill rows whose last page is partly unwritten (NaN there): the
    block-major kernel clears the V rows no query of a unit can see."""
    print("[case] prefill nan tail", flush=True)
    case = _build(seed=204, ctx_lens=[1500, 700], G=2, Hg=8, d_idx=128, k=3,
                  prefill_rows=[300, 90], paged=True, poison="nan")
    res = pu.gpu_path(case, prefill=True)
    rows = list(range(case.rows))
    _full_compare(case, res, rows)
    op, lp, o, lse = pu.oracle_attn(case, rows, res["sel"].numpy(), res["pt"].numpy())
    pu.check_partials(res["o_part"], res["lse_part"], op, lp)
    pu.check_output(res["o"], res["lse"], o, lse)


PREFILL_SHAPES = {
    # Hg 1 / 2 / 16 exercise the other block-major tile shapes (32 / 16 / 2 query
    # tokens per 32-row tile); n_idx 1 / 7 / 16 the scorer's index-vector loop
    "hg1-nidx1": dict(seed=205, ctx_lens=[1300], G=2, Hg=1, d_idx=128, k=3, n_idx=1,
                      prefill_rows=257),
    "hg2-nidx7-d64": dict(seed=206, ctx_lens=[1100], G=3, Hg=2, d_idx=64, k=4, n_idx=7,
                          prefill_rows=190),
    "hg16-nidx16": dict(seed=207, ctx_lens=[900], G=1, Hg=16, d_idx=128, k=2, n_idx=16,
                        prefill_rows=140),
    # only the own block, and every earlier block
    "k0": dict(seed=208, ctx_lens=[1000], G=2, Hg=8, d_idx=64, k=0, prefill_rows=200),
    "k-all": dict(seed=209, ctx_lens=[1000], G=2, Hg=8, d_idx=64, k=50, prefill_rows=200),
    # 4 groups x 4,200 pages = 16,800 (group, page) units: more than the LDS
    # histogram of the counting sort holds, so the atomic inversion runs
    "big-pool": dict(seed=210, ctx_lens=[1500], G=4, Hg=2, d_idx=64, k=3, prefill_rows=150,
                     pool_pages=4200),
}


@pytest.mark.parametrize("name", list(PREFILL_SHAPES))
def test_prefill_shapes(name):
    print(f"[case] prefill {name}", flush=True)
    case = _build(paged=True, **PREFILL_SHAPES[name])
    res = pu.gpu_path(case, prefill=True)
    rows = list(range(case.rows))
    _full_compare(case, res, rows)
    op, lp, o, lse = pu.oracle_attn(case, rows, res["sel"].numpy(), res["pt"].numpy())
    pu.check_partials(res["o_part"], res["lse_part"], op, lp)
    pu.check_output(res["o"], res["lse"], o, lse)


def _random_shape(i):
    """Seeded draw of one small case: groups, heads, index vectors and dims, k,
    request count and context lengths (partial blocks included), paging, lower
    bounds, poisoned tails, decode or prefill rows."""
    rng = np.random.default_rng(7000 + i)
    G = int(rng.choice([1, 2, 3, 4, 8]))
    Hg = int(rng.choice([h for h in (1, 2, 4, 8, 16) if G * h <= 64]))
    kw = dict(seed=7000 + i, G=G, Hg=Hg, d_idx=int(rng.choice([64, 128])),
              n_idx=int(rng.choice([1, 2, 4, 5, 8])), k=int(rng.choice([0, 1, 2, 3, 5, 8, 13, 21])),
              paged=bool(rng.integers(0, 2)), lo_frac=float(rng.choice([0.0, 0.4])),
              poison=["nan", True][int(rng.integers(0, 2))])
    if i % 2:
        reqs = int(rng.integers(1, 3))
        ctx = [int(rng.integers(200, 3000)) for _ in range(reqs)]
        kw.update(ctx_lens=ctx, prefill_rows=[int(rng.integers(1, min(c, 300 // reqs) + 1))
                                              for c in ctx])
    else:
        reqs = int(rng.integers(1, 7))
        kw.update(ctx_lens=[int(rng.integers(1, 5000)) for _ in range(reqs)])
    return kw


@pytest.mark.parametrize("i", range(32))
def test_random_shapes(i):
    """Thirty-two seeded random small cases, decode (even i) and prefill (odd i), the
    whole path against the oracle: scores, selection, page table, partials and
    merged output."""
    kw = _random_shape(i)
    print(f"[case] random shape {i}: {kw}", flush=True)
    case = _build(**kw)
    res = pu.gpu_path(case)
    rows = list(range(case.rows))
    _full_compare(case, res, rows)
    op, lp, o, lse = pu.oracle_attn(case, rows, res["sel"].numpy(), res["pt"].numpy())
    pu.check_partials(res["o_part"], res["lse_part"], op, lp)
    pu.check_output(res["o"], res["lse"], o, lse)


def test_prefill_several_requests():
    """Rows of three requests in one call: row tiles that straddle requests,
    request-specific pages and positions, through the tiled scorer and the
    block-major kernel."""
    print("[case] prefill 3 requests", flush=True)
    case = _build(seed=203, ctx_lens=[2000, 900, 1500], G=2, Hg=8, d_idx=128, k=3,
                  prefill_rows=[150, 200, 300], paged=True, lo_frac=0.2)
    res = pu.gpu_path(case, prefill=True)
    rows = list(range(case.rows))
    _full_compare(case, res, rows)
    op, lp, o, lse = pu.oracle_attn(case, rows, res["sel"].numpy(), res["pt"].numpy())
    pu.check_partials(res["o_part"], res["lse_part"], op, lp)
    pu.check_output(res["o"], res["lse"], o, lse)


def test_side_stream_matches_default_stream():
    """Every call runs on the caller's stream: the whole path (decode and
    prefill) issued on a side stream gives the default stream's results."""
    print("[case] side stream", flush=True)
    for prefill in (False, True):
        kw = dict(seed=302, ctx_lens=[2100, 900], G=2, Hg=4, d_idx=64, k=3, paged=True)
        if prefill:
            kw["prefill_rows"] = [120, 70]
        case = _build(**kw)
        a = pu.gpu_path(case)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            b = pu.gpu_path(case)
        torch.cuda.synchronize()
        for key in a:
            assert torch.equal(a[key], b[key]), (prefill, key)


def test_deterministic_and_placement_invariant():
    """Two runs are bit-identical; moving pages in the pool (paged vs contiguous)
    and a token-major cache layout give bit-identical results."""
    print("[case] determinism/placement", flush=True)
    case = _build(seed=301, ctx_lens=[3000, 1700], G=2, Hg=4, d_idx=128, k=3, paged=True,
                  poison=False)
    a = pu.gpu_path(case)
    b = pu.gpu_path(case)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    # contiguous placement of the same logical blocks
    bt = case.block_table.cpu()
    nblk = [(int(L) + 127) // 128 for L in case.ctx_len.cpu()]
    order = torch.cat([bt[r, :nblk[r]] for r in range(case.num_reqs)]).long().to(DEV)
    bt_c = torch.zeros_like(bt)
    off = 0
    for r in range(case.num_reqs):
        bt_c[r, :nblk[r]] = torch.arange(off, off + nblk[r], dtype=torch.int32)
        off += nblk[r]
    c2 = msa_synth.Case(**{**case.__dict__, "k_idx": case.k_idx[order].contiguous(),
                           "k_cache": case.k_cache[order].contiguous(),
                           "v_cache": case.v_cache[order].contiguous(),
                           "block_table": bt_c.to(DEV), "num_pages": off})
    c = pu.gpu_path(c2)
    for key in ("scores", "sel", "o_part", "lse_part", "o", "lse"):
        assert torch.equal(a[key], c[key]), key
    # token-major physical layout [page][token][group][dim], same logical view
    tm = {}
    for name in ("k_idx", "k_cache", "v_cache"):
        t = getattr(case, name)
        tm[name] = t.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)
    c3 = msa_synth.Case(**{**case.__dict__, **tm})
    d = pu.gpu_path(c3)
    for key in a:
        assert torch.equal(a[key], d[key]), key


def test_kv_cache_in_pinned_host_memory():
    """Decoupled offload: the key index stays on the GPU, K and V live in pinned
    host memory and the attention kernels read only the selected pages over the
    host link; results are bit-identical to a device-resident cache, for decode
    and for the block-major prefill."""
    for prefill in (False, True):
        print(f"[case] kv cache in pinned host memory, prefill={prefill}", flush=True)
        if prefill:
            case = _build(seed=311, ctx_lens=[1500], G=2, Hg=8, d_idx=128, k=3,
                          prefill_rows=300, poison="nan")
        else:
            case = _build(seed=312, ctx_lens=[3000, 1700, 257], G=2, Hg=4, d_idx=64, k=3,
                          paged=True, poison="nan")
        a = pu.gpu_path(case)
        host = msa_synth.Case(**{**case.__dict__,
                                 "k_cache": case.k_cache.cpu().pin_memory(),
                                 "v_cache": case.v_cache.cpu().pin_memory()})
        assert host.k_cache.is_pinned() and not host.k_cache.is_cuda
        b = pu.gpu_path(host)
        for key in a:
            assert torch.equal(a[key], b[key]), key
        # and the host-memory result itself against the oracle
        rows = list(range(case.rows))
        _full_compare(host, b)
        op, lp, o, lse = pu.oracle_attn(host, rows, b["sel"].numpy(), b["pt"].numpy())
        pu.check_partials(b["o_part"], b["lse_part"], op, lp)
        pu.check_output(b["o"], b["lse"], o, lse)


def test_gather_pages_then_decode():
    """On-demand load: gathering the selected pages (from pinned host memory or
    from the device cache) into a compact pool and running decode attention on
    the pool gives the same partials, bit for bit, as decode on the cache."""
    import block_sparse_attention_09_amd as msa
    print("[case] gather pages then decode", flush=True)
    case = _build(seed=314, ctx_lens=[3000, 1700, 257, 130], G=2, Hg=8, d_idx=128, k=3,
                  paged=True, poison="nan")
    d = pu.dims_of(case)
    scale = 1.0 / math.sqrt(case.D)
    scores = msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos,
                                 case.nb, row_req=case.row_req)
    sel, pt = msa.msa_topk_blocks_paged(d, scores, case.row_pos, case.k, case.block_table,
                                        row_req=case.row_req)
    ref = msa.msa_sparse_attn_decode(d, case.q, case.k_cache, case.v_cache, sel, pt,
                                     case.row_pos, scale)
    rows = list(range(case.rows))
    op, lp, o_ref, lse_ref = pu.oracle_attn(case, rows, sel.cpu().numpy(), pt.cpu().numpy())
    for where in ("device", "host"):
        kc, vc = case.k_cache, case.v_cache
        if where == "host":
            kc, vc = kc.cpu().pin_memory(), vc.cpu().pin_memory()
        kp, vp, ppt = msa.msa_gather_pages(d, pt, kc, vc)
        out = msa.msa_sparse_attn_decode(d, case.q, kp, vp, sel, ppt, case.row_pos, scale)
        torch.cuda.synchronize()
        ptc, pptc = pt.cpu(), ppt.cpu()
        assert torch.equal(pptc < 0, ptc < 0), where
        units = torch.arange(ptc.numel(), dtype=torch.int32).view_as(ptc)
        assert torch.equal(pptc[ptc >= 0], units[ptc >= 0]), where
        assert torch.equal(out[0], ref[0]) and torch.equal(out[1], ref[1]), where
        # the pool's partials and their merge against the oracle on the cache
        pu.check_partials(out[0].cpu(), out[1].cpu(), op, lp)
        o, lse = msa.msa_lse_merge(out[0], out[1])
        pu.check_output(o.cpu(), lse.cpu(), o_ref, lse_ref)


def test_host_cache_must_be_pinned():
    """A pageable host cache is refused before anything is launched."""
    import block_sparse_attention_09_amd as msa
    case = _build(seed=313, ctx_lens=[600], G=1, Hg=4, d_idx=64, k=2, poison=False)
    d = pu.dims_of(case)
    sel = msa.msa_topk_blocks(d, msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table,
                                                     case.row_pos, case.nb), case.row_pos, case.k)
    pt = msa.msa_build_page_table(d, sel, case.block_table)
    with pytest.raises(TypeError):
        msa.msa_sparse_attn_decode(d, case.q, case.k_cache.cpu(), case.v_cache.cpu(), sel, pt,
                                   case.row_pos)


@pytest.mark.parametrize("rows,H,nslot", [(33, 8, 9), (1100, 64, 5), (5500, 12, 3), (1030, 64, 18)])
def test_merge_matches_oracle_merge(rows, H, nslot):
    """The merge alone: oracle merge of exactly the bf16/fp32 partials the GPU merges
    (the three larger cases take the 512-thread workgroups: one with workgroups
    that straddle rows, one with two batches of slots)."""
    import block_sparse_attention_09_amd as msa
    print(f"[case] merge rows={rows} H={H} nslot={nslot}", flush=True)
    g = torch.Generator(device="cpu").manual_seed(5 + rows)
    op = torch.randn((rows, H, nslot, 128), generator=g).to(torch.bfloat16)
    lp = (torch.randn((rows, H, nslot), generator=g) * 4).float()
    lp[0, :, 2:] = -math.inf
    lp[1, 2, :] = -math.inf
    op[lp == -math.inf] = 0
    # partial LSEs in the C ABI's [rows][nslot][H] memory layout, viewed [row][head][slot]
    lp_dev = msa.empty_lse_part(rows, H, nslot, DEV)
    lp_dev.copy_(lp)
    with pytest.raises(ValueError):
        msa.msa_lse_merge(op.to(DEV), lp.to(DEV))  # [rows][H][nslot] memory: refused
    o, lse = msa.msa_lse_merge(op.to(DEV), lp_dev)
    o_ref, lse_ref = oracle.lse_merge(op.double().numpy(), lp.double().numpy())
    # the output is bf16: one rounding (at most half an ulp, <= 2^-8 relative) on
    # top of the fp32 sums
    err = np.abs(o.float().cpu().numpy() - o_ref)
    assert np.all(err <= 2.0 ** -8 * np.abs(o_ref) + 1e-3), float(np.max(err))
    l = lse.cpu().numpy()
    assert np.isneginf(l[1, 2]) and bool(torch.all(o[1, 2].cpu() == 0))
    fin = ~np.isneginf(lse_ref)
    assert np.allclose(l[fin], lse_ref[fin], rtol=1e-5, atol=1e-5)
    # partials of attention-output scale (a convex combination of N(0, 1) value
    # rows stays within a few units; a quarter of the draw keeps |o| <= ~1.2):
    # the attention bound itself, 1e-2 max-abs, holds for the merged output
    op4 = op * 0.25  # a power of two: exact in bf16
    o4, _ = msa.msa_lse_merge(op4.to(DEV), lp_dev)
    o4_ref, _ = oracle.lse_merge(op4.double().numpy(), lp.double().numpy())
    err4 = np.abs(o4.float().cpu().numpy() - o4_ref)
    assert float(np.max(err4)) <= pu.ATTN_ATOL, float(np.max(err4))


def test_empty_rows_is_noop():
    import block_sparse_attention_09_amd as msa
    case = _build(seed=401, ctx_lens=[300], G=2, Hg=4, d_idx=64, k=2)
    d = pu.dims_of(case)
    e = torch.empty((0, 2, 4, 64), dtype=torch.bfloat16, device=DEV)
    s = msa.msa_index_score(d, e, case.k_idx, case.block_table,
                            torch.empty(0, dtype=torch.int32, device=DEV), case.nb)
    assert s.shape == (0, 2, case.nb)


@pytest.mark.parametrize("form", ["decode", "decode-select", "decode-step", "prefill"])
def test_graph_replay_matches_eager(form):
    """The step captured in a HIP graph (five calls, or three with the fused
    select + decode attention): every replay (with eager work and
    synchronisations in between) equals the eager result bit for bit."""
    import block_sparse_attention_09_amd as msa
    prefill = form == "prefill"
    print(f"[case] graph replay {form}", flush=True)
    if prefill:
        case = _build(seed=501, ctx_lens=[2500], G=2, Hg=8, d_idx=128, k=3, prefill_rows=400)
    else:
        case = _build(seed=502, ctx_lens=[3000, 2000, 900], G=2, Hg=4, d_idx=64, k=4)
    d = pu.dims_of(case)
    dev = case.q.device
    scores = torch.empty((case.rows, case.G, case.nb), dtype=torch.float32, device=dev)
    sel = torch.empty((case.rows, case.G, case.nslot), dtype=torch.int32, device=dev)
    pt = torch.empty_like(sel)
    o_part = torch.empty((case.rows, case.H, case.nslot, 128), dtype=torch.bfloat16, device=dev)
    lse_part = msa.empty_lse_part(case.rows, case.H, case.nslot, dev)
    o = torch.empty((case.rows, case.H, 128), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.rows, case.H), dtype=torch.float32, device=dev)
    ws = torch.empty(msa.msa_prefill_workspace_size(d, case.rows, case.nslot, case.num_pages),
                     dtype=torch.uint8, device=dev)
    sync = torch.zeros(msa.decode_step_sync_words(case.rows, case.G), dtype=torch.int32,
                       device=dev)

    def step():
        if form == "decode-step":
            # the whole step as one kernel, its sync words reused by every replay
            msa.msa_decode_step(d, case.q_idx, case.k_idx, case.block_table, case.row_pos,
                                case.nb, case.k, case.q, case.k_cache, case.v_cache,
                                row_req=case.row_req, num_reqs=case.num_reqs,
                                mode=msa.MSA_STEP_ONE_LAUNCH, sync=sync, scores=scores, sel=sel,
                                page_table=pt, o_part=o_part, lse_part=lse_part, o=o, lse=lse)
            return
        msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos, case.nb,
                            row_req=case.row_req, num_reqs=case.num_reqs, scores=scores)
        if form == "decode-select":
            msa.msa_sparse_attn_decode_select(d, scores, case.k, case.block_table, case.q,
                                              case.k_cache, case.v_cache, case.row_pos,
                                              row_req=case.row_req, sel=sel, page_table=pt,
                                              o_part=o_part, lse_part=lse_part)
            msa.msa_lse_merge(o_part, lse_part, o=o, lse=lse)
            return
        msa.msa_topk_blocks(d, scores, case.row_pos, case.k, sel=sel)
        msa.msa_build_page_table(d, sel, case.block_table, row_req=case.row_req, page_table=pt)
        if prefill:
            msa.msa_sparse_attn_prefill(d, case.q, case.k_cache, case.v_cache, sel, pt,
                                        case.row_pos, case.num_pages, workspace=ws,
                                        o_part=o_part, lse_part=lse_part)
        else:
            msa.msa_sparse_attn_decode(d, case.q, case.k_cache, case.v_cache, sel, pt,
                                       case.row_pos, o_part=o_part, lse_part=lse_part)
        msa.msa_lse_merge(o_part, lse_part, o=o, lse=lse)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (scores, sel, pt, o_part, lse_part, o, lse)]
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    for rep in range(3):
        for t in (scores, o_part, o):
            t.zero_()
        sel.fill_(-7)
        pt.fill_(-7)
        lse_part.fill_(1.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip((scores, sel, pt, o_part, lse_part, o, lse), ref):
            assert torch.equal(a, b), f"replay {rep} differs"
        assert int(torch.count_nonzero(sync)) == 0, f"replay {rep}: sync words left set"
        step()  # eager work between replays
        torch.cuda.synchronize()
