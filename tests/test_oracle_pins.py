"""Pins for the CPU oracle: each check ties the oracle to something other than
itself (hand-derived fixtures, closed forms, exact integer brute force through a
library matmul, a set-property brute force, library attention, merge
identities).  CPU only."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import msa_synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")
BLK = 128


def _f(x):
    return -np.inf if x == "-inf" else float(x)


def to_bits(a) -> np.ndarray:
    """float array (values exactly representable in bf16) -> bf16 bit patterns."""
    t = torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
    back = t.to(torch.float32).numpy()
    assert np.array_equal(back, np.asarray(a, dtype=np.float32)), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


# ============================================================================ index score
def test_score_hand_fixture(oracle_mod):
    fx = json.load(open(os.path.join(GOLD, "score_hand.json")))
    d = fx["d_idx"]
    q = np.zeros((1, 1, 2, d), np.float32)
    q[0, 0, 0, 0] = 1.0
    q[0, 0, 1, 1] = 2.0
    pool = np.full((2, 1, BLK, d), 100.0, np.float32)
    bt = np.array([fx["block_table"]], np.int32)
    for t in range(fx["pos"] + 1):
        page, slot = bt[0, t // BLK], t % BLK
        pool[page, 0, slot, :] = 1.0
        pool[page, 0, slot, 0] = (7 * t) % 11 - 5
        pool[page, 0, slot, 1] = (3 * t) % 5 - 2
    s = oracle_mod.index_score(to_bits(q), to_bits(pool), bt, np.array([fx["pos"]]), fx["nb"])
    assert s[0, 0].tolist() == [_f(x) for x in fx["expected"]]


def _int_case(rng, ctx, G, n_idx, d_idx, paged, lo=None):
    """Small-integer inputs: every sum is exact in fp32 and fp64."""
    R = len(ctx)
    nblk = [(L + BLK - 1) // BLK for L in ctx]
    P = sum(nblk) + 3
    perm = rng.permutation(P) if paged else np.arange(P)
    bt = np.zeros((R, max(nblk)), np.int32)
    off = 0
    for r in range(R):
        bt[r, :nblk[r]] = perm[off:off + nblk[r]]
        off += nblk[r]
    q = rng.integers(-3, 4, size=(R, G, n_idx, d_idx)).astype(np.float32)
    pool = rng.integers(-3, 4, size=(P, G, BLK, d_idx)).astype(np.float32)
    return q, pool, bt, max(nblk)


def _dense_scores_bruteforce(q, pool, bt, ctx, pos, nb, lo):
    """Gather each request's keys densely and score with an integer matmul."""
    R, G, n_idx, d_idx = q.shape
    out = np.full((R, G, nb), -np.inf)
    for r in range(R):
        L = ctx[r]
        dense = np.concatenate([pool[bt[r, b]] for b in range((L + BLK - 1) // BLK)], axis=1)
        dense = dense[:, :L].astype(np.int64)                      # [G][L][d]
        for g in range(G):
            tok = (q[r, g].astype(np.int64) @ dense[g].T).sum(axis=0)   # [L] exact
            tok = tok.astype(np.float64) / math.sqrt(d_idx)
            tok[np.arange(L) > pos[r]] = -np.inf
            own = pos[r] // BLK
            for b in range(nb):
                if b == own or (lo[r][g] <= b < own):
                    out[r, g, b] = tok[b * BLK:min(L, (b + 1) * BLK)].max()
    return out


@pytest.mark.parametrize("d_idx", [64, 128])
@pytest.mark.parametrize("paged", [False, True])
def test_score_integer_bruteforce(oracle_mod, d_idx, paged):
    rng = np.random.default_rng(7 + d_idx + paged)
    ctx = [700, 1024, 129, 128]
    G, n_idx = 2, 4
    q, pool, bt, nb = _int_case(rng, ctx, G, n_idx, d_idx, paged)
    pos = np.array([L - 1 for L in ctx], np.int32)
    lo = np.array([[0, 2], [1, 0], [3, 0], [0, 0]], np.int32)   # row 2: lo above own
    got = oracle_mod.index_score(to_bits(q), to_bits(pool), bt, pos, nb + 1, blk_lo=lo)
    want = _dense_scores_bruteforce(q, pool, bt, ctx, pos, nb + 1, lo)
    if d_idx == 64:
        assert np.array_equal(got, want)        # /8 is exact
    else:
        np.testing.assert_allclose(got, want, rtol=1e-15, atol=0)
        assert np.array_equal(np.isinf(got), np.isinf(want))


def test_score_prefill_rows_causal(oracle_mod):
    """Rows of one request at consecutive positions: each row only sees t <= pos."""
    rng = np.random.default_rng(3)
    L = 900
    q1, pool, bt, nb = _int_case(rng, [L], 2, 4, 64, True)
    rows = 40
    pos = np.arange(L - rows, L, dtype=np.int32)
    q = rng.integers(-3, 4, size=(rows, 2, 4, 64)).astype(np.float32)
    got = oracle_mod.index_score(to_bits(q), to_bits(pool), bt, pos, nb,
                                 row_req=np.zeros(rows, np.int32))
    for i in range(rows):
        want = _dense_scores_bruteforce(q[i:i + 1], pool, bt, [L], pos[i:i + 1], nb,
                                        np.zeros((1, 2), np.int32))
        assert np.array_equal(got[i:i + 1], want)


def test_score_zero_keys(oracle_mod):
    case = msa_synth.build_case("z", seed=5, ctx_lens=[1000, 300], G=2, Hg=1, d_idx=64, k=2,
                                lo_frac=0.5)
    case.k_idx.zero_()
    s = oracle_mod.index_score(msa_synth.bits(case.q_idx), msa_synth.bits(case.k_idx),
                               case.block_table.numpy(), case.row_pos.numpy(), case.nb,
                               blk_lo=case.blk_lo.numpy())
    for r in range(2):
        own = int(case.row_pos[r]) // BLK
        for g in range(2):
            lo = int(case.blk_lo[r, g])
            fin = np.isfinite(s[r, g])
            assert np.all(s[r, g][fin] == 0.0)
            assert set(np.nonzero(fin)[0]) == set(range(min(lo, own), own)) | {own}


def test_score_planted_block_closed_form(oracle_mod):
    """k_t = qbar for every token of one block gives exactly |qbar|^2/sqrt(d) there,
    which beats every block whose keys are shorter than qbar (Cauchy-Schwarz)."""
    rng = np.random.default_rng(11)
    d = 64
    q = rng.integers(-2, 3, size=(1, 1, 4, d)).astype(np.float32)
    qbar = q[0, 0].sum(axis=0)
    L = 12 * BLK
    pool = rng.integers(-1, 2, size=(12, 1, BLK, d)).astype(np.float32) * 0.125
    planted = 7
    pool[planted, 0, :, :] = qbar
    bt = np.arange(12, dtype=np.int32)[None]
    s = oracle_mod.index_score(to_bits(q), to_bits(pool), bt, np.array([L - 1]), 12)
    assert s[0, 0, planted] == float(qbar @ qbar) / 8.0
    assert int(np.argmax(s[0, 0])) == planted


def test_score_positive_scaling(oracle_mod):
    case = msa_synth.build_case("s", seed=9, ctx_lens=[777], G=2, Hg=1, d_idx=128, k=2)
    args = (msa_synth.bits(case.k_idx), case.block_table.numpy(), case.row_pos.numpy(), case.nb)
    s1 = oracle_mod.index_score(msa_synth.bits(case.q_idx), *args)
    s2 = oracle_mod.index_score(msa_synth.bits(case.q_idx * 2), *args)   # exact in bf16
    assert np.array_equal(s2, 2 * s1)


def test_score_layout_and_permutation_invariance(oracle_mod):
    """Paged vs contiguous placement, and a token-major cache view, give identical
    scores (the page-table gather equals a contiguous gather)."""
    case = msa_synth.build_case("p", seed=21, ctx_lens=[650, 1300], G=2, Hg=1, d_idx=64, k=2,
                                paged=True)
    kb = msa_synth.bits(case.k_idx)
    bt = case.block_table.numpy()
    pos = case.row_pos.numpy()
    s_paged = oracle_mod.index_score(msa_synth.bits(case.q_idx), kb, bt, pos, case.nb)
    # contiguous: rebuild the pool in logical order
    nblk = [(int(L) + BLK - 1) // BLK for L in case.ctx_len]
    order = np.concatenate([bt[r, :nblk[r]] for r in range(2)])
    contig = np.ascontiguousarray(kb[order])
    bt_c = np.zeros_like(bt)
    bt_c[0, :nblk[0]] = np.arange(nblk[0])
    bt_c[1, :nblk[1]] = nblk[0] + np.arange(nblk[1])
    s_contig = oracle_mod.index_score(msa_synth.bits(case.q_idx), contig, bt_c, pos, case.nb)
    assert np.array_equal(s_paged, s_contig)
    # token-major physical layout [page][token][group][dim] seen through strides
    tm = np.ascontiguousarray(kb.transpose(0, 2, 1, 3))
    view = tm.transpose(0, 2, 1, 3)
    s_tm = oracle_mod.index_score(msa_synth.bits(case.q_idx), view, bt, pos, case.nb)
    assert np.array_equal(s_paged, s_tm)


# ============================================================================ top-k
def test_topk_hand_fixture(oracle_mod):
    fx = json.load(open(os.path.join(GOLD, "topk_hand.json")))
    scores = np.array([[[_f(x) for x in g] for g in row["scores"]] for row in fx["rows"]],
                      np.float32)
    pos = np.array([row["pos"] for row in fx["rows"]], np.int32)
    sel = oracle_mod.topk(scores, pos, fx["k"])
    assert sel.tolist() == fx["expected_sel"]
    pt = oracle_mod.page_table(sel, np.array(fx["block_table"], np.int32),
                               row_req=np.zeros(len(pos), np.int32))
    assert pt.tolist() == fx["expected_page_table"]


def _dominance_bruteforce(scores, own, k):
    """The unique subset S of the candidates, of size min(k, |C|), such that every
    member outranks every non-member: higher score, or equal score and lower index."""
    cand = [b for b in range(own) if scores[b] != -np.inf]
    m = min(k, len(cand))
    found = []
    for S in itertools.combinations(cand, m):
        rest = [c for c in cand if c not in S]
        if all(scores[b] > scores[c] or (scores[b] == scores[c] and b < c)
               for b in S for c in rest):
            found.append(S)
    assert len(found) == 1
    return sorted(found[0] + (own,))


def test_topk_set_property_bruteforce(oracle_mod):
    rng = np.random.default_rng(1234)
    levels = np.array([-1.5, 0.0, 0.25, 0.25, 1.0, 2.0], np.float32)   # many exact ties
    for trial in range(60):
        own = int(rng.integers(0, 10))
        nb = own + 1 + int(rng.integers(0, 3))
        G = 2
        sc = rng.choice(levels, size=(1, G, nb)).astype(np.float32)
        sc[0, :, own + 1:] = -np.inf
        if own > 2 and trial % 3 == 0:
            sc[0, 1, :own // 2] = -np.inf            # a lower bound on candidates
        pos = np.array([own * BLK + int(rng.integers(0, BLK))], np.int32)
        for k in range(0, own + 2):
            sel = oracle_mod.topk(sc, pos, k)
            for g in range(G):
                want = _dominance_bruteforce(sc[0, g], own, k)
                assert sel[0, g].tolist() == want + [-1] * (k + 1 - len(want))


def test_topk_special_cases(oracle_mod):
    own = 20
    pos = np.array([own * BLK + 5], np.int32)
    ties = np.zeros((1, 1, 32), np.float32)
    assert oracle_mod.topk(ties, pos, 4)[0, 0].tolist() == [0, 1, 2, 3, own]
    rnd = np.random.default_rng(0).standard_normal((1, 1, 32)).astype(np.float32)
    assert oracle_mod.topk(rnd, pos, 50)[0, 0].tolist() == list(range(own + 1)) + [-1] * 30
    assert oracle_mod.topk(rnd, pos, 0)[0, 0].tolist() == [own]
    first = np.array([own * 0 + 3], np.int32)     # own block 0: nothing to rank
    assert oracle_mod.topk(rnd, first, 3)[0, 0].tolist() == [0, -1, -1, -1]


# ============================================================================ attention
def _dense_sdpa(case, rows_idx=None):
    """Dense causal attention through torch's library routine, fp64 on the CPU."""
    q = case.q.to(torch.float64)
    out_o, out_lse = [], []
    for r in (rows_idx if rows_idx is not None else range(case.rows)):
        req = int(case.row_req[r])
        L = int(case.ctx_len[req])
        nblk = (L + BLK - 1) // BLK
        pages = case.block_table[req, :nblk].long()
        K = case.k_cache[pages].to(torch.float64)            # [nblk][G][128][D]
        V = case.v_cache[pages].to(torch.float64)
        K = K.permute(1, 0, 2, 3).reshape(case.G, nblk * BLK, case.D)[:, :L]
        V = V.permute(1, 0, 2, 3).reshape(case.G, nblk * BLK, case.D)[:, :L]
        K = K.repeat_interleave(case.Hg, dim=0)              # GQA: head h uses group h // Hg
        V = V.repeat_interleave(case.Hg, dim=0)
        pos = int(case.row_pos[r])
        mask = (torch.arange(L) <= pos)[None, None, :]
        qr = q[r][:, None, :]                                # [H][1][D]
        o = torch.nn.functional.scaled_dot_product_attention(
            qr, K, V, attn_mask=mask, scale=1.0 / math.sqrt(case.D))
        logits = (qr @ K.transpose(1, 2)) / math.sqrt(case.D)
        lse = torch.logsumexp(logits.masked_fill(~mask, -math.inf), dim=-1)
        out_o.append(o[:, 0].numpy())
        out_lse.append(lse[:, 0].numpy())
    return np.stack(out_o), np.stack(out_lse)


def _sel_all(case, rows_idx):
    own = case.row_pos.numpy()[rows_idx] // BLK
    nslot = case.nb
    sel = np.full((len(rows_idx), case.G, nslot), -1, np.int32)
    for i, o in enumerate(own):
        sel[i, :, :o + 1] = np.arange(o + 1)
    return sel


@pytest.mark.parametrize("prefill", [False, True])
def test_attn_all_blocks_equals_dense_causal(oracle_mod, prefill):
    if prefill:
        case = msa_synth.build_case("d", seed=31, ctx_lens=[1000], G=2, Hg=4, d_idx=64, k=8,
                                    prefill_rows=6, poison=True)
    else:
        case = msa_synth.build_case("d", seed=31, ctx_lens=[700, 1000, 128], G=2, Hg=4,
                                    d_idx=64, k=8, poison=True)
    rows = list(range(case.rows))
    sel = _sel_all(case, rows)
    pt = oracle_mod.page_table(sel, case.block_table.numpy(), case.row_req.numpy())
    o, lse = oracle_mod.attn(msa_synth.bits(case.q), msa_synth.bits(case.k_cache),
                             msa_synth.bits(case.v_cache), sel, pt, case.row_pos.numpy(),
                             1.0 / math.sqrt(case.D))
    o_ref, lse_ref = _dense_sdpa(case, rows)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=0)
    # top-k with k >= every candidate count selects exactly every block
    s = oracle_mod.index_score(msa_synth.bits(case.q_idx), msa_synth.bits(case.k_idx),
                               case.block_table.numpy(), case.row_pos.numpy(), case.nb,
                               row_req=case.row_req.numpy())
    assert np.array_equal(oracle_mod.topk(s.astype(np.float32), case.row_pos.numpy(),
                                          case.nb - 1), sel)


def test_attn_constant_values(oracle_mod):
    case = msa_synth.build_case("c", seed=41, ctx_lens=[900, 333], G=2, Hg=2, d_idx=64, k=3,
                                paged=True)
    vec = torch.tensor([[0.5, -1.25], [2.0, 0.75]], dtype=torch.float32)   # per group
    for g in range(2):
        case.v_cache[:, g, :, :] = vec[g].repeat(64).to(torch.bfloat16)
    sel = np.full((2, 2, 4), -1, np.int32)
    sel[0, :, :3] = [[0, 3, 7], [1, 2, 7]]
    sel[1, :, :2] = [[0, 2], [1, 2]]
    pt = oracle_mod.page_table(sel, case.block_table.numpy())
    o, _ = oracle_mod.attn(msa_synth.bits(case.q), msa_synth.bits(case.k_cache),
                           msa_synth.bits(case.v_cache), sel, pt, case.row_pos.numpy(), 0.088)
    for h in range(4):
        want = vec[h // 2].repeat(64).numpy().astype(np.float64)
        np.testing.assert_allclose(o[:, h], np.broadcast_to(want, (2, 128)), atol=1e-13)


def test_attn_dominant_logit(oracle_mod):
    case = msa_synth.build_case("m", seed=43, ctx_lens=[640], G=1, Hg=1, d_idx=64, k=4)
    page, slot = int(case.block_table[0, 2]), 17
    case.q[0, 0] = (case.k_cache[page, 0, slot].to(torch.float32) * 8).to(torch.bfloat16)
    sel = np.array([[[0, 2, 4, -1, -1]]], np.int32)
    pt = oracle_mod.page_table(sel, case.block_table.numpy())
    o, _ = oracle_mod.attn(msa_synth.bits(case.q), msa_synth.bits(case.k_cache),
                           msa_synth.bits(case.v_cache), sel, pt, case.row_pos.numpy(), 1.0)
    want = case.v_cache[page, 0, slot].to(torch.float64).numpy()
    np.testing.assert_allclose(o[0, 0], want, atol=1e-6)


def test_attn_own_block_only(oracle_mod):
    """k = 0: attention over the own block alone equals dense attention on a
    context that holds only that block's visible tokens."""
    case = msa_synth.build_case("o", seed=47, ctx_lens=[1000], G=2, Hg=2, d_idx=64, k=0,
                                prefill_rows=3)
    pos = case.row_pos.numpy()
    s = oracle_mod.index_score(msa_synth.bits(case.q_idx), msa_synth.bits(case.k_idx),
                               case.block_table.numpy(), pos, case.nb,
                               row_req=case.row_req.numpy())
    sel = oracle_mod.topk(s.astype(np.float32), pos, 0)
    assert np.all(sel[..., 0] == (pos // BLK)[:, None])
    pt = oracle_mod.page_table(sel, case.block_table.numpy(), case.row_req.numpy())
    o, lse = oracle_mod.attn(msa_synth.bits(case.q), msa_synth.bits(case.k_cache),
                             msa_synth.bits(case.v_cache), sel, pt, pos, 1 / math.sqrt(128))
    for i, p in enumerate(pos):
        b = p // BLK
        K = case.k_cache[int(case.block_table[0, b])].to(torch.float64)[:, :p % BLK + 1]
        V = case.v_cache[int(case.block_table[0, b])].to(torch.float64)[:, :p % BLK + 1]
        K, V = K.repeat_interleave(2, 0), V.repeat_interleave(2, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            case.q[i].to(torch.float64)[:, None], K, V, scale=1 / math.sqrt(128))[:, 0]
        np.testing.assert_allclose(o[i], ref.numpy(), atol=1e-12)


# ============================================================================ merge
def test_merge_of_partials_equals_single_softmax(oracle_mod):
    case = msa_synth.build_case("u", seed=51, ctx_lens=[1500, 900, 257], G=2, Hg=4, d_idx=64,
                                k=3, paged=True, poison=True)
    pos = case.row_pos.numpy()
    s = oracle_mod.index_score(msa_synth.bits(case.q_idx), msa_synth.bits(case.k_idx),
                               case.block_table.numpy(), pos, case.nb)
    sel = oracle_mod.topk(s.astype(np.float32), pos, case.k)
    pt = oracle_mod.page_table(sel, case.block_table.numpy())
    args = (msa_synth.bits(case.q), msa_synth.bits(case.k_cache), msa_synth.bits(case.v_cache),
            sel, pt, pos, 1 / math.sqrt(128))
    o, lse = oracle_mod.attn(*args)
    op, lp = oracle_mod.attn_partials(*args)
    assert np.all(np.isinf(lp[2, :, 3:]))          # 3rd request: 3 blocks -> 1 padded slot
    om, lm = oracle_mod.lse_merge(op, lp)
    np.testing.assert_allclose(om, o, atol=1e-12)
    np.testing.assert_allclose(lm, lse, rtol=1e-13)


def test_merge_identities(oracle_mod):
    rng = np.random.default_rng(5)
    D = 8
    o1, o2 = rng.standard_normal(D), rng.standard_normal(D)
    op = np.zeros((1, 4, 3, D))
    lp = np.full((1, 4, 3), -np.inf)
    op[0, 0, 1], lp[0, 0, 1] = o1, 0.7                       # one finite slot: identity
    op[0, 1, 0], op[0, 1, 2], lp[0, 1, 0], lp[0, 1, 2] = o1, o2, -2.0, -2.0   # equal weights
    op[0, 2, 0], op[0, 2, 1], lp[0, 2, 0], lp[0, 2, 1] = o1, o2, math.log(3.0), 0.0
    o, lse = oracle_mod.lse_merge(op, lp)
    np.testing.assert_allclose(o[0, 0], o1, atol=1e-15)
    assert lse[0, 0] == 0.7
    np.testing.assert_allclose(o[0, 1], (o1 + o2) / 2, atol=1e-15)
    np.testing.assert_allclose(lse[0, 1], -2.0 + math.log(2.0), atol=1e-15)
    np.testing.assert_allclose(o[0, 2], 0.75 * o1 + 0.25 * o2, atol=1e-15)
    np.testing.assert_allclose(lse[0, 2], math.log(4.0), atol=1e-15)
    assert np.all(o[0, 3] == 0) and lse[0, 3] == -np.inf     # nothing selected
    # shift invariance of the weights
    lp2 = lp + 5.0
    o_s, lse_s = oracle_mod.lse_merge(op, lp2)
    np.testing.assert_allclose(o_s[0, :3], o[0, :3], atol=1e-14)
    np.testing.assert_allclose(lse_s[0, :3], lse[0, :3] + 5.0, atol=1e-13)


def test_prefill_rows_equal_decode_rows(oracle_mod):
    """A prefill row at position p computes what a decode row at p computes."""
    pre = msa_synth.build_case("pr", seed=61, ctx_lens=[1200], G=2, Hg=2, d_idx=64, k=3,
                               prefill_rows=5, paged=True)
    res = oracle_mod.decode_path(msa_synth.bits(pre.q_idx), msa_synth.bits(pre.k_idx),
                                 msa_synth.bits(pre.q), msa_synth.bits(pre.k_cache),
                                 msa_synth.bits(pre.v_cache), pre.block_table.numpy(),
                                 pre.row_pos.numpy(), pre.k, pre.nb, 1 / math.sqrt(128),
                                 row_req=pre.row_req.numpy())
    bt5 = np.repeat(pre.block_table.numpy(), 5, axis=0)       # 5 requests, same cache
    dec = oracle_mod.decode_path(msa_synth.bits(pre.q_idx), msa_synth.bits(pre.k_idx),
                                 msa_synth.bits(pre.q), msa_synth.bits(pre.k_cache),
                                 msa_synth.bits(pre.v_cache), bt5, pre.row_pos.numpy(), pre.k,
                                 pre.nb, 1 / math.sqrt(128))
    for key in ("scores", "sel", "pt", "o", "lse"):
        assert np.array_equal(res[key], dec[key]), key
