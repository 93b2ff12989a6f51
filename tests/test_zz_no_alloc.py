"""The allocation-free prefill call (msa_sparse_attn_prefill_noalloc) against
msa_sparse_attn_prefill with a caller workspace: bit-identical partials on two
calls in a row, the second with a smaller input (the static scratch keeps the
first call's contents, which must not leak into the second), and both against
the oracle.  A prefill whose workspace exceeds the static scratch is refused
before anything is launched."""
import ctypes

import numpy as np
import pytest
import torch

import msa_synth
import parity_util as pu

pytestmark = pytest.mark.gpu


def _selection(case):
    import block_sparse_attention_09_amd as msa
    d = pu.dims_of(case)
    scores = msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos,
                                 case.nb, row_req=case.row_req, num_reqs=case.num_reqs)
    return msa.msa_topk_blocks_paged(d, scores, case.row_pos, case.k, case.block_table,
                                     row_req=case.row_req)


def test_noalloc_prefill_matches_workspace_call():
    import block_sparse_attention_09_amd as msa
    cases = [
        # first call: 3 requests, 650 rows, 4 groups x 8 heads, NaN-poisoned tails
        dict(seed=401, ctx_lens=[2000, 900, 1500], G=4, Hg=8, d_idx=128, k=4,
             prefill_rows=[150, 200, 300], paged=True, poison="nan"),
        # second call, smaller: 1 request, 96 rows, 2 groups, fewer pages
        dict(seed=402, ctx_lens=[700], G=2, Hg=8, d_idx=64, k=2, prefill_rows=96,
             paged=True, poison="nan"),
    ]
    for i, kw in enumerate(cases):
        print(f"[case] noalloc prefill call {i + 1}", flush=True)
        case = msa_synth.build_case("t", device="cuda", **kw)
        d = pu.dims_of(case)
        sel, pt = _selection(case)
        scale = 0.088
        ref = msa.msa_sparse_attn_prefill(d, case.q, case.k_cache, case.v_cache, sel, pt,
                                          case.row_pos, case.num_pages, scale)
        # outputs pre-filled with garbage: the call must write every element
        o_part = torch.full_like(ref[0], 7.0)
        lse_part = msa.empty_lse_part(case.rows, case.H, case.nslot, "cuda").fill_(3.0)
        got = msa.msa_sparse_attn_prefill_noalloc(d, case.q, case.k_cache, case.v_cache, sel,
                                                  pt, case.row_pos, case.num_pages, scale,
                                                  o_part=o_part, lse_part=lse_part)
        torch.cuda.synchronize()
        assert torch.equal(got[0].view(torch.int16), ref[0].view(torch.int16)), i
        assert torch.equal(got[1].view(torch.int32), ref[1].view(torch.int32)), i
        rows = list(range(case.rows))
        op, lp, o, lse = pu.oracle_attn(case, rows, sel.cpu().numpy(), pt.cpu().numpy(),
                                        sm_scale=scale)
        pu.check_partials(got[0].cpu(), got[1].cpu(), op, lp)
        om, lm = msa.msa_lse_merge(got[0], got[1])
        pu.check_output(om.cpu(), lm.cpu(), o, lse)


def test_noalloc_prefill_rejects_oversized_workspace():
    """Host-side refusal: no launch, MSA_ERR_WORKSPACE, message names the limit."""
    import block_sparse_attention_09_amd as msa
    from block_sparse_attention_09_amd import binding
    lib = msa.load()
    d = msa.Dims(G=8, Hg=8, D=128, n_idx=4, d_idx=128, blk=128)
    rows, nslot, pages = 65536, 33, 8192
    assert msa.msa_prefill_workspace_size(d, rows, nslot, pages) > (16 << 20)
    fake = ctypes.c_void_p(0x10000)
    view = binding.View(fake.value, 8 * 128 * 128, 128 * 128, 128)
    st = lib.msa_sparse_attn_prefill_noalloc(ctypes.byref(d), rows, fake, view, view, fake,
                                             fake, nslot, fake, pages, ctypes.c_float(0.088),
                                             fake, fake, None)
    assert st == 4, st      # MSA_ERR_WORKSPACE
    assert b"static scratch" in lib.msa_last_error()
