"""Benchmark of the MSA hot path on one MI355X.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--workloads 2,5,3,4,1]

A step is one pass of the whole path over one batch: index scores, top-k, the
page table, sparse attention (decode kernel, or the KV-block-major prefill), LSE
merge.  Decode with the caches in device memory runs top-k, page table and
decode attention as one call (msa_sparse_attn_decode_select, one kernel up to
1,024 blocks per row when the batch fits one round of the GPU); prefill and the run with K/V in host memory call
msa_topk_blocks_paged (one kernel for top-k and page table) and then the
attention.  Every decode workload is also timed as the four separate calls, for
the per-call figures.  The headline line is
the decode workload at 64K context, batch 8 (8 KV groups x 8 heads, d_idx 128,
top-16 + own block, paged): value = decode tokens/s of one MSA layer
= batch x steps / time.  Each timed step starts from cold caches (an untimed
1 GiB read runs before it) and is timed by its own HIP event pair;
the same replays back to back, caches warm, are reported beside it.

Also reported on the same line:
  roofline      the index-score kernel (dominant: >90% of the step's bytes)
                against 8 TB/s HBM, from HIP events around every launch in the
                timed region; traffic from the committed rocprofv3 counter
                summary when it was taken on the current kernel source
  cpu_baseline  the CPU oracle on the host cores over the same batch (every
                workload entry carries its own oracle timing, per stage)
  workloads     the other seeded workloads (1M-context decode, ragged decode,
                prefill chunk, 4K latency case), each timed the same way
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tok/s + index-scan HBM GB/s @64K/1M ctx; prefill sparse-attn TFLOP/s"
HBM_PEAK_GBPS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FLUSH_BYTES = 1 << 30
MAIN = 2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_index_score_decode-64k-b8.json")
# the index-score kernel's sources (the counter summary names their hash)
KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_09_amd", "csrc", f)
               for f in ("index_score.hip", "index_score_dev.h")]
# the same for the block-major prefill attention kernel
ATTN_TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                                 "traffic_attn_blockmajor_prefill-8k-on-60k.json")
ATTN_KERNEL_SRCS = [os.path.join(ROOT, "block_sparse_attention_09_amd", "csrc", "attn.hip")]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workloads", default="2,5,3,4,1",
                    help="comma list of workload ids; the first is the headline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kv-on-host", action="store_true",
                    help="skip the extra run of the headline workload with K/V in pinned host memory")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain 1-read/1-write fp32 elementwise kernel over this "
                         "many MiB (reference for rocprofv3 FETCH_SIZE/WRITE_SIZE scaling)")
    ap.add_argument("--eager-only", action="store_true",
                    help="time the eager step only (no graph capture), for counter runs")
    ap.add_argument("--no-slab-sweep", action="store_true",
                    help="skip the prefill slab-size sweep (so that a kernel trace holds only "
                         "the full-batch attention launches)")
    return ap.parse_args()


def algorithmic(case, sel=None):
    """Bytes and FLOPs the method itself must move / compute (not the dense work
    it avoids)."""
    import numpy as np
    pos = case.row_pos.cpu().numpy().astype(np.int64)
    G, d_idx, n_idx, D, H = case.G, case.d_idx, case.n_idx, case.D, case.H
    kidx = int(((pos + 1) * G * d_idx * 2).sum())                # visible key-index tokens
    qidx = case.rows * G * n_idx * d_idx * 2
    score_out = case.rows * G * case.nb * 4
    out = dict(kidx=kidx, qidx=qidx, score_bytes=kidx + qidx + score_out,
               index_flops=float(((pos + 1) * G * n_idx * d_idx * 2).sum()))
    if sel is not None:
        s = sel.cpu().numpy().astype(np.int64)
        valid = s >= 0
        own = (pos // 128)[:, None, None]
        vis = np.where(s == own, (pos % 128 + 1)[:, None, None], 128)
        tokens = int((vis * valid).sum())                           # per (row, group)
        nsel = valid.sum()
        out["attn_flops"] = 4.0 * D * tokens * case.Hg             # QK^T and PV, per head
        out["kv_bytes"] = int(nsel) * 128 * D * 2 * 2
        out["qo_bytes"] = case.rows * H * D * 2 * 2
        out["part_bytes"] = int(case.rows * H * case.nslot * (D * 2 + 4))
    return out


def run_workload(cfg, steps, warmup, graph_replay=True, kv_on_host=False, slab_sweep=True):
    import torch
    import block_sparse_attention_09_amd as msa
    import msa_synth

    case = msa_synth.config_case(cfg, device="cuda")
    if kv_on_host:
        # decoupled offload: key index on the GPU, K/V in pinned host memory,
        # read by the attention kernel page by page as the selection names them
        case.k_cache = case.k_cache.cpu().pin_memory()
        case.v_cache = case.v_cache.cpu().pin_memory()
        case.name += "-kv-on-host"
        torch.cuda.empty_cache()
    d = msa.Dims(G=case.G, Hg=case.Hg, D=case.D, n_idx=case.n_idx, d_idx=case.d_idx, blk=128)
    scale = 1.0 / math.sqrt(case.D)
    dev = case.q.device
    # outputs and workspace allocated once, outside the timed region
    scores = torch.empty((case.rows, case.G, case.nb), dtype=torch.float32, device=dev)
    sel = torch.empty((case.rows, case.G, case.nslot), dtype=torch.int32, device=dev)
    pt = torch.empty_like(sel)
    o_part = torch.empty((case.rows, case.H, case.nslot, case.D), dtype=torch.bfloat16,
                         device=dev)
    lse_part = msa.empty_lse_part(case.rows, case.H, case.nslot, dev)
    o = torch.empty((case.rows, case.H, case.D), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((case.rows, case.H), dtype=torch.float32, device=dev)
    ws = None
    if case.prefill:
        nbytes = msa.msa_prefill_workspace_size(d, case.rows, case.nslot, case.num_pages)
        ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    names = ["index_score", "topk_page_table", "attn", "merge"]
    gather = kv_on_host and not case.prefill
    if gather:
        # on-demand load: the selected pages are copied from host memory into a
        # device pool before decode attention (buffers allocated here, once)
        names = ["index_score", "topk_page_table", "gather", "attn", "merge"]
        units = case.rows * case.G * case.nslot
        pool_k = torch.empty((units, 128, case.D), dtype=torch.bfloat16, device=dev)
        pool_v = torch.empty_like(pool_k)
        pool_pt = torch.empty_like(pt)

    def step(ev=None):
        i = 0

        def mark():
            nonlocal i
            if ev is not None:
                ev[i].record()
            i += 1
        mark()
        msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos, case.nb,
                            row_req=case.row_req, blk_lo=case.blk_lo, num_reqs=case.num_reqs,
                            scores=scores)
        mark()
        msa.msa_topk_blocks_paged(d, scores, case.row_pos, case.k, case.block_table,
                                  row_req=case.row_req, sel=sel, page_table=pt)
        mark()
        kc, vc, ptab = case.k_cache, case.v_cache, pt
        if gather:
            kc, vc, ptab = msa.msa_gather_pages(d, pt, case.k_cache, case.v_cache, dst_k=pool_k,
                                                dst_v=pool_v, dst_page_table=pool_pt)
            mark()
        if case.prefill:
            msa.msa_sparse_attn_prefill(d, case.q, kc, vc, sel, ptab, case.row_pos,
                                        case.num_pages, scale, workspace=ws,
                                        o_part=o_part, lse_part=lse_part)
        else:
            msa.msa_sparse_attn_decode(d, case.q, kc, vc, sel, ptab, case.row_pos, scale,
                                       o_part=o_part, lse_part=lse_part)
        mark()
        msa.msa_lse_merge(o_part, lse_part, o=o, lse=lse)
        mark()

    # Decode with the caches in device memory: the step that is timed and graphed
    # runs selection, page table and decode attention as one call
    # (msa_sparse_attn_decode_select); the four-call step above is timed first
    # for the per-call breakdown.
    fused = not case.prefill and not gather
    fused_names = ["index_score", "select_attn", "merge"]

    def step_fused(ev=None):
        i = 0

        def mark():
            nonlocal i
            if ev is not None:
                ev[i].record()
            i += 1
        mark()
        msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos, case.nb,
                            row_req=case.row_req, blk_lo=case.blk_lo, num_reqs=case.num_reqs,
                            scores=scores)
        mark()
        msa.msa_sparse_attn_decode_select(d, scores, case.k, case.block_table, case.q,
                                          case.k_cache, case.v_cache, case.row_pos,
                                          row_req=case.row_req, sm_scale=scale, sel=sel,
                                          page_table=pt, o_part=o_part, lse_part=lse_part)
        mark()
        msa.msa_lse_merge(o_part, lse_part, o=o, lse=lse)
        mark()

    # The library's own decode step (msa_decode_step, automatic mode): one
    # kernel for a short context and a small batch, else the three calls above.
    # This is the step that is timed and graphed for decode.
    sync = torch.zeros(msa.decode_step_sync_words(case.rows, case.G), dtype=torch.int32,
                       device=dev)

    def step_lib(ev=None):
        if ev is not None:
            ev[0].record()
        msa.msa_decode_step(d, case.q_idx, case.k_idx, case.block_table, case.row_pos, case.nb,
                            case.k, case.q, case.k_cache, case.v_cache, row_req=case.row_req,
                            blk_lo=case.blk_lo, num_reqs=case.num_reqs, sm_scale=scale,
                            sync=sync, scores=scores, sel=sel, page_table=pt, o_part=o_part,
                            lse_part=lse_part, o=o, lse=lse)
        if ev is not None:
            ev[1].record()

    # Every timed step starts from cold caches: an untimed read of 1 GiB (four
    # times the 256 MB MALL) runs before it, so a step never finds the previous
    # step's K/V blocks or partials in L2/MALL (consecutive steps of one layer
    # would not either: the other layers run in between).  A read leaves the
    # caches clean, so the step pays no write-back of the flush's own lines.
    flush_buf = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
    flush_out = torch.empty((), dtype=torch.float32, device=dev)

    def flush():
        torch.sum(flush_buf, dim=0, out=flush_out)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)]
           for _ in range(steps)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i in range(steps):
        flush()
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = {n: sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)) / steps
           for j, n in enumerate(names)}
    # the eager step, first call start to last call end, per step
    step_ms = sorted(evs[i][0].elapsed_time(evs[i][len(names)]) for i in range(steps))
    eager_ms = sum(step_ms)
    pct = {q: step_ms[min(steps - 1, int(round(q / 100 * (steps - 1))))] for q in (10, 50, 90)}
    o_ref, lse_ref = o.clone(), lse.clone()
    sel_ref = sel.clone()
    alg = algorithmic(case, sel)
    # The index-score kernel alone, launched back to back between one event
    # pair after a cache flush: each dispatch overlaps the previous launch, so
    # the average is the kernel's own duration (the per-launch event pairs above
    # also hold the dispatch latency in front of the kernel).
    score_btb_ms = None
    if not case.prefill:
        reps = 10
        flush()
        b0 = torch.cuda.Event(enable_timing=True)
        b1 = torch.cuda.Event(enable_timing=True)
        b0.record()
        for _ in range(reps):
            msa.msa_index_score(d, case.q_idx, case.k_idx, case.block_table, case.row_pos,
                                case.nb, row_req=case.row_req, blk_lo=case.blk_lo,
                                num_reqs=case.num_reqs, scores=scores)
        b1.record()
        torch.cuda.synchronize()
        score_btb_ms = b0.elapsed_time(b1) / reps
    # Prefill: attention and merge scheduled by query slabs
    # (msa_sparse_attn_prefill_merged), each slab's partials merged right after
    # its pass, against the whole batch as one slab.  Same output bit for bit.
    slab_us = None
    if case.prefill and slab_sweep:
        slab_us = {}
        for div in (1, 2, 4, 8, 16, 32):
            slab = max(1, case.rows // div)
            nws = msa.msa_prefill_merged_workspace_size(d, case.rows, case.nslot, case.num_pages,
                                                        slab)
            wsm = torch.empty(nws, dtype=torch.uint8, device=dev)
            om = torch.empty_like(o)
            lm = torch.empty_like(lse)

            def run_slabs():
                msa.msa_sparse_attn_prefill_merged(d, case.q, case.k_cache, case.v_cache, sel, pt,
                                                   case.row_pos, case.num_pages, scale,
                                                   slab_rows=slab, workspace=wsm, o=om, lse=lm)
            run_slabs()
            torch.cuda.synchronize()
            if not (torch.equal(om, o) and torch.equal(lm, lse)):
                raise RuntimeError(f"{case.name}: slab {slab} output differs from the step")
            ts = []
            for _ in range(3):
                flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                run_slabs()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            slab_us[str(slab)] = round(min(ts), 1)
            del wsm, om, lm
        torch.cuda.empty_cache()
    # Prefill: the block-major kernel's memory pattern without its arithmetic
    # (msa_peak_row_copy): every (row, group, slot) entry's Hg query rows loaded
    # and its Hg partial rows stored, in the order of the kernel's (group, page)
    # units, 32-row tiles, about one unit of tiles per workgroup; queries loaded
    # in the matrix-core operand layout as the kernel loads them, and as whole
    # rows.  Written into o_part, which the next step overwrites.
    pattern = None
    if case.prefill:
        r_i, g_i, s_i = (sel >= 0).nonzero(as_tuple=True)
        order = torch.argsort(pt[r_i, g_i, s_i].long() * case.G + g_i, stable=True)
        r_i, g_i, s_i = r_i[order], g_i[order], s_i[order]
        hh = torch.arange(case.Hg, device=dev)
        qrow = r_i[:, None] * case.H + g_i[:, None] * case.Hg + hh[None, :]
        prow = (qrow * case.nslot + s_i[:, None]).reshape(-1)
        qrow = qrow.reshape(-1)
        n = qrow.numel() // 32 * 32
        l_idx, s_idx = qrow[:n].to(torch.int32).contiguous(), prow[:n].to(torch.int32).contiguous()
        tiles = n // 32
        tpw = max(1, min(64, round(tiles / max(1, int(torch.unique(pt[r_i, g_i, s_i].long() * case.G
                                                                    + g_i).numel())))))
        pattern = dict(rows=n, bytes_each_way=n * 256, tiles_per_workgroup=tpw)
        for layout, key in ((1, "operand_layout_us"), (0, "whole_rows_us")):
            def run_pattern():
                msa.msa_peak_row_copy(case.q, o_part, l_idx, s_idx, tiles_per_wg=tpw,
                                      load_layout=layout)
            run_pattern()
            torch.cuda.synchronize()
            ts = []
            for _ in range(3):
                flush()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
                run_pattern()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e3)
            pattern[key] = round(min(ts), 1)
        del l_idx, s_idx, qrow, prow, r_i, g_i, s_i, order
    per_fused = None
    if fused:
        for _ in range(warmup):
            step_fused()
        torch.cuda.synchronize()
        if not (torch.equal(o, o_ref) and torch.equal(lse, lse_ref) and torch.equal(sel, sel_ref)):
            raise RuntimeError(f"{case.name}: the fused step differs from the four-call step")
        fev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fused_names) + 1)]
               for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            flush()
            step_fused(fev[i])
        torch.cuda.synchronize()
        per_fused = {n: sum(fev[i][j].elapsed_time(fev[i][j + 1]) for i in range(steps)) / steps
                     for j, n in enumerate(fused_names)}
        for _ in range(warmup):
            step_lib()
        torch.cuda.synchronize()
        if not (torch.equal(o, o_ref) and torch.equal(lse, lse_ref) and torch.equal(sel, sel_ref)):
            raise RuntimeError(f"{case.name}: msa_decode_step differs from the four-call step")
        lev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        torch.cuda.synchronize()
        for i in range(steps):
            flush()
            step_lib(lev[i])
        torch.cuda.synchronize()
        step_ms = sorted(lev[i][0].elapsed_time(lev[i][1]) for i in range(steps))
        eager_ms = sum(step_ms)
        pct = {q: step_ms[min(steps - 1, int(round(q / 100 * (steps - 1))))] for q in (10, 50, 90)}
        step = step_lib
    if not graph_replay:
        return case, dict(total_ms=eager_ms, ms_per_step=eager_ms / steps, eager_ms=eager_ms,
                          eager_ms_per_step=eager_ms / steps, wall_s=wall, per_call_ms=per,
                          per_call_fused_ms=per_fused, step_pct_ms=pct, alg=alg, sel=sel.cpu(),
                          score_btb_ms=score_btb_ms, slab_us=slab_us, pattern=pattern)

    # The same step captured once in a HIP graph and replayed: removes the
    # host launch gaps between the calls.  Every replay must reproduce the
    # eager result bit for bit.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(cap):
        step()  # warm the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=cap):
            step()
    torch.cuda.current_stream().wait_stream(cap)
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    if not (torch.equal(o, o_ref) and torch.equal(lse, lse_ref)):
        raise RuntimeError(f"{case.name}: graph replay differs from the eager step")
    ge = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        flush()
        ge[i][0].record()
        graph.replay()
        ge[i][1].record()
    torch.cuda.synchronize()
    graph_ms = sum(b.elapsed_time(e) for b, e in ge)
    if not (torch.equal(o, o_ref) and torch.equal(lse, lse_ref)):
        raise RuntimeError(f"{case.name}: graph replay differs from the eager step")
    # for reference only: the same replays back to back, caches left warm
    w0 = torch.cuda.Event(enable_timing=True)
    w1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0.record()
    for _ in range(steps):
        graph.replay()
    w1.record()
    torch.cuda.synchronize()
    warm_ms = w0.elapsed_time(w1)
    # The eager step is the one reported: on this HIP stack replaying the graph
    # costs more GPU time per step than the launches it holds (graph_ms_per_step)
    return case, dict(total_ms=eager_ms, ms_per_step=eager_ms / steps, eager_ms=eager_ms,
                      eager_ms_per_step=eager_ms / steps, graph_ms_per_step=graph_ms / steps,
                      wall_s=wall, per_call_ms=per, per_call_fused_ms=per_fused,
                      step_pct_ms=pct, alg=alg, sel=sel.cpu(), warm_ms_per_step=warm_ms / steps,
                      score_btb_ms=score_btb_ms, slab_us=slab_us, pattern=pattern)


def traffic_from_profile(workload, path=TRAFFIC_FILE, srcs=KERNEL_SRCS):
    """HBM bytes per launch of a kernel (by default the index-score kernel) from
    its committed counter summary, if that was taken on this workload and on the
    current kernel source."""
    try:
        info = json.load(open(path))
    except (OSError, ValueError):
        return None
    if info.get("workload") != workload:
        return None
    src_hash = hashlib.sha256(b"".join(open(f, "rb").read() for f in srcs)).hexdigest()[:16]
    if info.get("kernel_source_sha256_16") != src_hash:
        return None
    return info.get("hbm_bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_NATIVE_ORACLE = None


def _oracle_for_host():
    """The oracle as it stands, compiled for this host's CPU (-O3 -march=native,
    strict IEEE: the same results as the portable build the tests use)."""
    global _NATIVE_ORACLE
    import oracle
    if _NATIVE_ORACLE is None:
        _NATIVE_ORACLE = oracle.build_native(os.path.join(ROOT, "oracle", "_host"))
        oracle.use_library(_NATIVE_ORACLE)
    return oracle


# rows of each workload the oracle is timed on: every row of the decode batches,
# 256 evenly spaced rows of the 8,192-row prefill chunk (scaled to the chunk)
CPU_MIN_SECONDS = {1: 2.0, 2: 10.0}     # repeat whole passes for at least this long
PREFILL_CPU_ROWS = 256


def cpu_oracle(cfg, case, alg):
    """The oracle timed per stage on the host cores, on host copies of the same
    inputs: index score, top-k, page table, per-block attention partials and the
    LSE merge (the stages of the GPU path), each by perf_counter around its call.
    Copies to the host are not timed.  Stage times are scaled to the whole batch
    when only a sample of rows is timed."""
    import numpy as np
    from oracle import inputs
    orc = _oracle_for_host()
    if case.prefill:
        rows = list(range(0, case.rows, max(1, case.rows // PREFILL_CPU_ROWS)))
    else:
        rows = list(range(case.rows))
    scale_rows = case.rows / len(rows)
    h = inputs.host_rows(case, rows)
    bt_real = case.block_table.cpu().numpy()
    rr_real = case.row_req.cpu().numpy()[rows]
    sm = 1.0 / math.sqrt(case.D)
    kv = {}

    def one_pass():
        t = [time.perf_counter()]
        s = orc.index_score(h["q_idx"], h["k_idx"], h["bt"], h["row_pos"], case.nb,
                            row_req=h["row_req"], blk_lo=h["blk_lo"])
        t.append(time.perf_counter())
        sel = orc.topk(s.astype(np.float32), h["row_pos"], case.k)
        t.append(time.perf_counter())
        orc.page_table(sel, h["bt"], h["row_req"])
        t.append(time.perf_counter())
        if "pools" not in kv:     # the K/V pages this selection names, copied once (untimed)
            pt_real = orc.page_table(sel, bt_real, rr_real)
            kv["pools"] = inputs.host_kv_pages(case, pt_real)
        kp, vp, pt_c = kv["pools"]
        t.append(time.perf_counter())
        op, lp = orc.attn_partials(h["q"], kp, vp, sel, pt_c, h["row_pos"], sm)
        t.append(time.perf_counter())
        orc.lse_merge(op, lp)
        t.append(time.perf_counter())
        return [t[1] - t[0], t[2] - t[1], t[3] - t[2], t[5] - t[4], t[6] - t[5]]

    runs = []
    min_s = CPU_MIN_SECONDS.get(cfg, 0.0)
    if min_s:
        one_pass()                               # warm-up
    t0 = time.perf_counter()
    while True:
        runs.append(one_pass())
        if time.perf_counter() - t0 >= min_s or len(runs) >= 1000:
            break
    med = [sorted(r[i] for r in runs)[len(runs) // 2] for i in range(5)]
    names = ["index_score", "topk", "page_table", "attn_partials", "merge"]
    stage_ms = {n: round(v * scale_rows * 1e3, 3) for n, v in zip(names, med)}
    step_s = sum(med) * scale_rows
    out = dict(kind="oracle", cores=orc.num_threads(), cpu_model=cpu_model(),
               build="gcc -O3 -march=native -fopenmp, strict IEEE, fp64 accumulation",
               rows_timed=len(rows), runs=len(runs), stage_ms=stage_ms,
               step_ms=round(step_s * 1e3, 3),
               sample=(f"{len(rows)} of {case.rows} rows (every {case.rows // len(rows)}th), "
                       f"stage times scaled by {scale_rows:g}" if scale_rows > 1 else
                       f"all {case.rows} rows, median of {len(runs)} pass(es)"))
    scan_s = (med[0] + med[1]) * scale_rows
    out["index_scan_GBps"] = round((alg["kidx"] + alg["qidx"]) / scan_s / 1e9, 3)
    if case.prefill:
        out["attn_tflops_with_merge"] = round(
            alg["attn_flops"] / ((med[3] + med[4]) * scale_rows) / 1e12, 5)
    else:
        out["decode_tok_s"] = round(case.rows / step_s, 3)
    return out


def measured_peaks():
    """What this device sustains with nothing else in the way (include/msa_peaks.h):
    a non-temporal streaming read of 4 GiB and a register-resident bf16 MFMA loop.
    Best of several timed launches after a warm-up."""
    import torch
    import block_sparse_attention_09_amd as msa
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")

    def best(fn, reps):
        fn()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1))
        return min(out)

    t_read = best(lambda: msa.msa_peak_stream_read(buf, sink), 5)
    # write, then read the same bytes back right away (after a 1 GiB read that
    # leaves the caches cold): below the 256 MB last-level cache the read can
    # find them there
    flush = buf[: (1 << 30) // 4]
    wb = {}
    for label, n in (("144MiB", 144 << 20), ("2GiB", 2 << 30)):
        tgt = buf[(1 << 30) // 4:(1 << 30) // 4 + n // 4]
        tw, tr = [], []
        for rep in range(3):
            msa.msa_peak_stream_read(flush, sink)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            msa.msa_peak_stream_write(tgt, rep)
            e[1].record()
            msa.msa_peak_stream_read(tgt, sink)
            e[2].record()
            torch.cuda.synchronize()
            tw.append(e[0].elapsed_time(e[1]))
            tr.append(e[1].elapsed_time(e[2]))
        wb[label] = dict(write_GBps=round(n / (min(tw) * 1e-3) / 1e9, 1),
                         read_back_GBps=round(n / (min(tr) * 1e-3) / 1e9, 1))
    del buf, flush
    torch.cuda.empty_cache()
    iters = 16384
    flops = msa.msa_peak_mfma_bf16(iters, sink)
    t_mfma = best(lambda: msa.msa_peak_mfma_bf16(iters, sink), 3)
    iters_r = 4096
    flops_r = msa.msa_peak_mfma_bf16_random(iters_r, sink)
    t_mfma_r = best(lambda: msa.msa_peak_mfma_bf16_random(iters_r, sink), 3)
    return dict(stream_read_GBps=round(nbytes / (t_read * 1e-3) / 1e9, 1),
                mfma_bf16_TFLOPs=round(flops / (t_mfma * 1e-3) / 1e12, 1),
                mfma_bf16_random_TFLOPs=round(flops_r / (t_mfma_r * 1e-3) / 1e12, 1),
                write_then_read_back=wb,
                method=("msa_peak_stream_read over 4 GiB (a workgroup per 64 KB chunk, 8 "
                        "non-temporal 16-B loads in flight per thread); msa_peak_mfma_bf16: 4 "
                        "independent 32x32x16 bf16 MFMA chains per wave on fixed operands, 2 "
                        "waves per SIMD; msa_peak_mfma_bf16_random: the same on pseudo-random "
                        "unit-variance operands (the matrix cores' rate depends on the data); "
                        "best of 5, 3 and 3 launches; write_then_read_back: msa_peak_stream_write "
                        "of 144 MiB / 2 GiB after a 1 GiB cache-clearing read, then "
                        "msa_peak_stream_read of the same bytes, best of 3"))


def summarize(cfg, case, r, peaks=None):
    a = r["alg"]
    t = r["per_call_ms"]
    res = dict(workload=case.name, ms_per_step=round(r["ms_per_step"], 4),
               eager_ms_per_step=round(r["eager_ms_per_step"], 4),
               eager_step_ms_p10_p50_p90=[round(r["step_pct_ms"][q], 4) for q in (10, 50, 90)],
               per_call_us={k: round(v * 1e3, 2) for k, v in t.items()})
    if r.get("per_call_fused_ms"):
        res["step_calls"] = "msa_decode_step (automatic mode)"
        res["fused_step_per_call_us"] = {k: round(v * 1e3, 2)
                                         for k, v in r["per_call_fused_ms"].items()}
    if "warm_ms_per_step" in r:
        res["warm_cache_ms_per_step"] = round(r["warm_ms_per_step"], 4)
    if "graph_ms_per_step" in r:
        res["graph_ms_per_step"] = round(r["graph_ms_per_step"], 4)
    if not case.prefill:
        score_gbps = a["score_bytes"] / (t["index_score"] * 1e-3) / 1e9
        res["index_score_GBps"] = round(score_gbps, 1)
        res["index_score_hbm_frac"] = round(score_gbps / HBM_PEAK_GBPS, 4)
        if peaks:
            res["index_score_frac_of_measured_read"] = round(
                score_gbps / peaks["stream_read_GBps"], 4)
        if r.get("score_btb_ms"):
            res["index_score_back_to_back_us"] = round(r["score_btb_ms"] * 1e3, 2)
            res["index_score_back_to_back_GBps"] = round(
                a["score_bytes"] / (r["score_btb_ms"] * 1e-3) / 1e9, 1)
        res["index_scan_GBps"] = round((a["kidx"] + a["qidx"]) /
                                       ((t["index_score"] + t["topk_page_table"]) * 1e-3) / 1e9, 1)
    merge_bytes = a["part_bytes"] + a["qo_bytes"] // 2   # partials read, output written
    res["merge_GBps"] = round(merge_bytes / (t["merge"] * 1e-3) / 1e9, 1)
    if case.prefill:
        res["attn_tflops_kernel_call"] = round(a["attn_flops"] / (t["attn"] * 1e-3) / 1e12, 2)
        res["attn_tflops_with_merge"] = round(a["attn_flops"] /
                                              ((t["attn"] + t["merge"]) * 1e-3) / 1e12, 2)
        res["attn_mfma_frac_call"] = round(res["attn_tflops_kernel_call"] / BF16_PEAK_TFLOPS, 4)
        if peaks:
            res["attn_frac_of_measured_mfma"] = round(
                res["attn_tflops_kernel_call"] / peaks["mfma_bf16_TFLOPs"], 4)
            res["attn_frac_of_random_operand_mfma"] = round(
                res["attn_tflops_kernel_call"] / peaks["mfma_bf16_random_TFLOPs"], 4)
        res["attn_flops"] = a["attn_flops"]
        # the kernel's measured HBM traffic (counters of the committed summary:
        # K/V, the queries it fetches past L2 and the partials it writes) over
        # its call time: how close the call runs to the memory roofline
        traffic = traffic_from_profile(case.name, ATTN_TRAFFIC_FILE, ATTN_KERNEL_SRCS)
        if traffic:
            res["attn_traffic_bytes"] = traffic
            res["attn_traffic_GBps"] = round(traffic / (t["attn"] * 1e-3) / 1e9, 1)
            res["attn_traffic_hbm_frac"] = round(res["attn_traffic_GBps"] / HBM_PEAK_GBPS, 4)
        if r.get("pattern"):
            # the kernel's query loads and partial stores alone (msa_peak_row_copy)
            res["attn_memory_pattern"] = r["pattern"]
        if r.get("slab_us"):
            # msa_sparse_attn_prefill_merged by slab size (rows per slab): the
            # block-major attention and the merge, partials slab by slab
            res["attn_merge_by_slab_us"] = r["slab_us"]
        # index scoring contracts qbar = sum_j q_j (one vector per (row, group))
        # with the visible key-index tokens: 2 d_idx FLOP per token, reported as
        # index_qbar_tflops; the matrix cores take qbar as bf16 hi + lo, two
        # passes, so they issue twice that (index_mfma_tflops, against the peak)
        qbar_flops = a["index_flops"] / case.n_idx
        res["index_qbar_tflops"] = round(qbar_flops / (t["index_score"] * 1e-3) / 1e12, 2)
        res["index_mfma_tflops"] = round(2 * qbar_flops / (t["index_score"] * 1e-3) / 1e12, 2)
        res["index_mfma_frac"] = round(res["index_mfma_tflops"] / BF16_PEAK_TFLOPS, 4)
        if peaks:
            res["index_mfma_frac_of_random_operand_mfma"] = round(
                res["index_mfma_tflops"] / peaks["mfma_bf16_random_TFLOPs"], 4)
    else:
        res["decode_tok_s"] = round(case.rows / (r["ms_per_step"] * 1e-3), 1)
        step_bytes = a["kidx"] + a["qidx"] + a["kv_bytes"] + a["qo_bytes"]
        res["step_alg_GBps"] = round(step_bytes / (r["ms_per_step"] * 1e-3) / 1e9, 1)
        res["step_hbm_frac"] = round(res["step_alg_GBps"] / HBM_PEAK_GBPS, 4)
        res["step_alg_bytes"] = step_bytes
        attn_bytes = a["kv_bytes"] + a["qo_bytes"] // 2 + a["part_bytes"]
        res["decode_attn_GBps"] = round(attn_bytes / (t["attn"] * 1e-3) / 1e9, 1)
        res["decode_attn_hbm_frac"] = round(res["decode_attn_GBps"] / HBM_PEAK_GBPS, 4)
        if peaks:
            res["decode_attn_frac_of_measured_read"] = round(
                res["decode_attn_GBps"] / peaks["stream_read_GBps"], 4)
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: --gpus {args.gpus} is not supported (the MSA path "
              "here is a single-GPU build; see the sharding notes in the design document)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import block_sparse_attention_09_amd as msa
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    msa.load()
    print("[bench] measured peaks", file=sys.stderr, flush=True)
    peaks = measured_peaks()
    order = [int(x) for x in args.workloads.split(",") if x]
    main_cfg = order[0]
    results = {}
    main_case = main_run = None
    for cfg in order:
        steps = args.steps if cfg == main_cfg else max(5, min(args.steps, 20))
        print(f"[bench] workload {cfg}: {steps} steps", file=sys.stderr, flush=True)
        case, r = run_workload(cfg, steps, args.warmup, graph_replay=not args.eager_only,
                               slab_sweep=not args.no_slab_sweep)
        results[cfg] = summarize(cfg, case, r, peaks)
        if not args.no_cpu_baseline:
            # the oracle on the host cores, same inputs, after the GPU timing
            print(f"[bench] workload {cfg}: cpu oracle", file=sys.stderr, flush=True)
            cpu = cpu_oracle(cfg, case, r["alg"])
            res = results[cfg]
            if case.prefill:
                cpu["gpu_over_cpu"] = round(res["attn_tflops_with_merge"] /
                                            cpu["attn_tflops_with_merge"], 1)
            else:
                cpu["gpu_over_cpu"] = round(res["decode_tok_s"] / cpu["decode_tok_s"], 1)
            res["cpu_oracle"] = cpu
        if cfg == main_cfg:
            main_case, main_run = case, r
        else:
            del case
            torch.cuda.empty_cache()

    if not args.no_kv_on_host and not args.eager_only and not main_case.prefill:
        print(f"[bench] workload {main_cfg} with K/V in pinned host memory", file=sys.stderr,
              flush=True)
        case, r = run_workload(main_cfg, 20, args.warmup, kv_on_host=True)
        res = summarize(main_cfg, case, r, peaks)
        a, t = r["alg"], r["per_call_ms"]
        res["host_link_gather_GBps"] = round(a["kv_bytes"] / (t["gather"] * 1e-3) / 1e9, 1)
        results["kv-on-host"] = res
        del case
        torch.cuda.empty_cache()

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.zeros(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(f"[bench] calibration: 3 x neg over {n} B read + {n} B written", file=sys.stderr,
              flush=True)

    m = results[main_cfg]
    a = main_run["alg"]
    t_score = main_run["per_call_ms"]["index_score"]
    achieved = a["score_bytes"] / (t_score * 1e-3) / 1e9
    if main_case.prefill:
        # a prefill headline: the block-major attention kernel against the bf16
        # matrix-core peak (traffic: its HBM bytes from the committed counters)
        t_attn = main_run["per_call_ms"]["attn"]
        tf = a["attn_flops"] / (t_attn * 1e-3) / 1e12
        roofline = dict(kernel="attn_blockmajor_kernel", bound="mfma", achieved=round(tf, 2),
                        peak=BF16_PEAK_TFLOPS, unit="TFLOP/s", frac=round(tf / BF16_PEAK_TFLOPS, 4),
                        traffic=traffic_from_profile(main_case.name, ATTN_TRAFFIC_FILE,
                                                     ATTN_KERNEL_SRCS),
                        alg_flops_per_launch=a["attn_flops"], avg_launch_us=round(t_attn * 1e3, 2),
                        frac_of_random_operand_mfma=round(tf / peaks["mfma_bf16_random_TFLOPs"], 4))
    else:
        roofline = dict(kernel="index_score_stream_kernel", bound="hbm",
                        achieved=round(achieved, 1), peak=HBM_PEAK_GBPS, unit="GB/s",
                        frac=round(achieved / HBM_PEAK_GBPS, 4),
                        traffic=traffic_from_profile(main_case.name),
                        alg_bytes_per_launch=a["score_bytes"],
                        avg_launch_us=round(t_score * 1e3, 2),
                        frac_of_measured_read=round(achieved / peaks["stream_read_GBps"], 4))
    btb = main_run.get("score_btb_ms")
    if btb and not main_case.prefill:
        # the same kernel timed back to back (see run_workload): its own duration,
        # without the dispatch latency each per-launch event pair also holds
        roofline["back_to_back_us"] = round(btb * 1e3, 2)
        roofline["back_to_back_achieved"] = round(a["score_bytes"] / (btb * 1e-3) / 1e9, 1)
        roofline["back_to_back_frac"] = round(roofline["back_to_back_achieved"] / HBM_PEAK_GBPS, 4)
    cpu = None
    mc = m.get("cpu_oracle")
    if mc:
        cpu = dict(value=mc.get("decode_tok_s", mc.get("attn_tflops_with_merge")),
                   unit="tok/s" if "decode_tok_s" in mc else "TFLOP/s", cores=mc["cores"],
                   kind="oracle", cpu_model=mc["cpu_model"], sample=mc["sample"],
                   stage_ms=mc["stage_ms"], build=mc["build"])
    value = main_case.rows * args.steps / (main_run["total_ms"] * 1e-3)
    line = dict(
        metric=METRIC, value=round(value, 1), unit="tok/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=round(main_run["ms_per_step"], 4),
        launch=("eager step: its calls launched from the host, one HIP event pair around "
                "each step" + ("" if args.eager_only else
                               "; the same step captured in a HIP graph and replayed is "
                               "reported as graph_ms_per_step")),
        step=("decode: msa_decode_step in its automatic mode -- one kernel (scores, top-k, "
              "page table, attention and merge) for a short context and a small batch, "
              "otherwise msa_index_score, msa_sparse_attn_decode_select (top-k, page table "
              "and decode attention in one launch) and msa_lse_merge; per_call_us in the "
              "workload entry times the path as four calls, fused_step_per_call_us as those "
              "three; prefill: msa_index_score, msa_topk_blocks_paged, "
              "msa_sparse_attn_prefill, msa_lse_merge"),
        timing=("sum over the steps of one HIP event pair around each step; an untimed "
                "1 GiB read before every step leaves L2 and MALL cold"),
        graph_ms_per_step=m.get("graph_ms_per_step"),
        warm_cache_ms_per_step=m.get("warm_cache_ms_per_step"),
        eager_ms_per_step=round(main_run["eager_ms_per_step"], 4), higher_is_better=True,
        scaling="weak", vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=main_case.name, batch=main_case.rows,
                    context=int(main_case.ctx_len[0]), G=main_case.G, Hg=main_case.Hg,
                    head_dim=main_case.D, n_idx=main_case.n_idx, d_idx=main_case.d_idx,
                    top_k=main_case.k, paged=True, parallelism="none (1 GPU)"),
        index_scan_GBps=m.get("index_scan_GBps"), roofline=roofline, cpu_baseline=cpu,
        measured_peaks=peaks,
        device=torch.cuda.get_device_name(0),
        workloads={results[c]["workload"]: results[c] for c in results})
    print(json.dumps(line))


if __name__ == "__main__":
    main()
