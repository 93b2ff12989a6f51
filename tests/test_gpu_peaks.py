"""GPU checks of the measured-peak probes (include/msa_peaks.h): they run,
report the work they did, and land in a plausible range for one MI355X.  The
bounds are loose on purpose: they catch a probe that reads nothing or issues
no matrix work, not a slow machine."""
import pytest
import torch

import block_sparse_attention_09_amd as msa

pytestmark = pytest.mark.gpu


def _time(fn, reps=3):
    fn()
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    return best


def test_stream_read_probe():
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    # a size that is not a multiple of the 64 KB workgroup chunk: ragged last chunk
    buf = torch.ones((1 << 30) // 4 + 4 * 37, dtype=torch.float32, device="cuda")
    ms = _time(lambda: msa.msa_peak_stream_read(buf, sink))
    gbps = buf.numel() * 4 / (ms * 1e-3) / 1e9
    assert 1000.0 < gbps < 8200.0, gbps
    assert sink.item() == 0.0  # the fold never matches the guard value on this data


def test_mfma_probe():
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    iters = 2048
    flops = msa.msa_peak_mfma_bf16(iters, sink)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == 2 * cus * 4 * iters * 4 * (2 * 32 * 32 * 16)
    ms = _time(lambda: msa.msa_peak_mfma_bf16(iters, sink))
    tflops = flops / (ms * 1e-3) / 1e12
    assert 200.0 < tflops < 2600.0, tflops


def test_stream_write_probe():
    """Every 16-byte unit i holds (tag ^ i) + 0, 1, 2, 3, including a ragged last chunk."""
    n16 = (64 << 10) // 16 * 5 + 37
    buf = torch.zeros(n16 * 4, dtype=torch.int32, device="cuda")
    tag = 0x5A5A1234
    msa.msa_peak_stream_write(buf, tag)
    got = buf.view(n16, 4).cpu().to(torch.int64) & 0xFFFFFFFF
    i = torch.arange(n16, dtype=torch.int64)
    x = (i ^ tag) & 0xFFFFFFFF
    want = torch.stack([(x + j) & 0xFFFFFFFF for j in range(4)], dim=1)
    assert torch.equal(got, want)


def test_random_operand_mfma_probe():
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    iters = 512
    flops = msa.msa_peak_mfma_bf16_random(iters, sink)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert flops == 2 * cus * 4 * iters * 16 * (2 * 32 * 32 * 16)
    ms = _time(lambda: msa.msa_peak_mfma_bf16_random(iters, sink))
    tflops = flops / (ms * 1e-3) / 1e12
    assert 200.0 < tflops < 2600.0, tflops


@pytest.mark.parametrize("layout,tpw", [(0, 64), (1, 64), (1, 7), (0, 1)])
def test_row_copy_probe(layout, tpw):
    """Destination row store_idx[i] holds source row load_idx[i] exactly, every
    other destination row is untouched; tile counts that leave ragged
    workgroups (3,001 tiles over 64, 7 and 1 tiles per workgroup)."""
    g = torch.Generator(device="cpu").manual_seed(11 + layout + tpw)
    src_rows, dst_rows, n = 5000, 120_000, 32 * 3001
    src = torch.randint(-2**31, 2**31 - 1, (src_rows, 64), generator=g, dtype=torch.int32)
    load_idx = torch.randint(0, src_rows, (n,), generator=g, dtype=torch.int32)
    store_idx = torch.randperm(dst_rows, generator=g)[:n].to(torch.int32)
    dst = torch.full((dst_rows, 64), 7, dtype=torch.int32, device="cuda")
    msa.msa_peak_row_copy(src.cuda(), dst, load_idx.cuda(), store_idx.cuda(), tiles_per_wg=tpw,
                          load_layout=layout)
    got = dst.cpu()
    assert torch.equal(got[store_idx.long()], src[load_idx.long()])
    untouched = torch.ones(dst_rows, dtype=torch.bool)
    untouched[store_idx.long()] = False
    assert bool(torch.all(got[untouched] == 7))
