"""The streaming probes of include/lsq_probe.h move exactly the bytes they
claim (they set the bandwidth ceiling the decode step is reported against)."""
import pytest
import torch

import quantized_recurrent_state_amd as lsq

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda")


@pytest.mark.parametrize("u", [1, 2, 4, 8])
@pytest.mark.parametrize("nt", [0, 1])
@pytest.mark.parametrize("wg", [0, 3, 1000])
@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 1 << 22])
def test_copy_and_write_cover_exactly(u, nt, wg, nbytes):
    src = torch.randint(0, 256, (nbytes + 64,), dtype=torch.uint8, device=DEV)
    dst = torch.zeros_like(src)
    lsq.lsq_probe_stream(lsq.PROBE_COPY, src, dst, nbytes, u, nt, wg)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert not dst[nbytes:].any()                    # nothing past the end
    dst.zero_()
    lsq.lsq_probe_stream(lsq.PROBE_WRITE, None, dst, nbytes, u, nt, wg)
    torch.cuda.synchronize()
    w = dst[:nbytes].view(torch.int32).view(-1, 4)
    assert not dst[nbytes:].any()
    # every 16-byte vector was written: its first word is its index
    idx = torch.arange(w.shape[0], device=DEV, dtype=torch.int32)
    assert torch.equal(w[:, 0], idx)


def test_read_leaves_memory_unchanged():
    src = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, device=DEV)
    ref = src.clone()
    sink = torch.zeros(64, dtype=torch.uint8, device=DEV)
    lsq.lsq_probe_stream(lsq.PROBE_READ, src, sink, src.numel(), 4, 1, 0)
    torch.cuda.synchronize()
    assert torch.equal(src, ref)


@pytest.mark.parametrize("span", [1, 2, 4, 8, 10, 16])
@pytest.mark.parametrize("nt", [0, 1])
def test_span_walk_rewrites_every_vector(span, nt):
    nbytes = span * 1024 * 37
    src = torch.randint(0, 1 << 30, (nbytes // 4 + 16,), dtype=torch.int32, device=DEV)
    ref = src.clone()
    lsq.lsq_probe_span(src, src, nbytes, span, nt)          # in place
    torch.cuda.synchronize()
    got = src[: nbytes // 4].view(-1, 4)
    want = ref[: nbytes // 4].view(-1, 4).clone()
    want[:, 0] ^= 1
    assert torch.equal(got, want)
    assert torch.equal(src[nbytes // 4:], ref[nbytes // 4:])
    dst = torch.zeros_like(src)
    lsq.lsq_probe_span(ref, dst, nbytes, span, nt)
    torch.cuda.synchronize()
    assert torch.equal(dst[: nbytes // 4].view(-1, 4), want)
    assert not dst[nbytes // 4:].any()


@pytest.mark.parametrize("form", list(range(10)))
def test_valu_probe_runs_and_writes_nothing(form):
    """The chains stay finite and never hit the sentinel, so out is untouched;
    a longer run takes longer (the work is not optimised away)."""
    out = torch.full((4,), 7.0, device=DEV)
    lsq.lsq_probe_valu(form, 1024, 64, out)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.full((4,), 7.0, device=DEV))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    ev[0].record(); lsq.lsq_probe_valu(form, 1024, 256, out); ev[1].record()
    ev[2].record(); lsq.lsq_probe_valu(form, 1024, 4096, out); ev[3].record()
    torch.cuda.synchronize()
    assert ev[2].elapsed_time(ev[3]) > 4 * ev[0].elapsed_time(ev[1])
