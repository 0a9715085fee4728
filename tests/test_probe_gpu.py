"""The stream-ceiling probes do what the bench takes them to do.

bench.py times a read, an in-place copy and a write of every head at the
decode kernels' access pattern (include/deltalog_probe.h) as the ceilings
that bound the append and the decode-and-fold.  Here: the read and the copy
leave the state bit for bit unchanged, the write reaches every element of
every head and nothing outside the tensor, at every built head shape.
"""
import pytest
import torch

import recurrent_state_updates_amd as dl

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    dl.load_library()
    yield


@pytest.mark.parametrize("dk,dv,Bsz,H", [(a, b, 3, 5) for a in (32, 64, 128) for b in (32, 64, 128)]
                         + [(128, 128, 64, 32)])
def test_probes_touch_exactly_the_state(dk, dv, Bsz, H):
    """Small batches, and a batch of 2048 heads of 128 x 128, whose last 512
    the probes (like the decode kernels) read and write as half-width tiles."""
    n = Bsz * H * dk * dv
    g = torch.Generator(device="cpu").manual_seed(dk * 1000 + dv)
    guard = 4096  # floats before and after the tensor, which no probe may touch
    buf = torch.randn(n + 2 * guard, generator=g).to(DEV)
    ref = buf.clone()
    state = buf[guard:guard + n]
    sink = torch.zeros(4, device=DEV)
    s = torch.cuda.current_stream().cuda_stream
    for mode in (dl.DL_PROBE_READ, dl.DL_PROBE_COPY):
        dl.dl_probe_stream(mode, state.data_ptr(), Bsz, H, dk, dv, sink.data_ptr(), s)
        torch.cuda.synchronize()
        assert torch.equal(buf, ref), f"mode {mode} changed memory"
    assert torch.equal(sink, torch.zeros_like(sink)), "the read probe stores only for a NaN sum"
    dl.dl_probe_stream(dl.DL_PROBE_WRITE, state.data_ptr(), Bsz, H, dk, dv, sink.data_ptr(), s)
    torch.cuda.synchronize()
    assert torch.equal(state, torch.ones_like(state))
    assert torch.equal(buf[:guard], ref[:guard]) and torch.equal(buf[guard + n:], ref[guard + n:])
