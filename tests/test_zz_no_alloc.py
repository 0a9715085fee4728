"""The allocation-free decode step (dl_decode_step_noalloc) on the GPU.

It runs the split-replay form of dl_decode_step with the per-head prep
records in the library's static device scratch instead of a caller buffer.
Checked through the C ABI against the existing entry point (dl_decode_step
with a prep buffer set) and against the oracle, on two trajectories in a
row, the second smaller than the first: every output and the materialised
state after every cycle.
"""
import numpy as np
import pytest
import torch

import recurrent_state_updates_amd as dl
import workloads
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    dl.load_library()
    yield


def _run(dev, op, dtype, C, T, noalloc):
    Tf, Bsz, H, dk, dv = gs.dims(dev)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, dtype, base, C, split_replay=not noalloc)
    outs = torch.empty((T, Bsz, H, dv), dtype=torch.float32, device=DEV)
    states = {}
    for t in range(T):
        tok = gs._token(dev, t)
        if noalloc:
            st.step_noalloc(out=outs[t], **tok)
        else:
            st.step(out=outs[t], **tok)
        if (t + 1) % C == 0 or t + 1 == T:
            states[t + 1] = st.materialize().view(Bsz * H, dk, dv).cpu()
    torch.cuda.synchronize()
    assert st.log_length == T % C
    st.close()
    return outs, states


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_noalloc_equals_the_split_replay_and_the_oracle(op):
    # first a serving-shape batch (4096 heads: 4.5 MB of records at d = 128),
    # then a smaller one with other widths, on the same static scratch
    cases = [(128, 32, 128, 128, 8, 24, "bf16"), (3, 2, 64, 32, 5, 17, "f32")]
    for i, (Bsz, H, dk, dv, C, T, dtype) in enumerate(cases):
        x = workloads.generate(op, Bsz, H, dk, dv, T, dtype, seed=3000 + 10 * i + len(op))
        dev = gs.to_device(x, DEV)
        a, sa = _run(dev, op, dtype, C, T, noalloc=True)
        b, sb = _run(dev, op, dtype, C, T, noalloc=False)
        # the same kernels on the same inputs: the same bits
        assert torch.equal(a, b), (op, i)
        for t in sa:
            assert torch.equal(sa[t], sb[t]), (op, i, t)
        N = Bsz * H
        heads = gs.head_sample(N, 64, seed=i)
        steps = sorted(sa)
        ref = gs.oracle_run(x, op, heads=heads, chk_steps=steps, nthreads=16)
        hs = torch.as_tensor(heads, dtype=torch.long, device=DEV)
        gs.assert_outputs(a.view(T, N, dv)[:, hs].cpu().numpy(), ref["out"], (op, i))
        for m, t in enumerate(steps):
            gs.assert_state(sa[t].numpy()[heads], ref["states"][m], (op, i, t))


def test_noalloc_refuses_a_per_slot_handle():
    x = workloads.generate("gdn", 2, 2, 64, 64, 1, "bf16", seed=3100)
    dev = gs.to_device(x, DEV)
    st = dl.DeltaLogState("gdn", "bf16", dev["S0"].clone(), 4, slots=True)
    st.activate(0)
    with pytest.raises(dl.DeltaLogError) as e:
        st.step_noalloc(**gs._token(dev, 0))
    assert e.value.status == dl._binding.DL_ERR_UNSUPPORTED
    st.close()
