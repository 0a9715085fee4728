"""Multi-token decode (dl_decode_tokens) on the GPU, against the fp64 oracle.

K tokens share one read of the base; the result must equal K single-token
steps: every token's output and the state after the chunk.
"""
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


def _chunk(dev, t0, t1):
    return dict(q=dev["q"][t0:t1], k=dev["k"][t0:t1], v=dev["v"][t0:t1],
                beta=None if dev["beta"] is None else dev["beta"][t0:t1],
                decay=dev["decay"][t0:t1], bonus=dev["bonus"])


def run_chunks(dev, op, dtype, C, sizes, state_steps=()):
    T, Bsz, H, d = dev["q"].shape
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, dtype, base, C)
    outs = torch.empty((T, Bsz, H, d), dtype=torch.float32, device=DEV)
    states = {}
    t = 0
    i = 0
    while t < T:
        K = min(sizes[i % len(sizes)], T - t)
        i += 1
        st.step_tokens(out=outs[t:t + K], **_chunk(dev, t, t + K))
        t += K
        if t in state_steps:
            states[t] = st.materialize().view(Bsz * H, d, d).cpu()
    torch.cuda.synchronize()
    return outs, states, st


CASES = [(op, dt, d, C, sizes) for op in ("gdn", "kda", "rwkv6") for dt in ("f32", "bf16")
         for d, C, sizes in ((32, 8, (3,)), (64, 4, (4, 1, 2)), (128, 8, (8,)), (128, 13, (5, 7, 1)),
                             (64, 1, (3,)), (128, 32, (8, 6)))]


@pytest.mark.parametrize("op,dtype,d,C,sizes", CASES)
def test_chunks_match_oracle(op, dtype, d, C, sizes):
    T, Bsz, H = 29, 2, 2
    x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=500 + d + C)
    dev = gs.to_device(x, DEV)
    # states at every chunk boundary the schedule produces
    bounds, t, i = [], 0, 0
    while t < T:
        t += min(sizes[i % len(sizes)], T - t)
        i += 1
        bounds.append(t)
    ref = gs.oracle_run(x, op, chk_steps=bounds)
    outs, states, st = run_chunks(dev, op, dtype, C, sizes, state_steps=set(bounds))
    o = outs.cpu().numpy().reshape(T, Bsz * H, d)
    eo = max(gs.rel(o[t], ref["out"][t]) for t in range(T))
    es = max(gs.rel(states[b].numpy(), ref["states"][m]) for m, b in enumerate(bounds))
    assert eo <= gs.OUT_GATE, eo
    assert es <= gs.STATE_GATE, es
    assert st.log_length == T % C
    # and the single-token path agrees far inside the gates
    single, _, _ = gs.run_deltalog(dev, op, dtype, C)
    assert max(gs.rel(outs[t].cpu(), single[t].cpu()) for t in range(T)) <= 1e-5


def test_full_size_chunk_of_four():
    w = workloads.WORKLOADS["gdn_b128_h32_d128"]
    x = workloads.generate_workload(w, T=32)
    dev = gs.to_device(x, DEV)
    heads = gs.head_sample(w.heads, 64, seed=3)
    ref = gs.oracle_run(x, "gdn", heads=heads, chk_steps=[32], nthreads=16)
    outs, states, _ = run_chunks(dev, "gdn", "bf16", 8, (4,), state_steps={32})
    hs = torch.as_tensor(heads, dtype=torch.long, device=outs.device)
    o = outs.view(32, w.heads, w.d)[:, hs].cpu().numpy()
    assert max(gs.rel(o[t], ref["out"][t]) for t in range(32)) <= gs.OUT_GATE
    assert gs.rel(states[32].numpy()[heads], ref["states"][0]) <= gs.STATE_GATE
