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


# d=64 heads take the matrix-core form from five tokens per call and the vector
# form below: (64, 8, (5, 7, 8)) and (64, 13, (6, 8)) run the former across
# folds inside calls, (64, 4, (4, 1, 2)) the latter.
CASES = [(op, dt, d, C, sizes) for op in ("gdn", "kda", "rwkv6") for dt in ("f32", "bf16")
         for d, C, sizes in ((32, 8, (3,)), (64, 4, (4, 1, 2)), (128, 8, (8,)), (128, 13, (5, 7, 1)),
                             (64, 1, (3,)), (128, 32, (8, 6)), (64, 8, (5, 7, 8)), (64, 13, (6, 8)))]


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
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, d), ref["out"])
    for m, b in enumerate(bounds):
        gs.assert_state(states[b].numpy(), ref["states"][m], b)
    assert st.log_length == T % C
    # and the single-token path agrees far inside the gates
    single, _, _ = gs.run_deltalog(dev, op, dtype, C)
    gs.assert_close_pair(outs, single, 1, 1e-5, "chunks vs single steps")


FULL_CASES = [("gdn_b128_h32_d128", "gdn", (4,)), ("gdn_b128_h32_d128", "gdn", (8,)),
              ("kda_b128_h32_d128", "kda", (8,)), ("rwkv6_b128_h32_d64", "rwkv6", (8,)),
              ("kda_b128_h32_d128", "kda", (5, 7)), ("rwkv6_b128_h32_d64", "rwkv6", (3, 6))]


@pytest.mark.parametrize("name,op,sizes", FULL_CASES)
def test_full_size_chunks(name, op, sizes):
    """Serving shape, C=8, in the launch configuration the multi-token bench times:
    every output of 64 sampled heads over 32 tokens, and their state at two
    chunk boundaries (one mid-cycle for the uneven schedules)."""
    w = workloads.WORKLOADS[name]
    T = 32
    x = workloads.generate_workload(w, T=T)
    dev = gs.to_device(x, DEV)
    bounds, t, i = [], 0, 0
    while t < T:
        t += min(sizes[i % len(sizes)], T - t)
        i += 1
        bounds.append(t)
    chk = sorted({bounds[len(bounds) // 2 - 1], T})
    heads = gs.head_sample(w.heads, 64, seed=3)
    ref = gs.oracle_run(x, op, heads=heads, chk_steps=chk, nthreads=16)
    outs, states, _ = run_chunks(dev, op, w.in_dtype, 8, sizes, state_steps=set(chk))
    hs = torch.as_tensor(heads, dtype=torch.long, device=outs.device)
    gs.assert_outputs(outs.view(T, w.heads, w.d)[:, hs].cpu().numpy(), ref["out"], sizes)
    for m, b in enumerate(chk):
        gs.assert_state(states[b].numpy()[heads], ref["states"][m], (sizes, b))


def test_token_axes_must_agree():
    """The torch front end rejects a chunk whose inputs carry different token counts
    before anything reaches the library."""
    x = workloads.generate("gdn", 1, 2, 32, 32, 4, "f32", seed=7)
    dev = gs.to_device(x, DEV)
    st = dl.DeltaLogState("gdn", "f32", dev["S0"].clone(), 4)
    c = _chunk(dev, 0, 3)
    c["v"] = dev["v"][0:2]
    with pytest.raises(ValueError, match="v carries 2 tokens"):
        st.step_tokens(**c)
    assert st.log_length == 0
    st.close()
