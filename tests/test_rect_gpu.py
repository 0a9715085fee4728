"""Heads whose key and value widths differ (dk != dv), on the GPU, against the oracle.

The state of a head is a dk x dv matrix (gist.science summary, "Problema"):
keys, queries (receptances), decays and the bonus have dk channels, values,
outputs and value factors dv.  Every path runs here at each of the six
rectangular pairs of {32, 64, 128}: single-token decode and its fold, the
eager kernel, calls of several tokens, the split replay, per-slot logs, and
two serving-shape workloads.
"""
import numpy as np
import pytest
import torch

import recurrent_state_updates_amd as dl
import workloads
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
RECT = [(32, 64), (32, 128), (64, 32), (64, 128), (128, 32), (128, 64)]
OPS = ("gdn", "kda", "rwkv6")


def _log(msg):
    print(msg, flush=True)


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


@pytest.mark.parametrize("op,dtype,dk,dv,C", [(op, dt, dk, dv, C) for op in OPS for dt in ("f32", "bf16")
                                              for dk, dv in RECT for C in (1, 3, 8, 13, 32)])
def test_rect_every_step(op, dtype, dk, dv, C):
    """Single-token decode on a ragged trajectory (T = 29): every output and
    the materialised state after every token."""
    T, Bsz, H = 29, 2, 3
    x = workloads.generate(op, Bsz, H, dk, dv, T, dtype, seed=2000 + dk + 3 * dv + 7 * C)
    dev = gs.to_device(x, DEV)
    steps = list(range(T + 1))
    ref = gs.oracle_run(x, op, chk_steps=steps)
    outs, states, st = gs.run_deltalog(dev, op, dtype, C, state_steps=steps)
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, dv), ref["out"])
    for t in steps:
        gs.assert_state(states[t].numpy(), ref["states"][t], t)
    assert st.log_length == T % C


@pytest.mark.parametrize("op", OPS)
def test_rect_eager_every_step(op):
    T, Bsz, H = 17, 2, 3
    for dtype in ("f32", "bf16"):
        for dk, dv in RECT:
            x = workloads.generate(op, Bsz, H, dk, dv, T, dtype, seed=2100 + dk + dv)
            dev = gs.to_device(x, DEV)
            steps = list(range(1, T + 1))
            ref = gs.oracle_run(x, op, chk_steps=steps)
            eouts, estates = gs.run_eager(dev, op, dtype, state_steps=steps)
            gs.assert_outputs(eouts.cpu().numpy().reshape(T, Bsz * H, dv), ref["out"], (dtype, dk, dv))
            for m, t in enumerate(steps):
                gs.assert_state(estates[t].numpy(), ref["states"][m], (dtype, dk, dv, t))


@pytest.mark.parametrize("op,dtype,dk,dv,C,sizes",
                         [(op, dt, dk, dv, C, sz) for op in OPS for dk, dv in RECT
                          for dt, C, sz in (("bf16", 8, (8,)), ("f32", 5, (3, 7, 1)), ("bf16", 13, (6, 8, 2)))])
def test_rect_chunks(op, dtype, dk, dv, C, sizes):
    """Calls of several tokens (some passing the log's end and folding inside
    the call): every output and the state at every call boundary, and the
    same outputs as single steps."""
    T, Bsz, H = 27, 2, 2
    x = workloads.generate(op, Bsz, H, dk, dv, T, dtype, seed=2200 + dk + dv + C)
    dev = gs.to_device(x, DEV)
    bounds, t, i = [], 0, 0
    while t < T:
        t += min(sizes[i % len(sizes)], T - t)
        i += 1
        bounds.append(t)
    ref = gs.oracle_run(x, op, chk_steps=bounds)
    st = dl.DeltaLogState(op, dtype, dev["S0"].clone(), C)
    outs = torch.empty((T, Bsz, H, dv), dtype=torch.float32, device=DEV)
    t0 = 0
    for m, t1 in enumerate(bounds):
        st.step_tokens(out=outs[t0:t1], **_chunk(dev, t0, t1))
        gs.assert_state(st.materialize().view(Bsz * H, dk, dv).cpu().numpy(), ref["states"][m], t1)
        t0 = t1
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, dv), ref["out"])
    single, _, _ = gs.run_deltalog(dev, op, dtype, C)
    gs.assert_close_pair(outs, single, 1, 1e-5, "chunks vs single steps")


@pytest.mark.parametrize("op,dk,dv", [(op, dk, dv) for op in OPS for dk, dv in RECT])
def test_rect_split_replay(op, dk, dv):
    """The split replay's key-side record has 2 dk floats, more than one per
    thread at 128 x 32 and 64 x 32: every step against the oracle and the
    fused form."""
    C, T, Bsz, H = 8, 19, 2, 3
    x = workloads.generate(op, Bsz, H, dk, dv, T, "bf16", seed=2300 + dk + dv)
    dev = gs.to_device(x, DEV)
    steps = list(range(1, T + 1))
    ref = gs.oracle_run(x, op, chk_steps=steps)
    outs, states, _ = gs.run_deltalog(dev, op, "bf16", C, state_steps=steps, split_replay=True)
    fused, _, _ = gs.run_deltalog(dev, op, "bf16", C)
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, dv), ref["out"])
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], t)
    gs.assert_close_pair(outs, fused, 1, 1e-6, "split vs fused")


def _slot_reference(x, op, slot, start, end, S0_seg):
    sl = {key: (None if x[key] is None else x[key][start:end, slot:slot + 1])
          for key in ("q", "k", "v", "beta", "decay")}
    sl["bonus"] = x["bonus"]
    sl["S0"] = S0_seg[None]
    return gs.oracle_run(sl, op, chk_steps=[end - start])


@pytest.mark.parametrize("op,dk,dv,C,chunked", [("gdn", 64, 128, 4, False), ("kda", 128, 32, 3, True),
                                                ("rwkv6", 32, 128, 5, True), ("gdn", 128, 64, 8, True),
                                                ("kda", 64, 32, 4, False), ("rwkv6", 128, 64, 8, False)])
def test_rect_per_slot_logs(op, dk, dv, C, chunked):
    """Slots join and leave at different tokens (single steps, or calls of up
    to eight tokens that fold each slot at its own token); each slot's
    outputs and final state against the oracle of its own tokens; one slot
    materialised alone equals its slice of the full state."""
    T, Bsz, H = 24, 4, 2
    x = workloads.generate(op, Bsz, H, dk, dv, T, "bf16", seed=2400 + dk + dv + C)
    dev = gs.to_device(x, DEV)
    segments = {0: [(0, 24)], 1: [(2, 11), (14, 24)], 2: [(3, 24)], 3: [(6, 19)]}
    events = sorted({t for segs in segments.values() for se in segs for t in se} | {T})
    g = torch.Generator().manual_seed(21 + C)
    seg_S0 = {(b, s): torch.randn((H, dk, dv), generator=g) * 0.02 for b, segs in segments.items()
              for s, _ in segs}
    base = torch.zeros((Bsz, H, dk, dv), dtype=torch.float32, device=DEV)
    st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
    outs = torch.full((T, Bsz, H, dv), float("nan"), dtype=torch.float32, device=DEV)
    sizes = [3, 8, 1, 5, 7, 2]
    t, i = 0, 0
    while t < T:
        for b, segs in segments.items():
            for s, e in segs:
                if e == t:
                    st.deactivate(b)
                if s == t:
                    base[b].copy_(seg_S0[(b, s)].to(DEV))
                    st.activate(b)
        nxt = next(e for e in events if e > t)
        t1 = min(t + (sizes[i % len(sizes)] if chunked else 1), nxt)
        i += 1
        st.step_tokens(out=outs[t:t1], **_chunk(dev, t, t1))
        t = t1
    final = st.materialize(torch.full_like(base, float("nan")))
    one = st.materialize_slot(2)
    torch.cuda.synchronize()
    assert torch.equal(one, final[2])
    o = outs.cpu().numpy()
    fin = final.cpu().numpy()
    for b, segs in segments.items():
        for s, e in segs:
            ref = _slot_reference(x, op, b, s, e, seg_S0[(b, s)])
            gs.assert_outputs(o[s:e, b], ref["out"], (b, s, e))
            if e == T:
                gs.assert_state(fin[b], ref["states"][0], b)
    assert np.isnan(fin[3]).all()


SERVING = [("gdn", 64, 128), ("kda", 128, 64)]


@pytest.mark.parametrize("op,dk,dv", SERVING)
def test_rect_serving_shape(op, dk, dv):
    """B = 128 slots of H = 32 heads, bf16 inputs, C = 8, 64 tokens, in the
    launch configuration of the decode step: every head's outputs at every
    step and its state right after folds and mid-cycle; then the same tokens
    in calls of eight on 64 sampled heads; and the eager kernel on all heads."""
    Bsz, H, T, C = 128, 32, 64, 8
    x = workloads.generate(op, Bsz, H, dk, dv, T, "bf16", seed=2500 + dk + dv)
    dev = gs.to_device(x, DEV)
    N = Bsz * H
    steps = [1, C // 2, C, T - C // 2, T]
    _log(f"rect serving {op} {dk}x{dv}: oracle on all {N} heads")
    ref = gs.oracle_run(x, op, chk_steps=steps, nthreads=16)
    outs, states, _ = gs.run_deltalog(dev, op, "bf16", C, state_steps=steps)
    eo, eo_el = gs.assert_outputs(outs.view(T, N, dv).cpu().numpy(), ref["out"], "deltalog")
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], t)
    _log(f"  out rel {eo:.3e} / per head {eo_el:.3e}")
    del states
    # calls of eight tokens
    heads = gs.head_sample(N, 64, seed=9)
    hs = torch.as_tensor(heads, dtype=torch.long, device=DEV)
    st = dl.DeltaLogState(op, "bf16", dev["S0"].clone(), C)
    couts = torch.empty((T, Bsz, H, dv), dtype=torch.float32, device=DEV)
    for t0 in range(0, T, 8):
        st.step_tokens(out=couts[t0:t0 + 8], **_chunk(dev, t0, t0 + 8))
    fin = st.materialize().view(N, dk, dv)[hs].cpu().numpy()
    gs.assert_outputs(couts.view(T, N, dv)[:, hs].cpu().numpy(), ref["out"][:, heads], "chunks")
    gs.assert_state(fin, ref["states"][-1][heads], "chunks")
    # the eager kernel
    eouts, est = gs.run_eager(dev, op, "bf16", state_steps=[T])
    gs.assert_outputs(eouts.view(T, N, dv).cpu().numpy(), ref["out"], "eager")
    gs.assert_state(est[T].numpy(), ref["states"][-1], "eager")
