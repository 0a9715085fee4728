"""Seeded random schedules of every lockstep call, on the GPU, against the oracle.

Each case draws a shape (B, H, head width, C, input dtype, T) and a schedule
that mixes single-token steps, multi-token chunks, early merges, switches
between the fused and the split replay preparation, and materialisations.
Whatever the order, every output must equal the oracle's eager recurrence of
the same tokens, and every materialised state the oracle's state at that
token (gist.science summary, "Meccanismo Core: Base + Log": the logical state
is the eager one).
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


def _chunk_tokens(dev, t0, t1):
    return dict(q=dev["q"][t0:t1], k=dev["k"][t0:t1], v=dev["v"][t0:t1],
                beta=None if dev["beta"] is None else dev["beta"][t0:t1],
                decay=dev["decay"][t0:t1], bonus=dev["bonus"])


@pytest.mark.parametrize("op,seed", [(op, s) for op in ("gdn", "kda", "rwkv6") for s in range(4)])
def test_random_schedule(op, seed):
    rng = np.random.default_rng(1000 * seed + {"gdn": 1, "kda": 2, "rwkv6": 3}[op])
    Bsz, H = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    d = int(rng.choice([32, 64, 128]))
    C = int(rng.choice([1, 2, 3, 5, 8, 11, 16, 23, 32]))
    dtype = str(rng.choice(["f32", "bf16"]))
    T = int(rng.integers(C, 3 * C + 6))
    x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=7000 + seed)
    dev = gs.to_device(x, DEV)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, dtype, base, C)
    outs = torch.full((T, Bsz, H, d), float("nan"), dtype=torch.float32, device=DEV)
    checks = {}  # token count -> materialised state on the CPU
    schedule = []
    t = 0
    while t < T:
        r = rng.random()
        if r < 0.15:
            st.set_split_replay(bool(rng.integers(0, 2)))
            schedule.append("split" if st.prep is not None else "fused")
        if r < 0.55:
            st.step(out=outs[t], **gs._token(dev, t))
            schedule.append("step")
            t += 1
        elif r < 0.85:
            K = int(rng.integers(1, min(dl.DL_MAX_TOKENS, T - t) + 1))
            st.step_tokens(out=outs[t:t + K], **_chunk_tokens(dev, t, t + K))
            schedule.append(f"chunk{K}")
            t += K
        elif r < 0.93:
            st.merge()
            schedule.append("merge")
        else:
            checks[t] = st.materialize().cpu()
            schedule.append("materialize")
    checks[T] = st.materialize().cpu()
    torch.cuda.synchronize()
    steps = sorted(checks)
    ref = gs.oracle_run(x, op, chk_steps=steps)
    o = outs.cpu().numpy().reshape(T, Bsz * H, d)
    assert not np.isnan(o).any(), schedule
    label = (Bsz, H, d, C, dtype, T, schedule)
    gs.assert_outputs(o, ref["out"], label)
    for m, s in enumerate(steps):
        gs.assert_state(checks[s].numpy().reshape(Bsz * H, d, d), ref["states"][m], (s, label))


def _slot_reference(x, op, slot, start, end, S0_seg):
    """Oracle of one slot's heads over tokens [start, end) from S0_seg [H, d, d]."""
    sl = {key: (None if x[key] is None else x[key][start:end, slot:slot + 1])
          for key in ("q", "k", "v", "beta", "decay")}
    sl["bonus"] = x["bonus"]
    sl["S0"] = S0_seg[None]
    return gs.oracle_run(sl, op, chk_steps=[end - start])


@pytest.mark.parametrize("op,seed", [(op, s) for op in ("gdn", "kda", "rwkv6") for s in range(3)])
def test_random_slot_schedule(op, seed):
    """Per-slot handles under a seeded random schedule: slots join and leave at
    random tokens with fresh states, calls of 1 to 8 tokens find every slot at
    its own log length (and fold some of them once or several times), and
    whole-handle and single-slot early merges come in between.  Every active
    slot's outputs and final state against the oracle of its own tokens."""
    rng = np.random.default_rng(5000 * seed + {"gdn": 11, "kda": 12, "rwkv6": 13}[op])
    Bsz, H = int(rng.integers(2, 6)), int(rng.integers(1, 3))
    d = int(rng.choice([32, 64, 128]))
    C = int(rng.choice([1, 2, 3, 5, 8, 11, 16]))
    dtype = str(rng.choice(["f32", "bf16"]))
    T = int(rng.integers(24, 40))
    x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=9000 + seed)
    dev = gs.to_device(x, DEV)
    g = torch.Generator().manual_seed(300 + seed)
    # each slot: one or two active segments [s, e)
    segments = {}
    for b in range(Bsz):
        s0 = int(rng.integers(0, T // 2))
        e0 = int(rng.integers(s0 + 1, T + 1))
        segs = [(s0, e0)]
        if e0 < T - 2 and rng.random() < 0.5:
            s1 = int(rng.integers(e0 + 1, T))
            segs.append((s1, T))
        segments[b] = segs
    seg_S0 = {(b, s): torch.randn((H, d, d), generator=g) * 0.02 for b, segs in segments.items()
              for s, _ in segs}
    events = sorted({t for segs in segments.values() for se in segs for t in se} | {T})
    base = torch.zeros((Bsz, H, d, d), dtype=torch.float32, device=DEV)
    st = dl.DeltaLogState(op, dtype, base, C, slots=True)
    outs = torch.full((T, Bsz, H, d), float("nan"), dtype=torch.float32, device=DEV)
    expect, t, schedule = {}, 0, []
    while t < T:
        for b, segs in segments.items():
            for s, e in segs:
                if e == t:
                    st.deactivate(b)
                    expect.pop(b, None)
                if s == t:
                    base[b].copy_(seg_S0[(b, s)].to(DEV))
                    st.activate(b)
                    expect[b] = 0
        r = rng.random()
        if r < 0.1 and expect:
            st.merge()
            expect = {b: 0 for b in expect}
            schedule.append("merge")
        elif r < 0.2 and expect:
            b = int(rng.choice(sorted(expect)))
            st.merge_slot(b)
            expect[b] = 0
            schedule.append(f"merge_slot{b}")
        nxt = next(e for e in events if e > t)
        t1 = min(t + int(rng.integers(1, dl.DL_MAX_TOKENS + 1)), nxt)
        st.step_tokens(out=outs[t:t1], **_chunk_tokens(dev, t, t1))
        schedule.append(f"call{t1 - t}")
        for b in expect:
            expect[b] = (expect[b] + t1 - t) % C
        for b in range(Bsz):
            assert st.slot_log_length(b) == expect.get(b, -1), (t1, b, schedule)
        t = t1
    final = st.materialize(torch.full_like(base, float("nan")))
    torch.cuda.synchronize()
    o = outs.cpu().numpy()
    fin = final.cpu().numpy()
    for b, segs in segments.items():
        active = np.zeros(T, dtype=bool)
        for s, e in segs:
            active[s:e] = True
            ref = _slot_reference(x, op, b, s, e, seg_S0[(b, s)])
            gs.assert_outputs(o[s:e, b], ref["out"], (b, s, e, d, C, dtype, schedule))
            if e == T:
                gs.assert_state(fin[b], ref["states"][0], (b, d, C, dtype, schedule))
        assert np.isnan(o[~active, b]).all()
        if not active[-1]:
            assert np.isnan(fin[b]).all()
