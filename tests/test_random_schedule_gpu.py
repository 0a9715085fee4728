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
    eo = max(gs.rel(o[i], ref["out"][i]) for i in range(T))
    es = max(gs.rel(checks[s].numpy().reshape(Bsz * H, d, d), ref["states"][m]) for m, s in enumerate(steps))
    assert eo <= gs.OUT_GATE and es <= gs.STATE_GATE, (eo, es, Bsz, H, d, C, dtype, T, schedule)
