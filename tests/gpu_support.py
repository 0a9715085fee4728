"""Helpers shared by the GPU tests: trajectories through the C ABI and oracle runs.

The GPU side goes only through ``recurrent_state_updates_amd`` (the C ABI);
the reference side only through ``oracle``; both consume the same tensors
from ``workloads``.
"""
import numpy as np
import torch

import oracle
import recurrent_state_updates_amd as dl

OUT_GATE = 2e-3    # normwise output relative error, max over checked steps
STATE_GATE = 1e-4  # normwise materialised-state relative error, max over checked steps


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def to_device(inputs, device="cuda:0"):
    return {k: (None if v is None else v.to(device)) for k, v in inputs.items()}


def oracle_run(inputs, op, heads=None, chk_steps=(), want_factors=False, nthreads=8, T=None):
    """The oracle on the selected heads (indices into B*H), from the CPU inputs."""
    q = inputs["q"]
    Tfull, Bsz, H, dk = q.shape
    T = Tfull if T is None else T
    dv = inputs["v"].shape[-1]
    N = Bsz * H
    sel = np.arange(N) if heads is None else np.asarray(heads)
    idx = torch.as_tensor(sel, dtype=torch.long)

    def per_head(t, width):
        return t[:T].reshape(T, N, width)[:, idx].double().numpy()

    beta = None if op == "rwkv6" else inputs["beta"][:T].reshape(T, N)[:, idx].double().numpy()
    if op == "gdn":
        decay = inputs["decay"][:T].reshape(T, N)[:, idx].double().numpy()
    else:
        decay = per_head(inputs["decay"], dk)
    bonus = None
    if op == "rwkv6":
        bonus = inputs["bonus"][torch.as_tensor(sel % H)].double().numpy()
    S0 = inputs["S0"].reshape(N, dk, dv)[idx].double().numpy()
    return oracle.eager_run(op, per_head(q, dk), per_head(inputs["k"], dk), per_head(inputs["v"], dv),
                            beta, decay, bonus, S0, chk_steps=chk_steps,
                            want_factors=want_factors, nthreads=nthreads)


def _token(dev, t):
    return dict(q=dev["q"][t], k=dev["k"][t], v=dev["v"][t],
                beta=None if dev["beta"] is None else dev["beta"][t],
                decay=dev["decay"][t], bonus=dev["bonus"])


def run_deltalog(dev, op, in_dtype, C, T=None, state_steps=(), heads=None, merge_after=(),
                 materialize_every_step=False, on_step=None, split_replay=False):
    """Decode T tokens through dl_decode_step (appends in the split-replay
    form with ``split_replay``).

    Returns (outputs [T,B,H,dv] on the device, {t: materialised state of the
    selected heads after t tokens, on the CPU}, the DeltaLogState).
    """
    q = dev["q"]
    Tfull, Bsz, H, d = q.shape
    T = Tfull if T is None else T
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, in_dtype, base, C, split_replay=split_replay)
    outs = torch.empty((T, Bsz, H, d), dtype=torch.float32, device=q.device)
    hsel = None if heads is None else torch.as_tensor(np.asarray(heads), dtype=torch.long, device=q.device)
    want = set(state_steps)
    states = {}
    scratch = torch.empty_like(base)

    def grab(t):
        m = st.materialize(scratch)
        flat = m.view(Bsz * H, d, d)
        states[t] = (flat if hsel is None else flat[hsel]).cpu()

    if 0 in want:
        grab(0)
    for t in range(T):
        st.step(out=outs[t], **_token(dev, t))
        if on_step is not None:
            on_step(t + 1, st)
        if (t + 1) in merge_after:
            st.merge()
        if (t + 1) in want:
            grab(t + 1)
        elif materialize_every_step:
            st.materialize(scratch)
    torch.cuda.synchronize()
    return outs, states, st


def run_eager(dev, op, in_dtype, T=None, state_steps=(), heads=None):
    """Decode T tokens through dl_eager_step on a copy of S0."""
    q = dev["q"]
    Tfull, Bsz, H, d = q.shape
    T = Tfull if T is None else T
    state = dev["S0"].clone()
    outs = torch.empty((T, Bsz, H, d), dtype=torch.float32, device=q.device)
    hsel = None if heads is None else torch.as_tensor(np.asarray(heads), dtype=torch.long, device=q.device)
    want = set(state_steps)
    states = {}
    for t in range(T):
        dl.eager_step(op, in_dtype, state, out=outs[t], **_token(dev, t))
        if (t + 1) in want:
            flat = state.view(Bsz * H, d, d)
            states[t + 1] = (flat if hsel is None else flat[hsel]).cpu()
    torch.cuda.synchronize()
    return outs, states


def head_sample(N, k, seed):
    """k distinct heads including the first and the last."""
    g = np.random.default_rng(seed)
    if k >= N:
        return np.arange(N)
    mid = g.choice(np.arange(1, N - 1), size=k - 2, replace=False)
    return np.sort(np.concatenate([[0, N - 1], mid]))
