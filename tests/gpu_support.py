"""Helpers shared by the GPU tests: trajectories through the C ABI, oracle runs
and the error measures.

The GPU side goes only through ``recurrent_state_updates_amd`` (the C ABI);
the reference side only through ``oracle``; both consume the same tensors
from ``workloads``.

Two error measures gate every comparison with the oracle (the pages report
an output relative error and a materialised-state relative error: the
signal-papers summary, Fig. 12 (a) and (b)):

* normwise: ||x - ref||_F / ||ref||_F over one step's whole tensor, the max
  over checked steps, gated at OUT_GATE (outputs) and STATE_GATE (states);
* element-wise per head: for each head (one step's output row [dv], or one
  state [dk, dv]) the largest |x - ref| over its elements divided by that
  head's largest |ref|, the max over heads and steps, gated at
  ELEM_OUT_GATE (outputs) and ELEM_STATE_GATE (states).
  A single wrong element of a large tensor barely moves the normwise
  figure; it moves this one by its whole size.
"""
import numpy as np
import torch

import oracle
import recurrent_state_updates_amd as dl

OUT_GATE = 2e-3    # normwise output relative error, max over checked steps
STATE_GATE = 1e-4  # normwise materialised-state relative error, max over checked steps
# Per-head element-wise bounds, max |x - ref| / max |ref| within a head.
# An fp32 sum of n terms is off by at most gamma_n = n * 2^-24 times the sum of
# its terms' magnitudes (about sqrt(n) * 2^-24 times it in practice).  The
# longest sums on the path have n = dk + C + 2 <= 162 terms.
#  - A state element is a decayed base value plus at most C logged rank-one
#    terms, without cancellation to speak of: a head's error stays near
#    2^-24 of its largest element (at most 3e-7 measured at serving shape),
#    and the gate leaves a factor of thirty over that.
#  - An output element is a dot product of a state column with the query
#    (receptance), which cancels: the sum of the terms' magnitudes over the
#    head's largest output, kappa, has a median of 4-5 and reaches 17-27 at the
#    99.9th percentile and 29-82 at the largest of 16384 sampled head-steps of
#    the serving-shape workloads.  sqrt(n) * 2^-24 * kappa is then up to
#    about 6e-5, which the output gate covers.
# A single corrupted element moves a head by about its own size (1e-1 or
# more), a thousand times either gate.
ELEM_OUT_GATE = 1e-4
ELEM_STATE_GATE = 1e-5


def elem_gate(tail):
    """The per-head gate of outputs and value factors (tail 1) or states (tail 2)."""
    return ELEM_OUT_GATE if tail == 1 else ELEM_STATE_GATE


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / den) if den > 0 else float(np.linalg.norm(a - b))


def head_err(a, b, tail):
    """Worst head of ``a`` against ``b``: max |a - b| over the head's elements
    divided by the head's max |b| (the absolute error where that is 0).
    ``tail`` is the number of trailing axes that make one head: 1 for outputs
    [..., dv], 2 for states [..., dk, dv].  Every leading axis (steps, slots,
    heads) is a separate head.  NaN anywhere gives NaN, which fails any gate."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError(f"shapes differ: {a.shape} vs {b.shape}")
    if a.size == 0:
        return 0.0
    n = int(np.prod(a.shape[len(a.shape) - tail:]))
    a2, b2 = a.reshape(-1, n), b.reshape(-1, n)
    err = np.abs(a2 - b2).max(axis=1)
    scale = np.abs(b2).max(axis=1)
    r = np.where(scale > 0, err / np.where(scale > 0, scale, 1.0), err)
    return float(r.max())


def out_errors(o, ref):
    """(normwise max over steps, worst per-head element error) of outputs
    [T, ..., dv] against the oracle's."""
    o = np.asarray(o, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if o.shape != ref.shape:
        o = o.reshape(ref.shape)
    norm = max((rel(o[t], ref[t]) for t in range(len(o))), default=0.0)
    return norm, head_err(o, ref, 1)


def assert_outputs(o, ref, label=""):
    """Outputs [T, ..., dv] within the normwise and the element-wise gates."""
    norm, elem = out_errors(o, ref)
    assert norm <= OUT_GATE and elem <= ELEM_OUT_GATE, (label, "outputs", norm, elem)
    return norm, elem


def state_errors(s, ref):
    """(normwise, worst per-head element error) of one state [..., dk, dv]."""
    s = np.asarray(s, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if s.shape != ref.shape:
        s = s.reshape(ref.shape)
    return rel(s, ref), head_err(s, ref, 2)


def assert_state(s, ref, label=""):
    """One materialised state [..., dk, dv] within the normwise and the element-wise gates."""
    norm, elem = state_errors(s, ref)
    assert norm <= STATE_GATE and elem <= ELEM_STATE_GATE, (label, "state", norm, elem)
    return norm, elem


def assert_close_pair(a, b, tail, norm_gate, label=""):
    """Two GPU results (outputs with tail=1, states with tail=2) that must agree:
    normwise per leading index within norm_gate, per head within twice the
    element-wise gate of the kind (each side is within one gate of the oracle)."""
    a = np.asarray(a.cpu() if torch.is_tensor(a) else a, dtype=np.float64)
    b = np.asarray(b.cpu() if torch.is_tensor(b) else b, dtype=np.float64)
    if tail == 1 and a.ndim > 2:
        norm = max(rel(a[t], b[t]) for t in range(len(a)))
    else:
        norm = rel(a, b)
    elem = head_err(a, b, tail)
    assert norm <= norm_gate and elem <= 2 * elem_gate(tail), (label, norm, elem)
    return norm, elem


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


def dims(dev):
    """(T, B, H, dk, dv) of a generated workload."""
    T, Bsz, H, dk = dev["q"].shape
    return T, Bsz, H, dk, dev["v"].shape[-1]


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
    Tfull, Bsz, H, dk, dv = dims(dev)
    T = Tfull if T is None else T
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, in_dtype, base, C, split_replay=split_replay)
    outs = torch.empty((T, Bsz, H, dv), dtype=torch.float32, device=dev["q"].device)
    hsel = None if heads is None else torch.as_tensor(np.asarray(heads), dtype=torch.long, device=dev["q"].device)
    want = set(state_steps)
    states = {}
    scratch = torch.empty_like(base)

    def grab(t):
        m = st.materialize(scratch)
        flat = m.view(Bsz * H, dk, dv)
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
    Tfull, Bsz, H, dk, dv = dims(dev)
    T = Tfull if T is None else T
    state = dev["S0"].clone()
    outs = torch.empty((T, Bsz, H, dv), dtype=torch.float32, device=dev["q"].device)
    hsel = None if heads is None else torch.as_tensor(np.asarray(heads), dtype=torch.long, device=dev["q"].device)
    want = set(state_steps)
    states = {}
    for t in range(T):
        dl.eager_step(op, in_dtype, state, out=outs[t], **_token(dev, t))
        if (t + 1) in want:
            flat = state.view(Bsz * H, dk, dv)
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
