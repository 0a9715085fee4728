"""GPU parity of the DeltaLog decode path against the fp64 oracle (needs an MI355X).

Gates (normwise relative error per checked step, max over steps): outputs
<= 2e-3, materialised states <= 1e-4.  Both sides consume identical inputs
from ``workloads``; only fp32 vs fp64 accumulation separates them.
"""
import numpy as np
import pytest
import torch

import workloads
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _log(msg):
    print(msg, flush=True)


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    _need_gpu()
    import recurrent_state_updates_amd as dl
    dl.load_library()
    yield


# ---------------------------------------------------------------- small: every step

def test_small_gdn_workload_every_step():
    """The tiny fp32 GDN workload: outputs and states at every step, C=4, C=1 and eager."""
    w = workloads.WORKLOADS["gdn_b1_h2_d32"]
    x = workloads.generate_workload(w)
    dev = gs.to_device(x, DEV)
    T = w.T
    steps = list(range(T + 1))
    ref = gs.oracle_run(x, "gdn", chk_steps=steps)
    runs = {}
    for C in (4, 1):
        _log(f"small gdn C={C}")
        outs, states, _ = gs.run_deltalog(dev, "gdn", "f32", C, state_steps=steps)
        o = outs.cpu().numpy().reshape(T, 2, 32)
        eo = max(gs.rel(o[t], ref["out"][t]) for t in range(T))
        es = max(gs.rel(states[t].numpy(), ref["states"][t]) for t in steps)
        _log(f"  C={C}: max out rel {eo:.3e}, max state rel {es:.3e}")
        assert eo <= gs.OUT_GATE and es <= gs.STATE_GATE
        runs[C] = o
    eouts, estates = gs.run_eager(dev, "gdn", "f32", state_steps=steps[1:])
    eo = eouts.cpu().numpy().reshape(T, 2, 32)
    assert max(gs.rel(eo[t], ref["out"][t]) for t in range(T)) <= gs.OUT_GATE
    assert max(gs.rel(estates[t].numpy(), ref["states"][t]) for t in steps[1:]) <= gs.STATE_GATE
    # the three GPU paths agree with each other far inside the gates
    assert max(gs.rel(runs[4][t], runs[1][t]) for t in range(T)) <= 1e-5
    assert max(gs.rel(runs[1][t], eo[t]) for t in range(T)) <= 1e-5


SMALL = [(op, dt, d, C) for op in ("gdn", "kda", "rwkv6") for dt in ("f32", "bf16")
         for d in (32, 64, 128) for C in (1, 3, 8, 13, 32)]


@pytest.mark.parametrize("op,dtype,d,C", SMALL)
def test_small_every_step(op, dtype, d, C):
    """Every op x dtype x width x capacity on a ragged trajectory (T = 37)."""
    T, Bsz, H = 37, 2, 3
    x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=1000 + d + 7 * C)
    dev = gs.to_device(x, DEV)
    steps = list(range(T + 1))
    _log(f"small {op} {dtype} d={d} C={C}")
    ref = gs.oracle_run(x, op, chk_steps=steps, want_factors=True)
    outs, states, st = gs.run_deltalog(dev, op, dtype, C, state_steps=steps)
    o = outs.cpu().numpy().reshape(T, Bsz * H, d)
    eo = max(gs.rel(o[t], ref["out"][t]) for t in range(T))
    es = max(gs.rel(states[t].numpy(), ref["states"][t]) for t in steps)
    assert eo <= gs.OUT_GATE, eo
    assert es <= gs.STATE_GATE, es
    assert st.log_length == T % C


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_log_contents(op):
    """Log entries: value factors match the oracle's, keys are exact copies, log-decays cumulate."""
    T, Bsz, H, d, C = 7, 2, 2, 64, 8
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=77)
    dev = gs.to_device(x, DEV)
    ref = gs.oracle_run(x, op, want_factors=True)
    outs, _, st = gs.run_deltalog(dev, op, "bf16", C)
    X, K, G = (t.cpu() for t in st.workspace_views())
    N = Bsz * H
    for t in range(T):
        fac = X[:, :, t].float().reshape(N, d).numpy()
        assert gs.rel(fac, ref["factors"][t]) <= 1e-5
        assert torch.equal(K[:, :, t], x["k"][t])
    dec = x["decay"][:T].double().numpy()
    cum = np.cumsum(np.log2(dec), axis=0)  # cumulative base-2 log-decay since the (empty) start
    got = G[:, :, :T].double().numpy()
    if op == "gdn":
        want = np.moveaxis(cum, 0, -1)[..., None]
    else:
        want = np.moveaxis(cum, 0, 2)
    assert np.max(np.abs(got - want)) <= 2e-6 * max(1.0, np.max(np.abs(want)))


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_c1_is_eager(op):
    """C = 1 folds every token: the same state and outputs as the eager kernel."""
    T, Bsz, H, d = 20, 4, 4, 128
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=21)
    dev = gs.to_device(x, DEV)
    o1, s1, _ = gs.run_deltalog(dev, op, "bf16", 1, state_steps=[T])
    oe, se = gs.run_eager(dev, op, "bf16", state_steps=[T])
    assert max(gs.rel(o1[t].cpu(), oe[t].cpu()) for t in range(T)) <= 1e-6
    assert gs.rel(s1[T].numpy(), se[T].numpy()) <= 1e-6


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_base_after_fold_equals_oracle(op):
    """Right after each fold (L = 0) the base itself equals the eager state."""
    T, Bsz, H, d, C = 24, 2, 3, 64, 8
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=22)
    dev = gs.to_device(x, DEV)
    folds = [8, 16, 24]
    ref = gs.oracle_run(x, op, chk_steps=folds)
    seen = {}

    def on_step(t, st):
        if st.log_length == 0:
            seen[t] = st.base.view(Bsz * H, d, d).cpu().numpy()

    gs.run_deltalog(dev, op, "bf16", C, on_step=on_step)
    assert sorted(seen) == folds
    for m, t in enumerate(folds):
        assert gs.rel(seen[t], ref["states"][m]) <= gs.STATE_GATE


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_early_merge_is_output_neutral(op):
    T, Bsz, H, d, C = 30, 2, 2, 128, 8
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=23)
    dev = gs.to_device(x, DEV)
    o_ref, s_ref, _ = gs.run_deltalog(dev, op, "bf16", C, state_steps=[T])
    lengths = []
    o_m, s_m, st = gs.run_deltalog(dev, op, "bf16", C, state_steps=[T], merge_after={3, 5, 11, 12, 30},
                                   on_step=lambda t, s: lengths.append(s.log_length))
    assert max(gs.rel(o_m[t].cpu(), o_ref[t].cpu()) for t in range(T)) <= 1e-5
    assert gs.rel(s_m[T].numpy(), s_ref[T].numpy()) <= 1e-5
    assert st.log_length == 0  # merged after the last token


@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_materialize_is_non_destructive_and_deterministic(op):
    T, Bsz, H, d, C = 19, 2, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=24)
    dev = gs.to_device(x, DEV)
    a, _, _ = gs.run_deltalog(dev, op, "bf16", C)
    b, _, _ = gs.run_deltalog(dev, op, "bf16", C, materialize_every_step=True)
    c, _, _ = gs.run_deltalog(dev, op, "bf16", C)
    assert torch.equal(a, b)
    assert torch.equal(a, c)


def test_resume_from_saved_base():
    """A fold's base saved and reloaded into a fresh handle continues bit-identically."""
    import recurrent_state_updates_amd as dl
    T, Bsz, H, d, C = 20, 2, 2, 128, 4
    x = workloads.generate("kda", Bsz, H, d, d, T, "bf16", seed=25)
    dev = gs.to_device(x, DEV)
    full, _, _ = gs.run_deltalog(dev, "kda", "bf16", C)
    base = dev["S0"].clone()
    st = dl.DeltaLogState("kda", "bf16", base, C)
    for t in range(10):
        st.step(**gs._token(dev, t))
    st.merge()
    saved = base.clone()
    st2 = dl.DeltaLogState("kda", "bf16", saved, C)
    outs = [st2.step(**gs._token(dev, t)) for t in range(10, T)]
    torch.cuda.synchronize()
    st3 = dl.DeltaLogState("kda", "bf16", base, C)  # the merged base, also at L = 0
    outs3 = [st3.step(**gs._token(dev, t)) for t in range(10, T)]
    for i, t in enumerate(range(10, T)):
        assert torch.equal(outs[i], outs3[i])
        assert gs.rel(outs[i].cpu(), full[t].cpu()) <= 1e-5


def test_outputs_independent_of_capacity():
    T, Bsz, H, d = 33, 2, 4, 128
    x = workloads.generate("gdn", Bsz, H, d, d, T, "bf16", seed=26)
    dev = gs.to_device(x, DEV)
    runs = {C: gs.run_deltalog(dev, "gdn", "bf16", C)[0].cpu() for C in (1, 2, 4, 8, 16, 32)}
    for C, o in runs.items():
        assert max(gs.rel(o[t], runs[1][t]) for t in range(T)) <= 1e-5, C


# ---------------------------------------------------------------- full-size workloads

_CACHE = {}


def _workload_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        w = workloads.WORKLOADS[name]
        _log(f"generating {name}")
        x = workloads.generate_workload(w)
        _CACHE[name] = (w, x, gs.to_device(x, DEV))
    return _CACHE[name]


FULL = [(name, C) for name in ("gdn_b128_h32_d128", "kda_b128_h32_d128", "rwkv6_b128_h32_d64")
        for C in (4, 8)]


@pytest.mark.parametrize("name,C", FULL)
def test_full_size_against_oracle(name, C):
    """Serving-shape workloads, T = 256, every head against the oracle: the
    outputs at every step, and the whole state at step 1, mid-cycle and right
    after folds in the first and last cycles, and at the end; the whole batch
    also against the eager GPU kernel at every step."""
    w, x, dev = _workload_inputs(name)
    T, N = w.T, w.heads
    steps = sorted({1, C // 2, C, 2 * C, T - C - C // 2, T - C, T - 1, T})
    _log(f"full {name} C={C}: oracle on all {N} heads")
    ref = gs.oracle_run(x, w.op, chk_steps=steps, nthreads=16)
    _log(f"full {name} C={C}: deltalog")
    outs, states, st = gs.run_deltalog(dev, w.op, w.in_dtype, C, state_steps=steps)
    o = outs.view(T, N, w.d).cpu().numpy()
    eo = max(gs.rel(o[t], ref["out"][t]) for t in range(T))
    es = max(gs.rel(states[t].numpy(), ref["states"][m]) for m, t in enumerate(steps))
    worst_head = max(gs.rel(o[:, h], ref["out"][:, h]) for h in range(N))
    _log(f"  max out rel {eo:.3e}, max state rel {es:.3e}, worst single head (all steps) {worst_head:.3e}")
    assert eo <= gs.OUT_GATE and es <= gs.STATE_GATE
    assert worst_head <= gs.OUT_GATE
    assert st.log_length == 0
    del ref, states
    _log(f"full {name} C={C}: eager")
    eouts, _ = gs.run_eager(dev, w.op, w.in_dtype)
    ee = max(gs.rel(outs[t].cpu(), eouts[t].cpu()) for t in range(T))
    _log(f"  deltalog vs eager (all heads) max rel {ee:.3e}")
    assert ee <= 1e-4


SWEEP = [("C", C) for C in (1, 2, 4, 8, 16, 32)] + [("B", B) for B in workloads.SWEEP_B]


@pytest.mark.parametrize("axis,val", SWEEP)
def test_sweep_against_oracle(axis, val):
    w = workloads.WORKLOADS["gdn_sweep_c"]
    B = w.B if axis == "C" else val
    C = val if axis == "C" else 8
    key = f"sweep_B{B}"
    if key not in _CACHE:
        _CACHE.clear()
        _log(f"generating sweep B={B}")
        x = workloads.generate_workload(w, B=B)
        _CACHE[key] = (x, gs.to_device(x, DEV))
    x, dev = _CACHE[key]
    T, N = w.T, B * w.H
    heads = gs.head_sample(N, 48, seed=B + C)
    steps = [C, T - 1, T]
    ref = gs.oracle_run(x, "gdn", heads=heads, chk_steps=steps, nthreads=16)
    outs, states, _ = gs.run_deltalog(dev, "gdn", "bf16", C, state_steps=steps, heads=heads)
    hs = torch.as_tensor(heads, dtype=torch.long, device=outs.device)
    o = outs.view(T, N, w.d)[:, hs].cpu().numpy()
    eo = max(gs.rel(o[t], ref["out"][t]) for t in range(T))
    es = max(gs.rel(states[t].numpy(), ref["states"][m]) for m, t in enumerate(steps))
    _log(f"sweep B={B} C={C}: max out rel {eo:.3e}, max state rel {es:.3e}")
    assert eo <= gs.OUT_GATE and es <= gs.STATE_GATE
