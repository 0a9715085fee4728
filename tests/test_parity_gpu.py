"""GPU parity of the DeltaLog decode path against the fp64 oracle (needs an MI355X).

Gates, on every comparison with the oracle: normwise relative error per
checked step (max over steps) <= 2e-3 for outputs and <= 1e-4 for
materialised states, and per head max |x - ref| / max |ref| <= 1e-4 for
outputs and <= 1e-5 for states (see ``gpu_support``).  Both sides consume identical inputs from ``workloads``;
only fp32 vs fp64 accumulation separates them.
"""
import numpy as np
import pytest
import torch

import recurrent_state_updates_amd as dl
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
        eo, eo_el = gs.assert_outputs(o, ref["out"], f"C={C}")
        es = [gs.assert_state(states[t].numpy(), ref["states"][t], f"C={C} t={t}") for t in steps]
        _log(f"  C={C}: out rel {eo:.3e} / per head {eo_el:.3e}; state rel {max(e[0] for e in es):.3e}"
             f" / per head {max(e[1] for e in es):.3e}")
        runs[C] = o
    eouts, estates = gs.run_eager(dev, "gdn", "f32", state_steps=steps[1:])
    eo = eouts.cpu().numpy().reshape(T, 2, 32)
    gs.assert_outputs(eo, ref["out"], "eager")
    for t in steps[1:]:
        gs.assert_state(estates[t].numpy(), ref["states"][t], f"eager t={t}")
    # the three GPU paths agree with each other far inside the gates
    gs.assert_close_pair(runs[4], runs[1], 1, 1e-5, "C=4 vs C=1")
    gs.assert_close_pair(runs[1], eo, 1, 1e-5, "C=1 vs eager")


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
    ref = gs.oracle_run(x, op, chk_steps=steps)
    outs, states, st = gs.run_deltalog(dev, op, dtype, C, state_steps=steps)
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, d), ref["out"])
    for t in steps:
        gs.assert_state(states[t].numpy(), ref["states"][t], t)
    assert st.log_length == T % C


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_small_eager_every_step(op):
    """The eager comparison kernel alone against the oracle at every width and
    both input dtypes: every output and the state after every step."""
    T, Bsz, H = 23, 2, 3
    for dtype in ("f32", "bf16"):
        for d in (32, 64, 128):
            x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=1100 + d)
            dev = gs.to_device(x, DEV)
            steps = list(range(1, T + 1))
            ref = gs.oracle_run(x, op, chk_steps=steps)
            eouts, estates = gs.run_eager(dev, op, dtype, state_steps=steps)
            gs.assert_outputs(eouts.cpu().numpy().reshape(T, Bsz * H, d), ref["out"], (dtype, d))
            for m, t in enumerate(steps):
                gs.assert_state(estates[t].numpy(), ref["states"][m], (dtype, d, t))


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
        assert gs.head_err(fac, ref["factors"][t], 1) <= gs.ELEM_OUT_GATE
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
    gs.assert_close_pair(o1, oe, 1, 1e-6, "outputs")
    gs.assert_close_pair(s1[T], se[T], 2, 1e-6, "state")


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
        gs.assert_state(seen[t], ref["states"][m], t)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_early_merge_is_output_neutral(op):
    T, Bsz, H, d, C = 30, 2, 2, 128, 8
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=23)
    dev = gs.to_device(x, DEV)
    o_ref, s_ref, _ = gs.run_deltalog(dev, op, "bf16", C, state_steps=[T])
    lengths = []
    o_m, s_m, st = gs.run_deltalog(dev, op, "bf16", C, state_steps=[T], merge_after={3, 5, 11, 12, 30},
                                   on_step=lambda t, s: lengths.append(s.log_length))
    gs.assert_close_pair(o_m, o_ref, 1, 1e-5, "outputs")
    gs.assert_close_pair(s_m[T], s_ref[T], 2, 1e-5, "state")
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
    gs.assert_close_pair(torch.stack(outs), full[10:T], 1, 1e-5, "resumed vs uninterrupted")


def test_outputs_independent_of_capacity():
    T, Bsz, H, d = 33, 2, 4, 128
    x = workloads.generate("gdn", Bsz, H, d, d, T, "bf16", seed=26)
    dev = gs.to_device(x, DEV)
    runs = {C: gs.run_deltalog(dev, "gdn", "bf16", C)[0].cpu() for C in (1, 2, 4, 8, 16, 32)}
    for C, o in runs.items():
        gs.assert_close_pair(o, runs[1], 1, 1e-5, C)


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
    after folds in the first and last cycles, and at the end, each head within
    the element-wise gate.  The eager GPU kernel on the same inputs is checked
    directly against the oracle too: every output, and the state at two of
    the same steps."""
    w, x, dev = _workload_inputs(name)
    T, N, d = w.T, w.heads, w.d
    steps = sorted({1, C // 2, C, 2 * C, T - C - C // 2, T - C, T - 1, T})
    _log(f"full {name} C={C}: oracle on all {N} heads")
    ref = gs.oracle_run(x, w.op, chk_steps=steps, nthreads=16)
    _log(f"full {name} C={C}: deltalog")
    outs, states, st = gs.run_deltalog(dev, w.op, w.in_dtype, C, state_steps=steps)
    eo, eo_el = gs.assert_outputs(outs.view(T, N, d).cpu().numpy(), ref["out"], "deltalog")
    es = [gs.assert_state(states[t].numpy(), ref["states"][m], ("deltalog", t)) for m, t in enumerate(steps)]
    _log(f"  out rel {eo:.3e} / per head {eo_el:.3e}; state rel {max(e[0] for e in es):.3e}"
         f" / per head {max(e[1] for e in es):.3e}")
    assert st.log_length == 0
    del states
    _log(f"full {name} C={C}: eager")
    esteps = (C, T)
    eouts, estates = gs.run_eager(dev, w.op, w.in_dtype, state_steps=esteps)
    eeo, eeo_el = gs.assert_outputs(eouts.view(T, N, d).cpu().numpy(), ref["out"], "eager")
    ees = [gs.assert_state(estates[t].numpy(), ref["states"][steps.index(t)], ("eager", t)) for t in esteps]
    _log(f"  eager: out rel {eeo:.3e} / per head {eeo_el:.3e}; state rel {max(e[0] for e in ees):.3e}"
         f" / per head {max(e[1] for e in ees):.3e}")
    gs.assert_close_pair(outs.cpu(), eouts.cpu(), 1, 1e-4, "deltalog vs eager")


@pytest.mark.parametrize("name,C", FULL)
def test_full_size_states_every_step_sampled_heads(name, C):
    """The materialised state of 256 seeded-random heads after every one of
    the 256 tokens, each head within the element-wise gate.  Heads are
    independent, so the oracle of the sampled heads is exact; it runs in
    segments of 32 tokens, each continuing from the previous segment's fp64
    state, so that no more than 32 states of each side are held at once."""
    w, x, dev = _workload_inputs(name)
    T, N, d, Bsz, H = w.T, w.heads, w.d, w.B, w.H
    heads = gs.head_sample(N, 256, seed=17 + C)
    hs = torch.as_tensor(heads, dtype=torch.long, device=DEV)
    idx = torch.as_tensor(heads, dtype=torch.long)
    import oracle

    def sel(t, t0, t1, width):
        return t[t0:t1].reshape(t1 - t0, N, width)[:, idx].double().numpy()

    S = x["S0"].reshape(N, d, d)[idx].double().numpy()
    bonus = x["bonus"][torch.as_tensor(heads % H)].double().numpy() if w.op == "rwkv6" else None
    base = dev["S0"].clone()
    st = dl.DeltaLogState(w.op, w.in_dtype, base, C)
    scratch = torch.empty_like(base)
    worst = (0.0, 0.0)
    seg = 32
    for t0 in range(0, T, seg):
        t1 = min(T, t0 + seg)
        got = []
        for t in range(t0, t1):
            st.step(**gs._token(dev, t))
            got.append(st.materialize(scratch).view(N, d, d)[hs].cpu())
        beta = None if w.op == "rwkv6" else x["beta"][t0:t1].reshape(t1 - t0, N)[:, idx].double().numpy()
        decay = (x["decay"][t0:t1].reshape(t1 - t0, N)[:, idx].double().numpy() if w.op == "gdn"
                 else sel(x["decay"], t0, t1, d))
        ref = oracle.eager_run(w.op, sel(x["q"], t0, t1, d), sel(x["k"], t0, t1, d), sel(x["v"], t0, t1, d),
                               beta, decay, bonus, S, chk_steps=range(1, t1 - t0 + 1), nthreads=16)
        for m in range(t1 - t0):
            e = gs.assert_state(got[m].numpy(), ref["states"][m], (name, C, t0 + m + 1))
            worst = (max(worst[0], e[0]), max(worst[1], e[1]))
        S = ref["states"][-1]
    _log(f"every step, 256 heads, {name} C={C}: state rel {worst[0]:.3e} / per head {worst[1]:.3e}")


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
    eo, eo_el = gs.assert_outputs(outs.view(T, N, w.d)[:, hs].cpu().numpy(), ref["out"], (B, C))
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], (B, C, t))
    _log(f"sweep B={B} C={C}: out rel {eo:.3e} / per head {eo_el:.3e}")
