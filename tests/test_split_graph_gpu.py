"""Split replay and graph replay of a merge cycle on the GPU.

Split replay runs each append as two launches: a once-per-head key-side
stage (scaled key and query, replay coefficients, the token's scalar term)
and the value-tile stage that reads its record (gist.science summary,
"Implementazione del Kernel": a shared ReplayPrep stage, then parallel
AppendDecode stages).  It must give the oracle's results like the fused
form.  Graph replay (signal-papers summary, Fig. 9) records one whole cycle
and replays it on refilled input buffers; every replay must equal the same
tokens decoded call by call.
"""
import sys

import pytest
import torch

import recurrent_state_updates_amd as dl
import workloads
from recurrent_state_updates_amd._binding import DL_ERR_ARG
from tests import gpu_support as gs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu tests must run on an MI355X")
    dl.load_library()
    yield


SMALL = [(op, dtype, d, C) for op in ("gdn", "kda", "rwkv6")
         for dtype, d in (("f32", 32), ("bf16", 64), ("bf16", 128)) for C in (3, 8, 13)]


@pytest.mark.parametrize("op,dtype,d,C", SMALL)
def test_split_every_step(op, dtype, d, C):
    """Outputs and materialised states at every step against the oracle, and
    equal to the fused form's; T = 2C + 3 ends inside a cycle."""
    T, Bsz, H = 2 * C + 3, 3, 2
    x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=70 + C + d)
    dev = gs.to_device(x, DEV)
    steps = list(range(1, T + 1))
    ref = gs.oracle_run(x, op, chk_steps=steps)
    outs, states, st = gs.run_deltalog(dev, op, dtype, C, state_steps=steps, split_replay=True)
    fused, _, _ = gs.run_deltalog(dev, op, dtype, C)
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, d), ref["out"])
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], t)
    gs.assert_close_pair(outs, fused, 1, 1e-6, "split vs fused")
    assert st.log_length == T % C


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_split_log_equals_fused(op):
    """Mid-cycle, the log the split form wrote equals the fused form's: key
    copies and log-decays exactly (the key-side stage computes them the same
    way), value factors to fp32 rounding."""
    C, T, Bsz, H, d = 8, 5, 2, 2, 128
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=81)
    dev = gs.to_device(x, DEV)
    logs = []
    for split in (False, True):
        _, _, st = gs.run_deltalog(dev, op, "bf16", C, split_replay=split)
        X, K, G = st.workspace_views()
        logs.append((X[:, :, :T].float().cpu(), K[:, :, :T].cpu(), G[:, :, :T].cpu()))
    (xf, kf, gf), (xs, ks, gs_) = logs
    assert torch.equal(kf, ks)
    assert torch.equal(gf, gs_)
    gs.assert_close_pair(xs, xf, 1, 1e-6, "value factors")


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_switching_mid_cycle(op):
    """Toggling between the fused and the split form at any step leaves the
    outputs unchanged: both read and write the same log."""
    C, T, Bsz, H, d = 4, 13, 2, 3, 64
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=82)
    dev = gs.to_device(x, DEV)
    fused, _, _ = gs.run_deltalog(dev, op, "bf16", C)
    toggles = {2, 3, 6, 9, 10}

    def flip(t, st):
        if t in toggles:
            st.set_split_replay(st.prep is None or t % 2 == 0)

    mixed, _, _ = gs.run_deltalog(dev, op, "bf16", C, on_step=flip)
    gs.assert_close_pair(mixed, fused, 1, 1e-6, "switching vs fused")


def _static_tokens(dev, C, Bsz, H, d):
    """Input and output buffers of one cycle, refilled before each replay."""
    def like(t):
        return torch.empty((C,) + tuple(t.shape[1:]), dtype=t.dtype, device=t.device)
    buf = {k: like(dev[k]) for k in ("q", "k", "v", "decay")}
    buf["beta"] = None if dev["beta"] is None else like(dev["beta"])
    buf["out"] = torch.empty((C, Bsz, H, d), dtype=torch.float32, device=DEV)
    tokens = [dict(q=buf["q"][i], k=buf["k"][i], v=buf["v"][i],
                   beta=None if buf["beta"] is None else buf["beta"][i], decay=buf["decay"][i],
                   bonus=dev["bonus"], out=buf["out"][i]) for i in range(C)]
    return buf, tokens


@pytest.mark.parametrize("op,split", [(op, s) for op in ("gdn", "kda", "rwkv6") for s in (False, True)])
def test_graph_replay_equals_direct(op, split):
    """Four replays of one captured cycle, inputs refilled in place and other
    device work (materialise, torch kernels) between them: each replay's
    outputs and the final base equal the call-by-call run bit for bit, and
    the final state matches the oracle."""
    C, R, Bsz, H, d = 4, 4, 2, 3, 128
    T = C * R
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=83)
    dev = gs.to_device(x, DEV)
    direct, _, dst = gs.run_deltalog(dev, op, "bf16", C, split_replay=split)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, "bf16", base, C, split_replay=split)
    buf, tokens = _static_tokens(dev, C, Bsz, H, d)
    graph = st.capture_cycle(tokens)
    assert st.log_length == 0
    scratch = torch.empty_like(base)
    noise = torch.randn((512, 512), device=DEV)
    for r in range(R):
        sl = slice(r * C, (r + 1) * C)
        for k in ("q", "k", "v", "decay", "beta"):
            if buf[k] is not None:
                buf[k].copy_(dev[k][sl])
        buf["out"].fill_(float("nan"))
        noise = noise @ noise.t() * 1e-3
        graph.launch()
        st.materialize(scratch)
        torch.cuda.synchronize()
        assert torch.equal(buf["out"], direct[sl]), r
        assert st.log_length == 0
    assert torch.equal(base, dst.base)
    ref = gs.oracle_run(x, op, chk_steps=[T])
    gs.assert_state(base.cpu().numpy().reshape(Bsz * H, d, d), ref["states"][0])
    graph.close()


def test_graph_needs_an_empty_log():
    C, Bsz, H, d = 4, 1, 2, 64
    x = workloads.generate("gdn", Bsz, H, d, d, 2, "bf16", seed=84)
    dev = gs.to_device(x, DEV)
    base = dev["S0"].clone()
    st = dl.DeltaLogState("gdn", "bf16", base, C)
    _, tokens = _static_tokens(dev, C, Bsz, H, d)
    graph = st.capture_cycle(tokens)
    st.step(**gs._token(dev, 0))  # L = 1: a replay would start mid-cycle
    with pytest.raises(dl.DeltaLogError) as e:
        graph.launch()
    assert e.value.status == DL_ERR_ARG
    with pytest.raises(dl.DeltaLogError):
        st.capture_cycle(tokens)
    torch.cuda.synchronize()
    graph.close()


_CACHE = {}


def _workload_inputs(name):
    if name not in _CACHE:
        _CACHE.clear()
        w = workloads.WORKLOADS[name]
        _log(f"generating {name}")
        x = workloads.generate_workload(w)
        _CACHE[name] = (w, x, gs.to_device(x, DEV))
    return _CACHE[name]


@pytest.mark.parametrize("name", ["gdn_b128_h32_d128", "kda_b128_h32_d128", "rwkv6_b128_h32_d64"])
def test_full_size_split_against_oracle(name):
    """Serving-shape workloads at C = 8 in the split form: sampled heads every
    step and states after folds against the oracle; all heads against the
    fused form."""
    C = 8
    w, x, dev = _workload_inputs(name)
    T, N = w.T, w.heads
    heads = gs.head_sample(N, 64, seed=5)
    steps = sorted({C // 2, C, T - C // 2, T})
    _log(f"split {name}: oracle on {len(heads)} heads")
    ref = gs.oracle_run(x, w.op, heads=heads, chk_steps=steps, nthreads=16)
    outs, states, _ = gs.run_deltalog(dev, w.op, w.in_dtype, C, state_steps=steps, heads=heads,
                                      split_replay=True)
    hs = torch.as_tensor(heads, dtype=torch.long, device=outs.device)
    eo, eo_el = gs.assert_outputs(outs.view(T, N, w.d)[:, hs].cpu().numpy(), ref["out"])
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], t)
    _log(f"  out rel {eo:.3e} / per head {eo_el:.3e}")
    fused, _, _ = gs.run_deltalog(dev, w.op, w.in_dtype, C)
    ef = gs.assert_close_pair(outs, fused, 1, 1e-6, "split vs fused")
    _log(f"  split vs fused (all heads) rel / per head {ef}")
