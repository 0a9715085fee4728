"""Edge cases of the decode path on the GPU, against the fp64 oracle.

The degenerate cases the method has: no decay (every log-decay stays 0), no
update (beta = 0), an exact overwrite (beta = 1 on a basis key), zero keys,
decays strong enough that the cumulative log-decay of a long cycle underflows
exp2 in fp32, a single head, an empty log (whose logical state is the base
itself, bit for bit), and a head count that splits unevenly over the launch
shapes of the decode kernels.
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


def _check(x, op, dtype, C, T):
    dev = gs.to_device(x, DEV)
    steps = list(range(T + 1))
    ref = gs.oracle_run(x, op, chk_steps=steps)
    outs, states, _ = gs.run_deltalog(dev, op, dtype, C, state_steps=steps)
    Bsz, H, d = x["q"].shape[1], x["q"].shape[2], x["v"].shape[-1]
    gs.assert_outputs(outs.cpu().numpy().reshape(T, Bsz * H, d), ref["out"])
    for t in steps:
        gs.assert_state(states[t].numpy(), ref["states"][t], t)
    return outs, states


@pytest.mark.parametrize("op,d", [(op, d) for op in ("gdn", "kda", "rwkv6") for d in (32, 64, 128)])
def test_single_head(op, d):
    """B = H = 1: one workgroup (one or two value tiles) per launch."""
    T, C = 11, 4
    x = workloads.generate(op, 1, 1, d, d, T, "bf16", seed=300 + d)
    _check(x, op, "bf16", C, T)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_no_decay(op):
    """decay = 1 everywhere: every cumulative log-decay is exactly 0."""
    T, Bsz, H, d, C = 13, 2, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=310)
    x["decay"] = torch.ones_like(x["decay"])
    _check(x, op, "bf16", C, T)


@pytest.mark.parametrize("op", ["gdn", "kda"])
def test_beta_zero_leaves_only_decay(op):
    """beta = 0: no token changes the state beyond its decay, so the logged
    value factors are 0 and the base after a fold is the decayed start."""
    T, Bsz, H, d, C = 9, 2, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=311)
    x["beta"] = torch.zeros_like(x["beta"])
    _check(x, op, "bf16", C, T)


@pytest.mark.parametrize("op", ["gdn", "kda"])
def test_exact_overwrite_on_basis_keys(op):
    """beta = 1 with k a basis vector e_c: the delta rule replaces row c of the
    (decayed) state with v, so S_t^T k_t = v_t after the step."""
    T, Bsz, H, d, C = 10, 1, 2, 32, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "f32", seed=312)
    g = torch.Generator().manual_seed(5)
    idx = torch.randint(0, d, (T, Bsz, H), generator=g)
    x["k"] = torch.nn.functional.one_hot(idx, d).to(torch.float32)
    x["beta"] = torch.ones_like(x["beta"])
    _, states = _check(x, op, "f32", C, T)
    # row idx of the state after step t equals v_t
    for t in range(1, T + 1):
        S = states[t].view(Bsz * H, d, d)
        rows = S[torch.arange(Bsz * H), idx[t - 1].reshape(-1)]
        ref = x["v"][t - 1].reshape(Bsz * H, d)
        assert gs.rel(rows.numpy(), ref.numpy()) <= 1e-5, t
        assert gs.head_err(rows.numpy(), ref.numpy(), 1) <= gs.ELEM_OUT_GATE, t


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_zero_keys(op):
    """k = 0: no token adds to the state; the replay coefficients are all 0."""
    T, Bsz, H, d, C = 9, 2, 2, 64, 8
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=313)
    x["k"] = torch.zeros_like(x["k"])
    _check(x, op, "bf16", C, T)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_strong_decay_underflows_cleanly(op):
    """decays of 0.01-0.1 per step over C = 32: the cumulative log-decay
    reaches about -200, exp2 of it underflows to 0 in fp32 exactly where the
    eager state has decayed below fp32 resolution, and nothing becomes NaN."""
    T, Bsz, H, d, C = 40, 2, 2, 64, 32
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=314)
    g = torch.Generator().manual_seed(6)
    x["decay"] = 0.01 + 0.09 * torch.rand(x["decay"].shape, generator=g)
    outs, states = _check(x, op, "bf16", C, T)
    assert torch.isfinite(outs).all()
    assert all(torch.isfinite(s).all() for s in states.values())


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_empty_log_is_the_base_bit_for_bit(op):
    """At L = 0 the logical state is 2^0 * base: materialise returns the base
    unchanged, right after init and right after a fold, and an early merge at
    L = 0 does nothing."""
    Bsz, H, d, C = 2, 3, 128, 4
    x = workloads.generate(op, Bsz, H, d, d, C, "bf16", seed=315)
    dev = gs.to_device(x, DEV)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, "bf16", base, C)
    assert torch.equal(st.materialize(), dev["S0"])
    st.merge()  # L = 0: a no-op
    torch.cuda.synchronize()
    assert torch.equal(base, dev["S0"])
    for t in range(C):  # one whole cycle: the last token folds
        st.step(**gs._token(dev, t))
    assert st.log_length == 0
    m = st.materialize()
    torch.cuda.synchronize()
    assert torch.equal(m, base)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_uneven_head_count_with_half_width_tail(op):
    """2049 heads of 128 x 128 (B = 2049, H = 1) at C = 8: the decode launches
    run the last 512 heads as two half-width tiles each, and the 1537 whole
    heads before them do not divide evenly over the eight XCDs' block ranges.
    A sample of heads that holds both sides of that boundary and both ends of
    the batch, against the oracle: outputs at every step and states at steps
    1, C - 1, C (right after the fold) and T."""
    Bsz, H, d, C, T = 2049, 1, 128, 8, 12
    N = Bsz * H
    nf = N - 512  # heads decoded whole
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=316)
    dev = gs.to_device(x, DEV)
    rng = np.random.default_rng(7)
    edges = [0, 1, nf - 2, nf - 1, nf, nf + 1, N - 2, N - 1]
    heads = np.unique(np.concatenate([edges, rng.choice(N, 56, replace=False)]))
    steps = [1, C - 1, C, T]
    ref = gs.oracle_run(x, op, heads=heads, chk_steps=steps, nthreads=16)
    outs, states, st = gs.run_deltalog(dev, op, "bf16", C, state_steps=steps, heads=heads)
    hs = torch.as_tensor(heads, dtype=torch.long, device=outs.device)
    gs.assert_outputs(outs.view(T, N, d)[:, hs].cpu().numpy(), ref["out"], (op, "uneven heads"))
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], (op, "uneven heads", t))
    assert st.log_length == T % C
