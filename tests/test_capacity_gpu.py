"""The capacity the library's chooser picks, run on the GPU against the oracle.

dl_choose_capacity picks the log capacity C (the merge interval) that
balances replay traffic against dense-write savings (gist.science summary,
"Modello di Traffico").  Whatever C it picks must decode exactly like any
other: at serving shape, GDN and KDA with the pick (a capacity that does not
divide the 256 tokens, so the last cycle is partial), every output of 64
sampled heads and their states right after folds and at the end.
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


@pytest.mark.parametrize("name", ["gdn_b128_h32_d128", "kda_b128_h32_d128", "rwkv6_b128_h32_d64"])
def test_chosen_capacity_against_oracle(name):
    w = workloads.WORKLOADS[name]
    cfg = dl.make_config(w.op, w.in_dtype, w.B, w.H, w.d, w.d, 8)
    C = dl.dl_choose_capacity(cfg, dl.DL_MAX_CAPACITY)
    assert 2 <= C <= dl.DL_MAX_CAPACITY
    x = workloads.generate_workload(w)
    dev = gs.to_device(x, DEV)
    T, N = w.T, w.heads
    heads = gs.head_sample(N, 64, seed=C)
    steps = sorted({C, 2 * C, (T // C) * C, T})
    ref = gs.oracle_run(x, w.op, heads=heads, chk_steps=steps, nthreads=16)
    outs, states, st = gs.run_deltalog(dev, w.op, w.in_dtype, C, state_steps=steps, heads=heads)
    hs = torch.as_tensor(heads, dtype=torch.long, device=DEV)
    eo, eo_el = gs.assert_outputs(outs.view(T, N, w.d)[:, hs].cpu().numpy(), ref["out"], (name, C))
    for m, t in enumerate(steps):
        gs.assert_state(states[t].numpy(), ref["states"][m], (name, C, t))
    assert st.log_length == T % C
    print(f"{name}: chosen C = {C}, out rel {eo:.3e} / per head {eo_el:.3e}", flush=True)
