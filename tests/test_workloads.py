"""The seeded input generator: shapes, dtypes, reproducibility and distributions."""
import numpy as np
import pytest
import torch

import workloads


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_shapes_dtypes_and_reproducibility(op):
    a = workloads.generate(op, 2, 3, 16, 8, 5, "bf16", seed=123)
    b = workloads.generate(op, 2, 3, 16, 8, 5, "bf16", seed=123)
    c = workloads.generate(op, 2, 3, 16, 8, 5, "bf16", seed=124)
    assert a["S0"].shape == (2, 3, 16, 8) and a["S0"].dtype == torch.float32
    for name in ("q", "k"):
        assert a[name].shape == (5, 2, 3, 16) and a[name].dtype == torch.bfloat16
    assert a["v"].shape == (5, 2, 3, 8) and a["v"].dtype == torch.bfloat16
    if op == "rwkv6":
        assert a["beta"] is None and a["bonus"].shape == (3, 16)
        assert a["decay"].shape == (5, 2, 3, 16)
    else:
        assert a["bonus"] is None and a["beta"].shape == (5, 2, 3)
        assert a["decay"].shape == ((5, 2, 3) if op == "gdn" else (5, 2, 3, 16))
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key])
    assert not torch.equal(a["q"], c["q"])


def test_distributions():
    x = workloads.generate("gdn", 8, 4, 64, 64, 32, "f32", seed=5)
    n = x["q"].norm(dim=-1)
    assert torch.allclose(n, torch.ones_like(n), atol=1e-5)
    assert float(x["decay"].min()) >= 0.9 and float(x["decay"].max()) < 1.0
    assert 0.0 < float(x["beta"].min()) and float(x["beta"].max()) < 1.0
    assert abs(float(x["S0"].std()) - 0.02) < 0.002
    y = workloads.generate("kda", 8, 4, 64, 64, 32, "bf16", seed=6)
    assert float(y["decay"].min()) > 0.0 and float(y["decay"].max()) < 1.0
    z = workloads.generate("rwkv6", 8, 4, 64, 64, 32, "bf16", seed=7)
    # w = exp(-exp(x)), x ~ N(-1, 0.5): median exp(-exp(-1)) ~ 0.69
    med = float(z["decay"].median())
    assert 0.6 < med < 0.78
    assert abs(float(z["bonus"].std()) - 0.1) < 0.02
    assert abs(float(z["v"].float().std()) - 1.0) < 0.05


def test_bf16_values_upcast_exactly():
    x = workloads.generate("gdn", 1, 2, 32, 32, 4, "bf16", seed=9)
    q = x["q"]
    assert torch.equal(q.float().to(torch.bfloat16), q)
    assert np.array_equal(q.double().numpy(), q.float().numpy().astype(np.float64))


def test_named_workloads():
    w = workloads.WORKLOADS["gdn_b128_h32_d128"]
    assert (w.op, w.B, w.H, w.d, w.T, w.in_dtype) == ("gdn", 128, 32, 128, 256, "bf16")
    assert w.capacities == (4, 8)
    assert w.state_bytes == 128 * 32 * 128 * 128 * 4
    seeds = {wl.seed for wl in workloads.WORKLOADS.values()}
    assert len(seeds) == len(workloads.WORKLOADS)
