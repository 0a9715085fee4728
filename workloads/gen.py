"""Seeded input generator (shared by the GPU path's callers and the oracle's).

Recipe (one ``torch.Generator('cpu')`` per workload, seeded with
``seed_for(index)``; draws happen in this fixed order, each as one tensor over
all T tokens):

  1. S0    [B,H,dk,dv] fp32 ~ N(0, 0.02)        (0.02 is the standard deviation)
  2. bonus [H,dk]      fp32 ~ N(0, 0.1)         RWKV6 only
  3. q     [T,B,H,dk]  ~ N(0,1)                 (r for RWKV6)
  4. k     [T,B,H,dk]  ~ N(0,1)
  5. v     [T,B,H,dv]  ~ N(0,1)
  6. beta  [T,B,H]     = sigmoid(N(0,1))        GDN/KDA only
  7. decay  GDN  alpha [T,B,H]    ~ U(0.9, 1.0)
            KDA  a     [T,B,H,dk] = exp(-softplus(N(0,1)) * 0.1)
            RWKV6 w    [T,B,H,dk] = exp(-exp(N(-1, 0.5)))

For GDN and KDA, q and k are L2-normalised over dk in fp32.  q, k, v are then
rounded once to the input dtype (round-to-nearest-even for bf16); every other
tensor stays fp32.  Both the GPU run and the oracle consume exactly these
rounded values.  The seed does not depend on the log capacity C, so runs at
different C see identical inputs and can be compared with each other.
"""
from dataclasses import dataclass, field

import torch

_BASE_SEED = 20260816


def seed_for(index: int) -> int:
    """Seed of the workload with the given index in ``WORKLOADS`` order."""
    return _BASE_SEED + 100 * int(index)


@dataclass(frozen=True)
class Workload:
    """One decode workload: operator, shape, input dtype, steps and capacities."""
    name: str
    index: int
    op: str
    B: int
    H: int
    d: int
    T: int
    in_dtype: str
    capacities: tuple = field(default=(4,))

    @property
    def seed(self) -> int:
        return seed_for(self.index)

    @property
    def heads(self) -> int:
        return self.B * self.H

    @property
    def state_bytes(self) -> int:
        return self.B * self.H * self.d * self.d * 4


# The five workloads: a tiny fp32 GDN case, GDN/KDA/RWKV6 at serving shape,
# and the GDN sweep over capacity C and batch B.
WORKLOADS = {
    "gdn_b1_h2_d32": Workload("gdn_b1_h2_d32", 0, "gdn", 1, 2, 32, 64, "f32", (4, 1)),
    "gdn_b128_h32_d128": Workload("gdn_b128_h32_d128", 1, "gdn", 128, 32, 128, 256, "bf16", (4, 8)),
    "kda_b128_h32_d128": Workload("kda_b128_h32_d128", 2, "kda", 128, 32, 128, 256, "bf16", (4, 8)),
    "rwkv6_b128_h32_d64": Workload("rwkv6_b128_h32_d64", 3, "rwkv6", 128, 32, 64, 256, "bf16", (4, 8)),
    "gdn_sweep_c": Workload("gdn_sweep_c", 4, "gdn", 128, 32, 128, 128, "bf16", (1, 2, 4, 8, 16, 32)),
}

# The batch sweep of the same GDN workload at C=8 (same seed as the C sweep).
SWEEP_B = (16, 64, 256, 512)


def _dtype(name: str) -> torch.dtype:
    if name in ("bf16", "bfloat16"):
        return torch.bfloat16
    if name in ("f32", "fp32", "float32"):
        return torch.float32
    raise ValueError(f"unsupported input dtype {name!r}")


def generate(op: str, B: int, H: int, dk: int, dv: int, T: int,
             in_dtype: str = "bf16", seed: int = 0) -> dict:
    """Draw one workload's inputs on the CPU (see the module docstring).

    Returns a dict of CPU tensors: ``S0``, ``q``, ``k``, ``v``, ``beta``
    (None for RWKV6), ``decay`` and ``bonus`` (None unless RWKV6).
    """
    if op not in ("gdn", "kda", "rwkv6"):
        raise ValueError(f"unknown op {op!r}")
    dt = _dtype(in_dtype)
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    f32 = torch.float32
    S0 = torch.randn((B, H, dk, dv), generator=g, dtype=f32) * 0.02
    bonus = None
    if op == "rwkv6":
        bonus = torch.randn((H, dk), generator=g, dtype=f32) * 0.1
    q = torch.randn((T, B, H, dk), generator=g, dtype=f32)
    k = torch.randn((T, B, H, dk), generator=g, dtype=f32)
    v = torch.randn((T, B, H, dv), generator=g, dtype=f32)
    beta = None
    if op != "rwkv6":
        q = q / q.norm(dim=-1, keepdim=True)
        k = k / k.norm(dim=-1, keepdim=True)
        beta = torch.sigmoid(torch.randn((T, B, H), generator=g, dtype=f32))
    if op == "gdn":
        decay = 0.9 + 0.1 * torch.rand((T, B, H), generator=g, dtype=f32)
    elif op == "kda":
        x = torch.randn((T, B, H, dk), generator=g, dtype=f32)
        decay = torch.exp(-torch.nn.functional.softplus(x) * 0.1)
    else:
        x = torch.randn((T, B, H, dk), generator=g, dtype=f32) * 0.5 - 1.0
        decay = torch.exp(-torch.exp(x))
    return {
        "S0": S0.contiguous(),
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "beta": None if beta is None else beta.contiguous(),
        "decay": decay.contiguous(),
        "bonus": None if bonus is None else bonus.contiguous(),
    }


def generate_workload(w: Workload, B: int = None, T: int = None) -> dict:
    """Inputs of a named workload, optionally with another batch or step count."""
    return generate(w.op, B or w.B, w.H, w.d, w.d, T or w.T, w.in_dtype, w.seed)
