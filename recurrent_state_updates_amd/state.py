"""Torch-tensor front end of the C ABI: memory and streams only.

PyTorch allocates the base state, the log workspace and the outputs and
supplies the current HIP stream; every step of the decode path runs in the
library's kernels.  Shapes and dtypes are checked here so that a wrong
tensor fails before it reaches the device.
"""
import torch

from . import _binding as B

_IN_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


def _stream(device):
    return torch.cuda.current_stream(device).cuda_stream


def _check_tensor(name, t, shape, dtype, device):
    if t is None:
        raise ValueError(f"{name} is required")
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must live on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _addr(t):
    return 0 if t is None else t.data_ptr()


def make_step_args(op, in_dtype, Bsz, H, dk, dv, device, q, k, v, beta, decay, bonus, out):
    """Validate one token's tensors and pack them into a StepArgs."""
    tin = _IN_DTYPES[in_dtype]
    _check_tensor("q", q, (Bsz, H, dk), tin, device)
    _check_tensor("k", k, (Bsz, H, dk), tin, device)
    _check_tensor("v", v, (Bsz, H, dv), tin, device)
    _check_tensor("out", out, (Bsz, H, dv), torch.float32, device)
    if op == "gdn":
        _check_tensor("decay", decay, (Bsz, H), torch.float32, device)
    else:
        _check_tensor("decay", decay, (Bsz, H, dk), torch.float32, device)
    if op == "rwkv6":
        if beta is not None:
            raise ValueError("beta must be None for RWKV6")
        _check_tensor("bonus", bonus, (H, dk), torch.float32, device)
    else:
        _check_tensor("beta", beta, (Bsz, H), torch.float32, device)
        if bonus is not None:
            raise ValueError("bonus must be None for GDN and KDA")
    return B.StepArgs(_addr(q), _addr(k), _addr(v), _addr(beta), _addr(decay), _addr(bonus),
                      _addr(out))


class DeltaLogState:
    """A base state plus its log workspace, driven through dl_decode_step.

    ``base`` is a caller-owned [B, H, d, d] fp32 CUDA tensor; it is updated in
    place at every fold.  The workspace is allocated here with torch.  With
    ``slots=True`` every slot keeps its own log length (continuous batching):
    slots start inactive and are switched with ``activate`` / ``deactivate``.
    ``split_replay=True`` runs each append as the staged pair (a once-per-head
    key-side launch, then the value tiles) with a prep buffer allocated here.
    """

    def __init__(self, op, in_dtype, base, C, slots=False, split_replay=False):
        if op not in B.OP_CODES or in_dtype not in B.DTYPE_CODES:
            raise ValueError(f"unknown op {op!r} or dtype {in_dtype!r}")
        if base.dim() != 4:
            raise ValueError("base must be [B, H, dk, dv]")
        Bsz, H, dk, dv = base.shape
        self.device = base.device
        _check_tensor("base", base, (Bsz, H, dk, dv), torch.float32, self.device)
        self.op, self.in_dtype, self.C = op, in_dtype, int(C)
        self.B, self.H, self.dk, self.dv = int(Bsz), int(H), int(dk), int(dv)
        self.cfg = B.make_config(op, in_dtype, self.B, self.H, self.dk, self.dv, self.C)
        B.dl_workspace_layout(self.cfg)  # raises with the library's reason for a bad config
        nbytes = B.dl_workspace_bytes(self.cfg)
        self.base = base
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.slots = bool(slots)
        if self.slots:
            self.handle = B.dl_state_init_slots(self.cfg, base.data_ptr(), self.workspace.data_ptr(), nbytes,
                                                _stream(self.device))
        else:
            self.handle = B.dl_state_init(self.cfg, base.data_ptr(), self.workspace.data_ptr(), nbytes)
        self.prep = None
        if split_replay:
            self.set_split_replay(True)

    def set_split_replay(self, on):
        """Switch between the fused (False) and the split (True) replay preparation."""
        if on:
            if self.prep is None:
                self.prep = torch.empty(B.dl_prep_bytes(self.cfg), dtype=torch.uint8, device=self.device)
            B.dl_set_split_replay(self.handle, self.prep.data_ptr(), self.prep.numel())
        else:
            B.dl_set_split_replay(self.handle, 0, 0)

    def step(self, q, k, v, beta, decay, bonus=None, out=None):
        """Decode one token for all heads; returns out [B, H, dv] fp32."""
        if out is None:
            out = torch.empty((self.B, self.H, self.dv), dtype=torch.float32, device=self.device)
        args = make_step_args(self.op, self.in_dtype, self.B, self.H, self.dk, self.dv,
                              self.device, q, k, v, beta, decay, bonus, out)
        B.dl_decode_step(self.handle, args, _stream(self.device))
        return out

    def step_noalloc(self, q, k, v, beta, decay, bonus=None, out=None):
        """dl_decode_step_noalloc: one token in the split-replay form with the
        library's static scratch (no prep buffer of this handle is used)."""
        if out is None:
            out = torch.empty((self.B, self.H, self.dv), dtype=torch.float32, device=self.device)
        args = make_step_args(self.op, self.in_dtype, self.B, self.H, self.dk, self.dv,
                              self.device, q, k, v, beta, decay, bonus, out)
        B.dl_decode_step_noalloc(self.handle, args, _stream(self.device))
        return out

    def step_tokens(self, q, k, v, beta, decay, bonus=None, out=None):
        """Decode K tokens in one call (dl_decode_tokens).  q, k, v, beta, decay
        carry a leading token axis [K, ...]; returns out [K, B, H, dv] fp32."""
        K = q.shape[0]
        for name, t in (("k", k), ("v", v), ("beta", beta), ("decay", decay), ("out", out)):
            if t is not None and t.shape[0] != K:
                raise ValueError(f"{name} carries {t.shape[0]} tokens, q carries {K}")
        if out is None:
            out = torch.empty((K, self.B, self.H, self.dv), dtype=torch.float32, device=self.device)
        args = [make_step_args(self.op, self.in_dtype, self.B, self.H, self.dk, self.dv, self.device,
                               q[t], k[t], v[t], None if beta is None else beta[t], decay[t], bonus, out[t])
                for t in range(K)]
        B.dl_decode_tokens(self.handle, args, _stream(self.device))
        return out

    def step_args(self, q, k, v, beta, decay, bonus, out):
        """Pre-validated StepArgs for repeated low-overhead ``step_packed`` calls."""
        return make_step_args(self.op, self.in_dtype, self.B, self.H, self.dk, self.dv,
                              self.device, q, k, v, beta, decay, bonus, out)

    def step_packed(self, args, stream=None):
        B.dl_decode_step(self.handle, args, _stream(self.device) if stream is None else stream)

    def capture_cycle(self, tokens):
        """Record one merge cycle as a HIP graph.  ``tokens`` holds C dicts of the
        step inputs (q, k, v, beta, decay, bonus, out); the graph replays on those
        same tensors, so refill them in place between replays."""
        if len(tokens) != self.C:
            raise ValueError(f"a cycle is {self.C} tokens, got {len(tokens)}")
        args = [self.step_args(t["q"], t["k"], t["v"], t.get("beta"), t["decay"], t.get("bonus"), t["out"])
                for t in tokens]
        return CycleGraph(self, B.dl_graph_capture_cycle(self.handle, args), tokens)

    def merge(self):
        B.dl_merge(self.handle, _stream(self.device))

    def materialize(self, dst=None):
        if dst is None:
            dst = torch.empty_like(self.base)
        _check_tensor("dst", dst, tuple(self.base.shape), torch.float32, self.device)
        B.dl_materialize(self.handle, dst.data_ptr(), _stream(self.device))
        return dst

    @property
    def log_length(self):
        return B.dl_log_length(self.handle)

    def activate(self, slot):
        B.dl_slot_activate(self.handle, slot, _stream(self.device))

    def deactivate(self, slot):
        B.dl_slot_deactivate(self.handle, slot, _stream(self.device))

    def slot_log_length(self, slot):
        return B.dl_slot_log_length(self.handle, slot)

    def materialize_slot(self, slot, dst=None):
        """The logical [H, dk, dv] state of one slot (e.g. of a request that leaves)."""
        if dst is None:
            dst = torch.empty(tuple(self.base.shape[1:]), dtype=torch.float32, device=self.device)
        _check_tensor("dst", dst, tuple(self.base.shape[1:]), torch.float32, self.device)
        B.dl_materialize_slot(self.handle, slot, dst.data_ptr(), _stream(self.device))
        return dst

    def merge_slot(self, slot):
        """Fold one slot's log into its base block now (per-slot handles)."""
        B.dl_slot_merge(self.handle, slot, _stream(self.device))

    def workspace_views(self):
        """(X, K, G) views of the log for inspection: [B,H,C,dv], [B,H,C,dk], [B,H,C(,dk)]."""
        ox, ok, og = B.dl_workspace_layout(self.cfg)
        Bsz, H, C, dk, dv = self.B, self.H, self.C, self.dk, self.dv
        n = Bsz * H * C
        tin = _IN_DTYPES[self.in_dtype]
        xdt = tin if self.op == "rwkv6" else torch.float32
        ws = self.workspace
        X = ws[ox:ox + n * dv * xdt.itemsize].view(xdt).view(Bsz, H, C, dv)
        K = ws[ok:ok + n * dk * tin.itemsize].view(tin).view(Bsz, H, C, dk)
        gw = 1 if self.op == "gdn" else dk
        G = ws[og:og + n * gw * 4].view(torch.float32).view(Bsz, H, C, gw)
        return X, K, G

    def close(self):
        if getattr(self, "handle", None):
            B.dl_state_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CycleGraph:
    """One captured merge cycle of a DeltaLogState (dl_graph_capture_cycle)."""

    def __init__(self, state, graph, tokens):
        self.state, self.graph = state, graph
        self._keep = tokens  # the recorded tensors must outlive the graph

    def launch(self, stream=None):
        B.dl_graph_launch(self.graph, _stream(self.state.device) if stream is None else stream)

    def close(self):
        if getattr(self, "graph", None):
            B.dl_graph_destroy(self.graph)
            self.graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def eager_step(op, in_dtype, state, q, k, v, beta, decay, bonus=None, out=None):
    """The eager dense update on ``state`` in place (dl_eager_step); returns out."""
    Bsz, H, dk, dv = state.shape
    _check_tensor("state", state, (Bsz, H, dk, dv), torch.float32, state.device)
    if out is None:
        out = torch.empty((Bsz, H, dv), dtype=torch.float32, device=state.device)
    cfg = B.make_config(op, in_dtype, Bsz, H, dk, dv, 1)
    args = make_step_args(op, in_dtype, Bsz, H, dk, dv, state.device, q, k, v, beta, decay, bonus, out)
    B.dl_eager_step(cfg, state.data_ptr(), args, _stream(state.device))
    return out
