"""Per-slot logs (continuous batching) on the GPU, against the fp64 oracle.

Slots join and leave at different tokens, so each slot's log length differs
from the others'; every active slot's outputs and state must still equal the
eager recurrence of that slot's own token sequence from its own start state.
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


def _token(dev, t):
    return gs._token(dev, t)


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_all_slots_together_equals_lockstep(op):
    T, Bsz, H, d, C = 13, 3, 2, 128, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=31)
    dev = gs.to_device(x, DEV)
    lock, _, _ = gs.run_deltalog(dev, op, "bf16", C)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
    for b in range(Bsz):
        st.activate(b)
    outs = torch.empty_like(lock)
    for t in range(T):
        st.step(out=outs[t], **_token(dev, t))
        assert all(st.slot_log_length(b) == (t + 1) % C for b in range(Bsz))
    torch.cuda.synchronize()
    assert torch.equal(outs, lock)


@pytest.mark.parametrize("op", ["gdn", "kda"])
def test_all_slots_together_equals_lockstep_at_serving_shape(op):
    """B=128 H=32 d=128: the decode launches split the last 512 heads into
    half-width tiles, in the per-slot kernel as in the lockstep ones, so the
    two give the same bits there too (appends and folds, C=4)."""
    T, Bsz, H, d, C = 9, 128, 32, 128, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=37)
    dev = gs.to_device(x, DEV)
    lock, _, _ = gs.run_deltalog(dev, op, "bf16", C)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
    for b in range(Bsz):
        st.activate(b)
    outs = torch.empty_like(lock)
    for t in range(T):
        st.step(out=outs[t], **_token(dev, t))
    torch.cuda.synchronize()
    assert torch.equal(outs, lock)


def _segment_reference(x, op, slot, H, start, end, S0_seg, chk_end):
    """Oracle of one slot's heads over tokens [start, end) from S0_seg [H, d, d]."""
    sl = {}
    for key in ("q", "k", "v", "beta", "decay"):
        sl[key] = None if x[key] is None else x[key][start:end, slot:slot + 1]
    sl["bonus"] = x["bonus"]
    sl["S0"] = S0_seg[None]
    return gs.oracle_run(sl, op, chk_steps=[end - start] if chk_end else [])


@pytest.mark.parametrize("op,C", [("gdn", 4), ("kda", 3), ("rwkv6", 4), ("gdn", 1), ("kda", 8)])
def test_continuous_batching_schedule(op, C):
    T, Bsz, H, d = 24, 5, 2, 64
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=41 + C)
    dev = gs.to_device(x, DEV)
    # slot -> list of [start, end) active segments
    segments = {0: [(0, 24)], 1: [(1, 10), (13, 24)], 2: [(2, 24)], 3: [(5, 19)], 4: [(7, 24)]}
    g = torch.Generator().manual_seed(7 + C)
    seg_S0 = {(b, s): torch.randn((H, d, d), generator=g) * 0.02 for b, segs in segments.items()
              for s, _ in segs}
    base = torch.zeros((Bsz, H, d, d), dtype=torch.float32, device=DEV)
    st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
    outs = torch.full((T, Bsz, H, d), float("nan"), dtype=torch.float32, device=DEV)
    merge_after = {11, 17}
    expect = {}  # slot -> expected log length while active
    for t in range(T):
        for b, segs in segments.items():
            for s, e in segs:
                if e == t:
                    st.deactivate(b)
                    expect.pop(b, None)
                if s == t:
                    base[b].copy_(seg_S0[(b, s)].to(DEV))
                    st.activate(b)
                    expect[b] = 0
        st.step(out=outs[t], **_token(dev, t))
        for b in expect:
            expect[b] = (expect[b] + 1) % C
        if t + 1 in merge_after:
            st.merge()
            for b in expect:
                expect[b] = 0
        for b in range(Bsz):
            assert st.slot_log_length(b) == expect.get(b, -1), (t, b)
    final = st.materialize(torch.full_like(base, float("nan")))
    torch.cuda.synchronize()
    o = outs.cpu().numpy()
    fin = final.cpu().numpy()
    for b, segs in segments.items():
        for s, e in segs:
            ref = _segment_reference(x, op, b, H, s, e, seg_S0[(b, s)], chk_end=(e == T))
            got = o[s:e, b]  # [steps, H, d]
            gs.assert_outputs(got, ref["out"], (b, s, e))
            if e == T:
                gs.assert_state(fin[b], ref["states"][0], b)
        # steps where the slot was inactive keep the untouched (NaN) output
        active = np.zeros(T, dtype=bool)
        for s, e in segs:
            active[s:e] = True
        assert np.isnan(o[~active, b]).all()
    # slot 3 ended before T: materialise leaves inactive slots untouched
    assert np.isnan(fin[3]).all()


@pytest.mark.parametrize("op,slots", [("gdn", False), ("kda", True), ("rwkv6", True), ("rwkv6", False)])
def test_materialize_slot_is_the_slice_of_the_full_state(op, slots):
    T, Bsz, H, d, C = 6, 3, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=51)
    dev = gs.to_device(x, DEV)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, "bf16", base, C, slots=slots)
    if slots:
        for b in range(Bsz):
            st.activate(b)
    for t in range(T):  # ends mid-cycle: the log is not empty
        st.step(**_token(dev, t))
    full = st.materialize()
    for b in range(Bsz):
        one = st.materialize_slot(b)
        torch.cuda.synchronize()
        assert torch.equal(one, full[b]), b


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_slot_merge_is_output_neutral_and_local(op):
    """Folding one slot's log early changes no output and empties only that log."""
    T, Bsz, H, d, C = 14, 3, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=52)
    dev = gs.to_device(x, DEV)
    runs = []
    for merge in (False, True):
        base = dev["S0"].clone()
        st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
        for b in range(Bsz):
            st.activate(b)
        outs = torch.empty((T, Bsz, H, d), dtype=torch.float32, device=DEV)
        for t in range(T):
            st.step(out=outs[t], **_token(dev, t))
            if merge and t in (2, 9):
                lengths = [st.slot_log_length(b) for b in range(Bsz)]
                st.merge_slot(1)
                assert st.slot_log_length(1) == 0
                assert [st.slot_log_length(b) for b in (0, 2)] == [lengths[0], lengths[2]]
        torch.cuda.synchronize()
        runs.append(outs.cpu())
    gs.assert_close_pair(runs[1], runs[0], 1, 1e-5, "merged vs not")
    ref = gs.oracle_run(x, op)
    gs.assert_outputs(runs[1].numpy().reshape(T, Bsz * H, d), ref["out"])


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_evict_and_resume_a_request(op):
    """Slot 1's request is saved with materialize_slot and leaves at token 5;
    another request uses the slot for a while; the first one comes back at
    token 9 from its saved state and continues with its own tokens 5..T-1:
    its outputs equal the oracle of its uninterrupted sequence."""
    T, Bsz, H, d, C = 13, 2, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=53)
    other = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=54)
    dev, dev_o = gs.to_device(x, DEV), gs.to_device(other, DEV)
    base = dev["S0"].clone()
    st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
    st.activate(0)
    st.activate(1)
    outs = torch.full((T, Bsz, H, d), float("nan"), dtype=torch.float32, device=DEV)
    for t in range(5):
        st.step(out=outs[t], **_token(dev, t))
    saved = st.materialize_slot(1)
    st.deactivate(1)
    base[1].copy_(dev_o["S0"][1])  # another request takes the slot
    st.activate(1)
    for t in range(5, 9):  # slot 0 keeps its own tokens; slot 1 decodes the other request's
        tok = _token(dev, t)
        tok_o = _token(dev_o, t)
        mixed = {k: (None if v is None else (v if k == "bonus" else torch.stack([v[0], tok_o[k][1]])))
                 for k, v in tok.items()}
        st.step(out=outs[t], **mixed)
    st.deactivate(1)
    base[1].copy_(saved)  # the first request returns
    st.activate(1)
    # slot 1 continues with its own tokens 5.. while slot 0 continues with tokens 9..
    resumed = torch.empty((T - 9, Bsz, H, d), dtype=torch.float32, device=DEV)
    for i in range(T - 9):
        t0, t1 = 9 + i, 5 + i
        tok0, tok1 = _token(dev, t0), _token(dev, t1)
        mixed = {k: (None if v is None else (v if k == "bonus" else torch.stack([v[0], tok1[k][1]])))
                 for k, v in tok0.items()}
        st.step(out=resumed[i], **mixed)
    torch.cuda.synchronize()
    ref = gs.oracle_run(x, op)  # both slots' uninterrupted sequences
    ro = ref["out"].reshape(T, Bsz, H, d)
    r = resumed.cpu().numpy()
    n = T - 9
    gs.assert_outputs(r[:, 1], ro[5:5 + n, 1], "slot 1 resumed")
    gs.assert_outputs(r[:, 0], ro[9:9 + n, 0], "slot 0 uninterrupted")


@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_tokens_on_a_per_slot_handle_equal_single_steps(op):
    """dl_decode_tokens on a per-slot handle (slots started at different
    tokens, so their logs fill at different tokens) equals one step per token
    up to rounding: the chunk kernel adds the same terms in another order."""
    T, Bsz, H, d, C = 12, 3, 2, 64, 4
    x = workloads.generate(op, Bsz, H, d, d, T, "bf16", seed=55)
    dev = gs.to_device(x, DEV)
    chunks = [(0, 1), (1, 2), (2, 5), (5, 12)]  # slot b joins at token b
    runs = []
    for fused in (False, True):
        base = dev["S0"].clone()
        st = dl.DeltaLogState(op, "bf16", base, C, slots=True)
        outs = torch.full((T, Bsz, H, d), float("nan"), dtype=torch.float32, device=DEV)
        for t0, t1 in chunks:
            if t0 < Bsz:
                st.activate(t0)
            if fused:
                tok = {k: (v if v is None or k == "bonus" else v[t0:t1]) for k, v in dev.items()
                       if k in ("q", "k", "v", "beta", "decay", "bonus")}
                st.step_tokens(out=outs[t0:t1], **tok)
            else:
                for t in range(t0, t1):
                    st.step(out=outs[t], **_token(dev, t))
        torch.cuda.synchronize()
        runs.append((outs.cpu(), st.materialize().cpu(), [st.slot_log_length(b) for b in range(Bsz)]))
    # slots not yet started keep their NaN outputs in both runs
    assert torch.equal(torch.isnan(runs[0][0]), torch.isnan(runs[1][0]))
    a, b = torch.nan_to_num(runs[0][0]), torch.nan_to_num(runs[1][0])
    gs.assert_close_pair(b, a, 1, 1e-5, "outputs")
    gs.assert_close_pair(runs[1][1], runs[0][1], 2, 1e-5, "state")
    assert runs[0][2] == runs[1][2]


CHUNK_CASES = [("gdn", "bf16", 128, 8), ("kda", "bf16", 128, 4), ("rwkv6", "bf16", 64, 8),
               ("gdn", "f32", 32, 3), ("kda", "f32", 64, 13), ("rwkv6", "bf16", 128, 5),
               ("gdn", "f32", 128, 6), ("kda", "f32", 128, 8), ("rwkv6", "f32", 128, 8),
               ("kda", "bf16", 128, 16), ("gdn", "bf16", 128, 32), ("gdn", "bf16", 64, 1)]


@pytest.mark.parametrize("op,dtype,d,C", CHUNK_CASES)
def test_continuous_batching_in_chunks(op, dtype, d, C):
    """Slots join, leave and rejoin between calls of up to eight tokens, so one
    call finds every slot at its own log length; some calls cross a slot's
    fold once or (C < 8) several times.  Every active slot's outputs and its
    final state must equal the oracle of its own token sequence."""
    T, Bsz, H = 30, 5, 2
    x = workloads.generate(op, Bsz, H, d, d, T, dtype, seed=61 + C + d)
    dev = gs.to_device(x, DEV)
    segments = {0: [(0, 30)], 1: [(3, 14), (17, 30)], 2: [(3, 30)], 3: [(6, 22)], 4: [(9, 30)]}
    events = sorted({t for segs in segments.values() for se in segs for t in se} | {T})
    g = torch.Generator().manual_seed(17 + C)
    seg_S0 = {(b, s): torch.randn((H, d, d), generator=g) * 0.02 for b, segs in segments.items()
              for s, _ in segs}
    base = torch.zeros((Bsz, H, d, d), dtype=torch.float32, device=DEV)
    st = dl.DeltaLogState(op, dtype, base, C, slots=True)
    outs = torch.full((T, Bsz, H, d), float("nan"), dtype=torch.float32, device=DEV)
    sizes = [5, 8, 3, 7, 2, 6, 1, 8]
    expect, t, i, calls = {}, 0, 0, 0
    while t < T:
        for b, segs in segments.items():
            for s, e in segs:
                if e == t:
                    st.deactivate(b)
                    expect.pop(b, None)
                if s == t:
                    base[b].copy_(seg_S0[(b, s)].to(DEV))
                    st.activate(b)
                    expect[b] = 0
        t1 = min(t + sizes[i % len(sizes)], next(e for e in events if e > t))
        i += 1
        tok = {k: (v if v is None or k == "bonus" else v[t:t1]) for k, v in dev.items()
               if k in ("q", "k", "v", "beta", "decay", "bonus")}
        st.step_tokens(out=outs[t:t1], **tok)
        calls += 1
        for b in expect:
            expect[b] = (expect[b] + t1 - t) % C
        if calls == 4:
            st.merge()
            for b in expect:
                expect[b] = 0
        for b in range(Bsz):
            assert st.slot_log_length(b) == expect.get(b, -1), (t1, b)
        t = t1
    final = st.materialize(torch.full_like(base, float("nan")))
    torch.cuda.synchronize()
    o = outs.cpu().numpy()
    fin = final.cpu().numpy()
    for b, segs in segments.items():
        for s, e in segs:
            ref = _segment_reference(x, op, b, H, s, e, seg_S0[(b, s)], chk_end=(e == T))
            gs.assert_outputs(o[s:e, b], ref["out"], (b, s, e))
            if e == T:
                gs.assert_state(fin[b], ref["states"][0], b)
        active = np.zeros(T, dtype=bool)
        for s, e in segs:
            active[s:e] = True
        assert np.isnan(o[~active, b]).all()
    assert np.isnan(fin[3]).all()


def test_full_size_staggered_calls_of_eight():
    """The staggered serving shape the multi-token bench times: GDN B=128 H=32
    d=128 C=8, slot b started at token b mod 8 (single steps while the slots
    join), then calls of eight tokens, every call folding seven slots in eight
    in its middle.  Eight sampled slots (all their heads): every output and the
    final state against the oracle of each slot's own tokens."""
    w = workloads.WORKLOADS["gdn_b128_h32_d128"]
    T, C = 32, 8
    x = workloads.generate_workload(w, T=T)
    dev = gs.to_device(x, DEV)
    base = dev["S0"].clone()
    st = dl.DeltaLogState("gdn", w.in_dtype, base, C, slots=True)
    outs = torch.full((T, w.B, w.H, w.d), float("nan"), dtype=torch.float32, device=DEV)
    for t in range(C):
        for b in range(t, w.B, C):
            st.activate(b)
        st.step(out=outs[t], **_token(dev, t))
    for t0 in range(C, T, 8):
        tok = {k: (v if v is None or k == "bonus" else v[t0:t0 + 8]) for k, v in dev.items()
               if k in ("q", "k", "v", "beta", "decay", "bonus")}
        st.step_tokens(out=outs[t0:t0 + 8], **tok)
    final = st.materialize()
    torch.cuda.synchronize()
    for b in (0, 1, 6, 7, 63, 64, 121, 127):
        s = b % C
        ref = _segment_reference(x, "gdn", b, w.H, s, T, x["S0"][b], chk_end=True)
        gs.assert_outputs(outs[s:, b].cpu().numpy(), ref["out"], b)
        gs.assert_state(final[b].cpu().numpy(), ref["states"][0], b)
        assert np.isnan(outs[:s, b].cpu().numpy()).all()
