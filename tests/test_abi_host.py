"""Host side of the C ABI, on the CPU: exports, sizing and argument validation.

No call here reaches a kernel: every call either fails validation before any
HIP call, or (``dl_state_init``, ``dl_merge`` at L = 0, ``dl_log_length``,
``dl_state_destroy``) does no device work by design.  Device addresses are
fake, aligned integers that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import recurrent_state_updates_amd as dl
from recurrent_state_updates_amd import _binding as B
from recurrent_state_updates_amd import build as dlbuild

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]
FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced
# a fake device layout with no two buffers overlapping: the base at FAKE, the
# workspace, the token inputs 1 MB apart, the prep records, a materialise dst
WS = FAKE + 0x10000000
IN = FAKE + 0x20000000
PREP = FAKE + 0x30000000
DST = FAKE + 0x40000000


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(B.LIB_PATH):
        dlbuild.build()
    return B.load_library()


def declared_functions():
    names = set()
    for path in HEADERS:
        with open(path) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(dl_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert len(names) == 30, names
    for name in names:
        assert hasattr(lib, name), f"{name} is declared in deltalog.h but not exported"
    for name in names:
        assert hasattr(dl, name), f"the Python binding lacks {name}"


def test_status_strings():
    assert dl.dl_status_string(0) == "ok"
    for code in (-1, -2, -3, -4, -5):
        assert dl.dl_status_string(code) not in ("", "unknown status")
    assert dl.dl_status_string(-99) == "unknown status"


def _round(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("op,dtype,d,dv,C", [("gdn", "bf16", 128, 128, 8), ("kda", "bf16", 128, 128, 4),
                                             ("rwkv6", "bf16", 64, 64, 8), ("gdn", "f32", 32, 32, 4),
                                             ("rwkv6", "f32", 32, 32, 32), ("gdn", "bf16", 64, 128, 8),
                                             ("kda", "f32", 128, 32, 3), ("rwkv6", "bf16", 32, 128, 16)])
def test_workspace_size_and_layout(op, dtype, d, dv, C):
    Bsz, H = 3, 5
    cfg = dl.make_config(op, dtype, Bsz, H, d, dv, C)
    n = Bsz * H * C
    isz = 2 if dtype == "bf16" else 4
    xsz = isz if op == "rwkv6" else 4
    gw = 1 if op == "gdn" else d
    x = _round(n * dv * xsz)
    k = _round(n * d * isz)
    g = _round(n * gw * 4)
    slots = _round(Bsz * 4) + _round(Bsz)  # per-slot log origin and active flag
    assert dl.dl_workspace_bytes(cfg) == x + k + g + slots
    assert dl.dl_workspace_layout(cfg) == (0, x, x + k)


@pytest.mark.parametrize("kw,code", [
    (dict(op=7), B.DL_ERR_ARG), (dict(in_dtype=5), B.DL_ERR_ARG),
    (dict(B=0), B.DL_ERR_SHAPE), (dict(H=-1), B.DL_ERR_SHAPE),
    (dict(C=0), B.DL_ERR_SHAPE), (dict(C=33), B.DL_ERR_SHAPE),
    (dict(dk=128, dv=48), B.DL_ERR_UNSUPPORTED), (dict(dk=96, dv=96), B.DL_ERR_UNSUPPORTED),
    (dict(dk=16, dv=64), B.DL_ERR_UNSUPPORTED),
    (dict(B=(1 << 22) + 1, H=2, dk=32, dv=32), B.DL_ERR_SHAPE), (dict(B=1 << 30, H=1 << 30), B.DL_ERR_SHAPE),
])
def test_invalid_configs(kw, code):
    """Every bad config fails at size query and at init, with the status and a reason."""
    base = dict(op=0, in_dtype=1, B=2, H=2, dk=64, dv=64, C=4)
    base.update(kw)
    cfg = B.Config(**base)
    assert dl.dl_workspace_bytes(cfg) == 0
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_state_init(cfg, FAKE, FAKE, 1 << 30)
    assert ei.value.status == code
    assert dl.dl_last_error() != ""


def test_state_init_validation_and_bookkeeping():
    cfg = dl.make_config("gdn", "bf16", 2, 4, 64, 64, 4)
    need = dl.dl_workspace_bytes(cfg)
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_state_init(cfg, 0, FAKE, need)
    assert ei.value.status == B.DL_ERR_ARG
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_state_init(cfg, FAKE + 4, FAKE, need)
    assert ei.value.status == B.DL_ERR_ARG
    with pytest.raises(dl.DeltaLogError) as ei:
        dl.dl_state_init(cfg, FAKE, FAKE, need - 1)
    assert ei.value.status == B.DL_ERR_WORKSPACE
    lib = B.load_library()
    assert lib.dl_state_init(None, ctypes.byref(cfg), FAKE, WS, need) == B.DL_ERR_ARG
    with pytest.raises(dl.DeltaLogError) as ei:  # the workspace starts inside the base
        dl.dl_state_init(cfg, FAKE, FAKE + 0x1000, need)
    assert ei.value.status == B.DL_ERR_ARG
    h = dl.dl_state_init(cfg, FAKE, WS, need)
    try:
        assert dl.dl_log_length(h) == 0
        dl.dl_merge(h)  # L == 0: a no-op, nothing is launched
        assert dl.dl_log_length(h) == 0
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_materialize(h, FAKE)  # dst is the base
        assert ei.value.status == B.DL_ERR_ARG
        with pytest.raises(dl.DeltaLogError):
            dl.dl_materialize(h, 0)
        with pytest.raises(dl.DeltaLogError):
            dl.dl_materialize(h, DST + 8)
    finally:
        dl.dl_state_destroy(h)
    assert dl.dl_log_length(None) == -1
    dl.dl_state_destroy(None)


MB = 0x100000


def _args(**over):
    a = dict(q=IN, k=IN + MB, v=IN + 2 * MB, beta=IN + 3 * MB, decay=IN + 4 * MB, bonus=0, out=IN + 5 * MB)
    a.update(over)
    return B.StepArgs(**a)


@pytest.mark.parametrize("op,over", [
    ("gdn", dict(q=0)), ("gdn", dict(out=0)), ("gdn", dict(decay=0)), ("gdn", dict(beta=0)),
    ("gdn", dict(bonus=IN + 6 * MB)), ("kda", dict(beta=0)),
    ("rwkv6", dict()),  # beta given, bonus missing
    ("rwkv6", dict(beta=0)),  # bonus missing
    ("gdn", dict(k=IN + MB + 1)), ("gdn", dict(out=IN + 5 * MB + 2)), ("gdn", dict(beta=IN + 3 * MB + 2)),
    # q and k are read four channels at a time, per-channel decays and the bonus as float4
    ("gdn", dict(q=IN + 2)), ("kda", dict(k=IN + MB + 4)), ("gdn", dict(v=IN + 2 * MB + 1)),
    ("kda", dict(decay=IN + 4 * MB + 4)), ("rwkv6", dict(beta=0, bonus=IN + 6 * MB + 8)),
    # aliasing: the output over an input, an input or the output over the base or the log
    ("gdn", dict(out=IN + 2 * MB + 0x100)), ("kda", dict(out=IN + 4 * MB)), ("gdn", dict(out=FAKE + 0x4000)),
    ("gdn", dict(out=WS + 0x100)), ("gdn", dict(q=FAKE)), ("kda", dict(decay=WS + 0x1000)),
    ("rwkv6", dict(beta=0, bonus=IN + 5 * MB + 0x10)),
])
def test_decode_step_rejects_bad_args_without_state_change(op, over):
    cfg = dl.make_config(op, "bf16", 2, 4, 64, 64, 4)
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_decode_step(h, _args(**over))
        assert ei.value.status == B.DL_ERR_ARG
        assert dl.dl_log_length(h) == 0
        with pytest.raises(dl.DeltaLogError):
            dl.dl_eager_step(cfg, FAKE, _args(**over))
    finally:
        dl.dl_state_destroy(h)
    lib = B.load_library()
    assert lib.dl_decode_step(None, ctypes.byref(_args()), None) == B.DL_ERR_ARG


def test_eager_state_must_not_alias_the_token():
    cfg = dl.make_config("gdn", "bf16", 2, 4, 64, 64, 1)
    for over in (dict(out=FAKE + 0x1000), dict(q=FAKE), dict(v=FAKE + 0x800)):
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_eager_step(cfg, FAKE, _args(**over))
        assert ei.value.status == B.DL_ERR_ARG
        assert "state" in dl.dl_last_error()


def test_materialize_dst_must_not_overlap_what_the_handle_holds():
    cfg = dl.make_config("kda", "bf16", 2, 4, 64, 64, 4)
    lib = B.load_library()
    state_bytes = 8 * 64 * 64 * 4
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        assert lib.dl_set_split_replay(h, PREP, dl.dl_prep_bytes(cfg)) == B.DL_OK
        # partial overlaps with the base (from either side), the workspace, the prep records
        for dst in (FAKE + 0x100, FAKE - state_bytes + 0x100, WS - 0x1000, WS + 0x2000, PREP - 0x100):
            assert lib.dl_materialize(h, dst, None) == B.DL_ERR_ARG, hex(dst)
            assert "dst overlaps" in dl.dl_last_error()
        blk = 4 * 64 * 64 * 4
        for dst in (FAKE + 0x100, WS, PREP + 0x100):
            assert lib.dl_materialize_slot(h, 1, dst, None) == B.DL_ERR_ARG, hex(dst)
        # prep over the base or the workspace is refused too
        assert lib.dl_set_split_replay(h, FAKE + 0x400, dl.dl_prep_bytes(cfg)) == B.DL_ERR_ARG
        assert lib.dl_set_split_replay(h, WS + 0x400, dl.dl_prep_bytes(cfg)) == B.DL_ERR_ARG
        assert blk  # the slot's block is part of the base
    finally:
        dl.dl_state_destroy(h)


def test_decode_tokens_validates_before_launching():
    cfg = dl.make_config("kda", "bf16", 2, 4, 64, 64, 4)
    lib = B.load_library()
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        for K in (0, 9):
            arr = (B.StepArgs * max(K, 1))(*([_args()] * max(K, 1)))
            assert lib.dl_decode_tokens(h, arr, K, None) == B.DL_ERR_SHAPE
        assert lib.dl_decode_tokens(h, None, 2, None) == B.DL_ERR_ARG
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_decode_tokens(h, [_args(), _args(), _args(k=0)])  # the third token is bad
        assert ei.value.status == B.DL_ERR_ARG
        assert dl.dl_log_length(h) == 0
    finally:
        dl.dl_state_destroy(h)
    # tokens of one call: no output over another token's input or output
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        t0 = _args()
        t1 = _args(q=IN + 8 * MB, k=IN + 9 * MB, v=IN + 10 * MB, beta=IN + 11 * MB, decay=IN + 12 * MB,
                   out=IN + 13 * MB)
        for bad in (_args(**{**{f: getattr(t1, f) for f in ("q", "k", "v", "beta", "decay")}, "out": IN + 5 * MB}),
                    _args(**{**{f: getattr(t1, f) for f in ("q", "k", "v", "beta", "decay")}, "out": IN + MB})):
            with pytest.raises(dl.DeltaLogError) as ei:
                dl.dl_decode_tokens(h, [t0, bad])
            assert ei.value.status == B.DL_ERR_ARG
            assert "another token" in dl.dl_last_error() or "overlapping outputs" in dl.dl_last_error()
        assert dl.dl_log_length(h) == 0
    finally:
        dl.dl_state_destroy(h)
    # RWKV6: one bonus for all tokens of a call
    cfg = dl.make_config("rwkv6", "bf16", 2, 4, 64, 64, 4)
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        a0 = _args(beta=0, bonus=IN + 6 * MB)
        a1 = _args(q=IN + 8 * MB, k=IN + 9 * MB, v=IN + 10 * MB, beta=0, decay=IN + 12 * MB, out=IN + 13 * MB,
                   bonus=IN + 7 * MB)
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_decode_tokens(h, [a0, a1])
        assert ei.value.status == B.DL_ERR_ARG
        assert "bonus" in dl.dl_last_error()
        assert dl.dl_log_length(h) == 0
    finally:
        dl.dl_state_destroy(h)


def test_slot_calls_validate_on_the_host():
    cfg = dl.make_config("gdn", "bf16", 2, 4, 64, 64, 4)
    lib = B.load_library()
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        # a lockstep handle has no slots
        with pytest.raises(dl.DeltaLogError):
            dl.dl_slot_activate(h, 0)
        with pytest.raises(dl.DeltaLogError):
            dl.dl_slot_deactivate(h, 0)
        assert dl.dl_slot_log_length(h, 0) == -1
    finally:
        dl.dl_state_destroy(h)
    # init_slots validates before enqueueing anything
    with pytest.raises(dl.DeltaLogError):
        dl.dl_state_init_slots(cfg, FAKE, FAKE, 16)
    with pytest.raises(dl.DeltaLogError):
        dl.dl_state_init_slots(B.Config(0, 1, 0, 4, 64, 64, 4), FAKE, FAKE, 1 << 20)
    assert lib.dl_slot_log_length(None, 0) == -1


def test_per_slot_fold_calls_validate_on_the_host():
    cfg = dl.make_config("gdn", "bf16", 2, 4, 64, 64, 4)
    lib = B.load_library()
    dst = DST
    assert lib.dl_materialize_slot(None, 0, dst, None) == B.DL_ERR_ARG
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        for slot in (-1, 2):
            assert lib.dl_materialize_slot(h, slot, dst, None) == B.DL_ERR_ARG
        assert lib.dl_materialize_slot(h, 0, None, None) == B.DL_ERR_ARG
        assert lib.dl_materialize_slot(h, 0, dst + 8, None) == B.DL_ERR_ARG  # misaligned
        blk = 4 * 64 * 64 * 4  # one slot's [H, dk, dv] fp32
        assert lib.dl_materialize_slot(h, 1, FAKE + blk + 256, None) == B.DL_ERR_ARG  # inside slot 1's base
        assert lib.dl_slot_merge(h, 0, None) == B.DL_ERR_ARG  # a lockstep handle has no per-slot logs
    finally:
        dl.dl_state_destroy(h)
    assert lib.dl_slot_merge(None, 0, None) == B.DL_ERR_ARG


def test_prep_bytes():
    # N records of 2*dk + 2*M + 4 floats, M the smallest of 8, 16, 32 not below C
    assert dl.dl_prep_bytes(dl.make_config("gdn", "bf16", 2, 4, 64, 64, 4)) == 8 * (128 + 16 + 4) * 4
    assert dl.dl_prep_bytes(dl.make_config("kda", "bf16", 2, 4, 64, 64, 13)) == 8 * (128 + 32 + 4) * 4
    assert dl.dl_prep_bytes(dl.make_config("kda", "bf16", 2, 4, 64, 64, 17)) == 8 * (128 + 64 + 4) * 4
    assert dl.dl_prep_bytes(dl.make_config("rwkv6", "f32", 128, 32, 64, 64, 8)) == 4096 * (128 + 16 + 4) * 4
    assert dl.dl_prep_bytes(B.Config(0, 1, 2, 4, 48, 48, 4)) == 0
    # the record holds the scaled key and query: its width is dk, whatever dv is
    assert dl.dl_prep_bytes(dl.make_config("gdn", "bf16", 2, 4, 128, 32, 8)) == 8 * (256 + 16 + 4) * 4
    assert dl.dl_prep_bytes(dl.make_config("gdn", "bf16", 2, 4, 32, 128, 8)) == 8 * (64 + 16 + 4) * 4


def test_split_replay_and_graph_validate_on_the_host():
    cfg = dl.make_config("gdn", "bf16", 2, 4, 64, 64, 4)
    lib = B.load_library()
    need = dl.dl_prep_bytes(cfg)
    assert lib.dl_set_split_replay(None, PREP, need) == B.DL_ERR_ARG
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        assert lib.dl_set_split_replay(h, PREP + 8, need) == B.DL_ERR_ARG  # misaligned
        assert lib.dl_set_split_replay(h, PREP, need - 4) == B.DL_ERR_WORKSPACE
        assert lib.dl_set_split_replay(h, PREP, need) == B.DL_OK
        # with the prep records set, a token whose output lands in them is refused
        with pytest.raises(dl.DeltaLogError) as ei:
            dl.dl_decode_step(h, _args(out=PREP + 0x100))
        assert "prep" in dl.dl_last_error()
        assert lib.dl_set_split_replay(h, None, 0) == B.DL_OK  # back to the fused form
        g = ctypes.c_void_p()
        arr = (B.StepArgs * 4)(*([_args()] * 4))
        assert lib.dl_graph_capture_cycle(None, h, arr) == B.DL_ERR_ARG
        assert lib.dl_graph_capture_cycle(ctypes.byref(g), None, arr) == B.DL_ERR_ARG
        assert lib.dl_graph_capture_cycle(ctypes.byref(g), h, None) == B.DL_ERR_ARG
        bad = (B.StepArgs * 4)(_args(), _args(), _args(), _args(q=0))  # the last token is bad
        assert lib.dl_graph_capture_cycle(ctypes.byref(g), h, bad) == B.DL_ERR_ARG
        assert g.value is None
        assert dl.dl_log_length(h) == 0
    finally:
        dl.dl_state_destroy(h)
    assert lib.dl_graph_launch(None, None) == B.DL_ERR_ARG
    lib.dl_graph_destroy(None)


def test_eager_step_rejects_bad_state():
    cfg = dl.make_config("gdn", "bf16", 2, 4, 64, 64, 1)
    with pytest.raises(dl.DeltaLogError):
        dl.dl_eager_step(cfg, 0, _args())
    with pytest.raises(dl.DeltaLogError):
        dl.dl_eager_step(cfg, FAKE + 4, _args())


def test_library_is_built_for_gfx950():
    with open(B.LIB_PATH, "rb") as f:
        blob = f.read()
    assert b"gfx950" in blob


def test_largest_head_count_is_accepted():
    cfg = B.Config(op=0, in_dtype=1, B=1 << 21, H=4, dk=32, dv=32, C=32)
    assert B.DL_MAX_HEADS == 1 << 23
    # X (fp32) and K (bf16) for 32 entries of width 32 per head, plus the decays
    assert dl.dl_workspace_bytes(cfg) > (1 << 23) * 32 * 32 * (4 + 2)


def test_probe_validates_on_the_host():
    lib = B.load_library()
    sink = FAKE + 0x50000000
    assert lib.dl_probe_stream(3, FAKE, 1, 1, 64, 64, sink, None) == -1          # bad mode
    assert lib.dl_probe_stream(-1, FAKE, 1, 1, 64, 64, sink, None) == -1         # bad mode
    assert lib.dl_probe_stream(0, FAKE + 8, 1, 1, 64, 64, sink, None) == -1      # misaligned state
    assert lib.dl_probe_stream(0, FAKE, 1, 1, 64, 64, 0, None) == -1             # no sink
    assert lib.dl_probe_stream(1, FAKE, 0, 1, 64, 64, sink, None) == -2          # empty batch
    assert lib.dl_probe_stream(1, FAKE, 1 << 22, 4, 64, 64, sink, None) == -2    # too many heads
    assert lib.dl_probe_stream(0, FAKE, 1, 1, 64, 48, sink, None) == -3          # width not built
    assert "32, 64 or 128" in lib.dl_probe_last_error().decode()


def test_noalloc_step_validates_on_the_host():
    lib = B.load_library()
    assert lib.dl_decode_step_noalloc(None, ctypes.byref(_args()), None) == B.DL_ERR_ARG
    # a configuration whose prep records exceed the static scratch is refused before anything runs
    big = dl.make_config("gdn", "bf16", 2048, 4, 128, 128, 8)  # 8192 heads x 1104 B > 8 MiB
    assert dl.dl_prep_bytes(big) > B.DL_NOALLOC_PREP_BYTES
    h = dl.dl_state_init(big, FAKE + (1 << 36), FAKE + (1 << 37), dl.dl_workspace_bytes(big))
    try:
        assert lib.dl_decode_step_noalloc(h, ctypes.byref(_args()), None) == B.DL_ERR_WORKSPACE
        assert "DL_NOALLOC_PREP_BYTES" in dl.dl_last_error()
        assert dl.dl_log_length(h) == 0
    finally:
        dl.dl_state_destroy(h)
    cfg = dl.make_config("kda", "bf16", 2, 4, 64, 64, 4)
    h = dl.dl_state_init(cfg, FAKE, WS, dl.dl_workspace_bytes(cfg))
    try:
        assert lib.dl_decode_step_noalloc(h, ctypes.byref(_args(k=0)), None) == B.DL_ERR_ARG
        assert lib.dl_decode_step_noalloc(h, ctypes.byref(_args(out=WS + 0x100)), None) == B.DL_ERR_ARG
        assert dl.dl_log_length(h) == 0
    finally:
        dl.dl_state_destroy(h)
