"""ctypes binding of ``libdeltalog.so`` -- argument marshalling only.

Every function here has the name and meaning of the C entry point declared
in ``include/deltalog.h``; device buffers are passed as integer addresses and
streams as integer ``hipStream_t`` handles.  Errors come back as
``DeltaLogError`` carrying the status code and the library's message.  The
library is loaded on first use and must have been built
(``python -m recurrent_state_updates_amd.build``); there is no fallback path.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdeltalog.so")

DL_GDN, DL_KDA, DL_RWKV6 = 0, 1, 2
DL_F32, DL_BF16 = 0, 1
DL_OK = 0
DL_ERR_ARG, DL_ERR_SHAPE, DL_ERR_UNSUPPORTED, DL_ERR_HIP, DL_ERR_WORKSPACE = -1, -2, -3, -4, -5
DL_MAX_CAPACITY = 32
DL_MAX_TOKENS = 8
DL_MAX_HEADS = 1 << 23
DL_NOALLOC_PREP_BYTES = 8 << 20

OP_CODES = {"gdn": DL_GDN, "kda": DL_KDA, "rwkv6": DL_RWKV6}
DTYPE_CODES = {"f32": DL_F32, "bf16": DL_BF16}


class DeltaLogError(RuntimeError):
    """A non-zero dl_status from the library."""

    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


class Config(ctypes.Structure):
    """dl_config."""
    _fields_ = [("op", ctypes.c_int), ("in_dtype", ctypes.c_int), ("B", ctypes.c_int),
                ("H", ctypes.c_int), ("dk", ctypes.c_int), ("dv", ctypes.c_int), ("C", ctypes.c_int)]


class StepArgs(ctypes.Structure):
    """dl_step_args; every field is a device address (0 = NULL)."""
    _fields_ = [("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("beta", ctypes.c_void_p), ("decay", ctypes.c_void_p), ("bonus", ctypes.c_void_p),
                ("out", ctypes.c_void_p)]


_lib = None


def library_path():
    return LIB_PATH


def load_library():
    """Load libdeltalog.so (once); raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "'python -m recurrent_state_updates_amd.build' (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, cp, i, sz = ctypes.c_void_p, ctypes.POINTER(Config), ctypes.c_int, ctypes.c_size_t
    ap = ctypes.POINTER(StepArgs)
    sigs = {
        "dl_workspace_bytes": (sz, [cp]),
        "dl_workspace_layout": (i, [cp, ctypes.POINTER(sz)]),
        "dl_state_init": (i, [ctypes.POINTER(vp), cp, vp, vp, sz]),
        "dl_decode_step": (i, [vp, ap, vp]),
        "dl_decode_step_noalloc": (i, [vp, ap, vp]),
        "dl_decode_tokens": (i, [vp, ap, i, vp]),
        "dl_merge": (i, [vp, vp]),
        "dl_materialize": (i, [vp, vp, vp]),
        "dl_log_length": (i, [vp]),
        "dl_eager_step": (i, [cp, vp, ap, vp]),
        "dl_state_destroy": (None, [vp]),
        "dl_state_init_slots": (i, [ctypes.POINTER(vp), cp, vp, vp, sz, vp]),
        "dl_slot_activate": (i, [vp, i, vp]),
        "dl_slot_deactivate": (i, [vp, i, vp]),
        "dl_slot_log_length": (i, [vp, i]),
        "dl_materialize_slot": (i, [vp, i, vp, vp]),
        "dl_slot_merge": (i, [vp, i, vp]),
        "dl_predict_token_us": (ctypes.c_double, [cp, ctypes.c_double, ctypes.c_double]),
        "dl_choose_capacity": (i, [cp, i, ctypes.c_double, ctypes.c_double]),
        "dl_predict_token_us_bounds": (ctypes.c_double, [cp, ctypes.POINTER(ctypes.c_double),
                                                         ctypes.POINTER(ctypes.c_double)]),
        "dl_choose_capacity_bounds": (i, [cp, i, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
        "dl_prep_bytes": (sz, [cp]),
        "dl_set_split_replay": (i, [vp, vp, sz]),
        "dl_graph_capture_cycle": (i, [ctypes.POINTER(vp), vp, ap]),
        "dl_graph_launch": (i, [vp, vp]),
        "dl_graph_destroy": (None, [vp]),
        "dl_status_string": (ctypes.c_char_p, [i]),
        "dl_last_error": (ctypes.c_char_p, []),
        # measurement kernels (include/deltalog_probe.h)
        "dl_probe_stream": (i, [i, vp, i, i, i, i, vp, vp]),
        "dl_probe_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != DL_OK:
        lib = load_library()
        msg = lib.dl_last_error().decode() or lib.dl_status_string(status).decode()
        raise DeltaLogError(status, msg)


DL_PROBE_READ, DL_PROBE_COPY, DL_PROBE_WRITE = 0, 1, 2


def dl_probe_last_error():
    return load_library().dl_probe_last_error().decode()


def dl_probe_stream(mode, state, B, H, dk, dv, sink, stream=None):
    """One launch of a stream-ceiling probe (include/deltalog_probe.h)."""
    lib = load_library()
    st = lib.dl_probe_stream(mode, state, B, H, dk, dv, sink, stream)
    if st != 0:
        raise DeltaLogError(st, lib.dl_probe_last_error().decode())


def make_config(op, in_dtype, B, H, dk, dv, C=1):
    """Build a Config from names ('gdn'|'kda'|'rwkv6', 'f32'|'bf16') or codes."""
    return Config(OP_CODES.get(op, op), DTYPE_CODES.get(in_dtype, in_dtype), B, H, dk, dv, C)


def dl_workspace_bytes(cfg):
    return int(load_library().dl_workspace_bytes(ctypes.byref(cfg)))


def dl_workspace_layout(cfg):
    off = (ctypes.c_size_t * 3)()
    _check(load_library().dl_workspace_layout(ctypes.byref(cfg), off))
    return tuple(int(x) for x in off)


def dl_state_init(cfg, base, workspace, workspace_bytes):
    """Returns the opaque handle (an integer)."""
    h = ctypes.c_void_p()
    _check(load_library().dl_state_init(ctypes.byref(h), ctypes.byref(cfg), base, workspace,
                                        workspace_bytes))
    return h.value


def dl_state_init_slots(cfg, base, workspace, workspace_bytes, stream=0):
    """Per-slot handle, every slot inactive; returns the handle (an integer)."""
    h = ctypes.c_void_p()
    _check(load_library().dl_state_init_slots(ctypes.byref(h), ctypes.byref(cfg), base, workspace,
                                              workspace_bytes, stream))
    return h.value


def dl_slot_activate(handle, slot, stream=0):
    _check(load_library().dl_slot_activate(handle, slot, stream))


def dl_slot_deactivate(handle, slot, stream=0):
    _check(load_library().dl_slot_deactivate(handle, slot, stream))


def dl_slot_log_length(handle, slot):
    return int(load_library().dl_slot_log_length(handle, slot))


def dl_materialize_slot(handle, slot, dst, stream=0):
    _check(load_library().dl_materialize_slot(handle, slot, dst, stream))


def dl_slot_merge(handle, slot, stream=0):
    _check(load_library().dl_slot_merge(handle, slot, stream))


def dl_decode_step(handle, args, stream=0):
    _check(load_library().dl_decode_step(handle, ctypes.byref(args), stream))


def dl_decode_step_noalloc(handle, args, stream=0):
    _check(load_library().dl_decode_step_noalloc(handle, ctypes.byref(args), stream))


def dl_decode_tokens(handle, args_list, stream=0):
    """args_list: a sequence of StepArgs, the tokens in order."""
    arr = (StepArgs * len(args_list))(*args_list)
    _check(load_library().dl_decode_tokens(handle, arr, len(args_list), stream))


def dl_merge(handle, stream=0):
    _check(load_library().dl_merge(handle, stream))


def dl_materialize(handle, dst, stream=0):
    _check(load_library().dl_materialize(handle, dst, stream))


def dl_log_length(handle):
    return int(load_library().dl_log_length(handle))


def dl_eager_step(cfg, state, args, stream=0):
    _check(load_library().dl_eager_step(ctypes.byref(cfg), state, ctypes.byref(args), stream))


def dl_predict_token_us(cfg, read_gbps=0.0, copy_gbps=0.0):
    us = float(load_library().dl_predict_token_us(ctypes.byref(cfg), read_gbps, copy_gbps))
    if us < 0:
        raise DeltaLogError(DL_ERR_ARG, dl_last_error() or "invalid config")
    return us


def dl_choose_capacity(cfg, max_c=DL_MAX_CAPACITY, read_gbps=0.0, copy_gbps=0.0):
    c = int(load_library().dl_choose_capacity(ctypes.byref(cfg), max_c, read_gbps, copy_gbps))
    if c < 0:
        _check(c)
    return c


def _three(rates):
    r = [float(x) for x in rates]
    if len(r) != 3:
        raise ValueError("three rates are needed: the kernels built for 8, 16 and 32 log entries")
    return (ctypes.c_double * 3)(*r)


def dl_predict_token_us_bounds(cfg, read_gbps, copy_gbps):
    us = float(load_library().dl_predict_token_us_bounds(ctypes.byref(cfg), _three(read_gbps), _three(copy_gbps)))
    if us < 0:
        raise DeltaLogError(DL_ERR_ARG, dl_last_error() or "invalid config")
    return us


def dl_choose_capacity_bounds(cfg, read_gbps, copy_gbps, max_c=DL_MAX_CAPACITY):
    c = int(load_library().dl_choose_capacity_bounds(ctypes.byref(cfg), max_c, _three(read_gbps),
                                                     _three(copy_gbps)))
    if c < 0:
        _check(c)
    return c


def dl_prep_bytes(cfg):
    return int(load_library().dl_prep_bytes(ctypes.byref(cfg)))


def dl_set_split_replay(handle, prep, prep_bytes):
    """prep: device address of the record buffer, or 0 for the fused preparation."""
    _check(load_library().dl_set_split_replay(handle, prep, prep_bytes))


def dl_graph_capture_cycle(handle, args_list):
    """Record one merge cycle (len(args_list) == C tokens); returns the graph (an integer)."""
    arr = (StepArgs * len(args_list))(*args_list)
    g = ctypes.c_void_p()
    _check(load_library().dl_graph_capture_cycle(ctypes.byref(g), handle, arr))
    return g.value


def dl_graph_launch(graph, stream=0):
    _check(load_library().dl_graph_launch(graph, stream))


def dl_graph_destroy(graph):
    load_library().dl_graph_destroy(graph)


def dl_state_destroy(handle):
    load_library().dl_state_destroy(handle)


def dl_status_string(status):
    return load_library().dl_status_string(status).decode()


def dl_last_error():
    return load_library().dl_last_error().decode()
