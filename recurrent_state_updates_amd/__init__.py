"""DeltaLog single-token recurrent-state decode for linear attention on MI355X.

GDN, KDA and RWKV6 heads keep a dense fp32 base state plus a bounded log of
compact update factors; most decode steps read the base and append to the
log, every C-th step folds the log into the base (DeltaLog: Deferred
Materialization of Recurrent States for Linear Attention Decoding).  The
work runs in hand-written HIP kernels for gfx950 behind the C ABI of
``include/deltalog.h``; this package is its Python binding.
"""
from ._binding import (  # noqa: F401
    DL_BF16, DL_F32, DL_GDN, DL_KDA, DL_MAX_CAPACITY, DL_MAX_HEADS, DL_MAX_TOKENS, DL_NOALLOC_PREP_BYTES, DL_RWKV6, Config, DeltaLogError, StepArgs,
    dl_choose_capacity, dl_choose_capacity_bounds, dl_decode_step, dl_decode_step_noalloc, dl_decode_tokens, dl_eager_step, dl_graph_capture_cycle,
    dl_graph_destroy, dl_graph_launch, dl_last_error, dl_log_length, dl_materialize, dl_materialize_slot, dl_merge,
    dl_predict_token_us, dl_predict_token_us_bounds, dl_prep_bytes, dl_probe_last_error, dl_probe_stream, DL_PROBE_READ, DL_PROBE_COPY, DL_PROBE_WRITE, dl_set_split_replay, dl_slot_activate, dl_slot_deactivate,
    dl_slot_log_length, dl_slot_merge, dl_state_destroy, dl_state_init, dl_state_init_slots, dl_status_string,
    dl_workspace_bytes, dl_workspace_layout, library_path, load_library, make_config)
from .state import CycleGraph, DeltaLogState, eager_step  # noqa: F401
