"""ctypes declarations of the C ABI in include/cb.h.

Loading fails loudly when the library has not been built: there is no
fallback implementation anywhere in this package.
"""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcb.so")

CB_OK, CB_ERR_INVALID, CB_ERR_UNSUPPORTED, CB_ERR_WORKSPACE, CB_ERR_DEVICE, CB_ERR_CAPACITY = 0, -1, -2, -3, -4, -5
CB_F32, CB_BF16 = 0, 1
CB_POLICY_FIFO, CB_POLICY_PREFILL_FIRST = 0, 1
PAGE_SIZE = 16

i32, i64, f32, vp, sz = C.c_int32, C.c_int64, C.c_float, C.c_void_p, C.c_size_t
P_i32 = C.POINTER(C.c_int32)
P_i64 = C.POINTER(C.c_int64)


class BuilderConfig(C.Structure):
    _fields_ = [("max_batch_tokens", i32), ("max_requests_per_batch", i32), ("num_pages", i32),
                ("page_size", i32), ("max_prefill_chunk", i32), ("safety_margin", f32),
                ("page_shuffle_seed", C.c_uint64), ("policy", i32), ("max_partial_prefills", i32),
                ("max_long_partial_prefills", i32), ("long_prefill_threshold", i32),
                ("allow_block_sharing", i32), ("sliding_window", i32)]


class StepDesc(C.Structure):
    _fields_ = [("num_seqs", i32), ("num_decodes", i32), ("num_tokens", i32), ("max_query_len", i32),
                ("max_context_len", i32), ("block_table_stride", i32), ("num_finished", i32),
                ("num_stalled", i32), ("new_pages", i32), ("prefix_hit_tokens", i32),
                ("req_ids", P_i64), ("query_start_loc", P_i32), ("context_lens", P_i32),
                ("q_offsets", P_i32), ("block_tables", P_i32), ("slot_mapping", P_i32),
                ("finished_ids", P_i64), ("stalled_ids", P_i64)]


class BuilderStats(C.Structure):
    _fields_ = [("num_pages", i32), ("free_pages", i32), ("num_waiting", i32), ("num_prefilling", i32),
                ("num_decoding", i32), ("num_finished_pending", i32), ("used_slots", i64),
                ("allocated_slots", i64), ("steps", i64), ("total_stalls", i64),
                ("total_finished", i64), ("fragmentation", C.c_double), ("prefix_hit_tokens", i64),
                ("cached_pages", i32)]


class EngineConfig(C.Structure):
    _fields_ = [("builder", BuilderConfig), ("num_q_heads", i32), ("num_kv_heads", i32), ("head_dim", i32),
                ("dtype", i32), ("scale", f32), ("k_cache", vp), ("v_cache", vp), ("meta_device", vp),
                ("meta_host", vp), ("meta_bytes", sz), ("workspace", vp), ("workspace_bytes", sz)]


class EngineStats(C.Structure):
    _fields_ = [("steps_scheduled", i64), ("steps_attended", i64), ("slot_waits", i64),
                ("graph_captures", i64), ("graph_replays", i64), ("graphs_cached", i64),
                ("cu_split_steps", i64)]


# name -> (restype, argtypes); one line per declaration of include/cb.h
SIGNATURES = {
    "cb_status_string": (C.c_char_p, [C.c_int]),
    "cb_last_error": (C.c_char_p, []),
    "cb_abi_version": (C.c_int, []),
    "cb_profile_events": (C.c_int, [vp, vp]),
    "cb_profile_clock": (C.c_int, [vp]),
    "cb_attention_step_noalloc": (C.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                            i32, i32, f32, i32, i32, vp, vp]),
    "cb_attention_noalloc_scratch_bytes": (sz, []),
    "cb_kv_append": (C.c_int, [vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]),
    "cb_attention_workspace_bytes": (sz, [i32, i32, i32, i32, i32, i32, i32, i32]),
    "cb_attention_step": (C.c_int, [vp, vp, vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32,
                                    i32, i32, f32, i32, i32, vp, vp, sz, vp]),
    "cb_builder_create": (C.c_int, [C.POINTER(BuilderConfig), C.POINTER(vp)]),
    "cb_builder_clone": (C.c_int, [vp, C.POINTER(vp)]),
    "cb_builder_destroy": (None, [vp]),
    "cb_builder_submit": (C.c_int, [vp, i64, i32, i32, i32]),
    "cb_builder_submit_tokens": (C.c_int, [vp, i64, P_i32, i32, i32]),
    "cb_builder_step": (C.c_int, [vp, C.POINTER(StepDesc)]),
    "cb_builder_block_table": (C.c_int, [vp, i64, P_i32, i32, P_i32]),
    "cb_builder_stats_get": (C.c_int, [vp, C.POINTER(BuilderStats)]),
    "cb_builder_slots": (C.c_int, [vp, i64, i32, i32, P_i32]),
    "cb_engine_create": (C.c_int, [C.POINTER(EngineConfig), C.POINTER(vp)]),
    "cb_engine_destroy": (None, [vp]),
    "cb_engine_builder": (vp, [vp]),
    "cb_engine_set_metadata": (C.c_int, [vp, vp, vp, sz]),
    "cb_engine_set_workspace": (C.c_int, [vp, vp, sz]),
    "cb_engine_schedule": (C.c_int, [vp, vp, C.POINTER(StepDesc)]),
    "cb_engine_attend": (C.c_int, [vp, vp, vp, vp, vp, vp]),
    "cb_engine_workspace_bytes": (sz, [vp]),
    "cb_engine_stats_get": (C.c_int, [vp, C.POINTER(EngineStats)]),
    "cb_engine_load_builder": (C.c_int, [vp, vp]),
    "cb_engine_set_graphs": (C.c_int, [vp, i32, i32, i32]),
    "cb_engine_padded_tokens": (i32, [vp]),
    "cb_engine_graph_stats": (C.c_int, [vp, C.POINTER(i64), C.POINTER(i64), C.POINTER(i64)]),
}

_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library {LIB_PATH} is not built; run `python -m chunked_prefill_attention_amd.build`")
        lib = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class CbError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{load().cb_status_string(status).decode()}: {msg}")
        self.status = status


def check(status: int) -> None:
    if status != CB_OK:
        raise CbError(status, load().cb_last_error().decode())
