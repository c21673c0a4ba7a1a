"""ctypes binding of libspec.so (argument marshalling only).

Every compute function here forwards to the C ABI declared in include/spec.h
with the same name; tensors are passed as raw device pointers and the current
torch stream is used unless one is given.  Loading fails loudly if the HIP
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# SPEC_LIB_PATH selects another build of the same library (the host-sanitizer
# test loads an ASan/UBSan build this way)
LIB_PATH = os.environ.get("SPEC_LIB_PATH") or os.path.join(HERE, "libspec.so")

SPEC_F32, SPEC_BF16 = 0, 1
SPEC_MLP_SEQUENTIAL, SPEC_MLP_PARALLEL = 0, 1
STATUS = {0: "SPEC_OK", -1: "SPEC_ERR_INVALID_ARG", -2: "SPEC_ERR_SHAPE", -3: "SPEC_ERR_VOCAB_MISMATCH",
          -4: "SPEC_ERR_PLAN", -5: "SPEC_ERR_CAPACITY", -6: "SPEC_ERR_WORKSPACE", -7: "SPEC_ERR_HIP",
          -8: "SPEC_ERR_UNSUPPORTED"}

# every symbol include/spec.h declares
EXPORTS = ("spec_model_create", "spec_model_destroy", "spec_check_pair", "spec_default_group_plan",
           "spec_workspace_bytes", "spec_draft_group_step", "spec_calibrate_kv", "spec_verify_forward",
           "spec_accept_workspace_bytes", "spec_accept_resample", "spec_status_string", "spec_last_error",
           "spec_version", "spec_profile_enable", "spec_profile_reset", "spec_profile_collect",
           "spec_profile_entry", "spec_draft_attention_cosine", "spec_draft_group_step_noalloc")
SPEC_SCRATCH_BYTES = 32 << 20


class SpecError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status


class ModelDesc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("d_model", C.c_int32), ("n_q_heads", C.c_int32),
                ("n_kv_heads", C.c_int32), ("head_dim", C.c_int32), ("d_ffn", C.c_int32),
                ("vocab", C.c_int32), ("has_qkv_bias", C.c_int32), ("dtype", C.c_int32),
                ("rms_eps", C.c_float), ("rope_theta", C.c_float)]


class Weights(C.Structure):
    _fields_ = [(n, C.c_void_p) for n in ("embed", "attn_norm", "wqkv", "bqkv", "wo", "ffn_norm",
                                          "w_gate_up", "w_down", "final_norm", "lm_head")]


class KV(C.Structure):
    _fields_ = [("k", C.c_void_p), ("v", C.c_void_p), ("capacity", C.c_int32), ("batch", C.c_int32)]


_lib = None


def load() -> C.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m layer_speculative_decoding_amd.build`")
    lib = C.CDLL(LIB_PATH)
    vp, i32, i64, sz, f32, u64 = C.c_void_p, C.c_int, C.c_int64, C.c_size_t, C.c_float, C.c_uint64
    sig = {
        "spec_model_create": (i32, [C.POINTER(ModelDesc), C.POINTER(Weights), C.POINTER(vp)]),
        "spec_model_destroy": (None, [vp]),
        "spec_check_pair": (i32, [vp, vp]),
        "spec_default_group_plan": (i32, [i32, i32, C.POINTER(C.c_int32), i32, C.POINTER(C.c_int)]),
        "spec_workspace_bytes": (sz, [vp, i32, i32, i32]),
        "spec_draft_group_step": (i32, [vp, C.POINTER(KV), C.POINTER(C.c_int32), i32, i32, i32, vp, i32, vp, i32,
                                        f32, u64, vp, i64, vp, i32, vp, sz, vp]),
        "spec_draft_group_step_noalloc": (i32, [vp, C.POINTER(KV), C.POINTER(C.c_int32), i32, i32, i32, vp, i32, vp,
                                                i32, f32, u64, vp, i64, vp, i32, vp]),
        "spec_calibrate_kv": (i32, [vp, C.POINTER(KV), i32, vp, i32, vp, vp, i32, i32, f32, u64, vp, i64, vp, i32, vp,
                                    sz, vp]),
        "spec_verify_forward": (i32, [vp, C.POINTER(KV), i32, vp, vp, i32, i32, vp, vp, sz, vp]),
        "spec_accept_workspace_bytes": (sz, [i32, i32, i32]),
        "spec_accept_resample": (i32, [i32, i32, i32, vp, vp, vp, i32, vp, f32, u64, vp, vp, i32, vp, vp, sz, vp]),
        "spec_status_string": (C.c_char_p, [i32]),
        "spec_last_error": (C.c_char_p, []),
        "spec_version": (C.c_char_p, []),
        "spec_draft_attention_cosine": (i32, [vp, C.POINTER(KV), C.POINTER(C.c_int32), i32, i32, vp, i32, vp, i32,
                                              vp, i32, vp, sz, vp]),
        "spec_profile_enable": (i32, [i32]),
        "spec_profile_reset": (None, []),
        "spec_profile_collect": (i32, []),
        "spec_profile_entry": (i32, [i32, C.c_char_p, i32, C.POINTER(C.c_int64), C.POINTER(C.c_double),
                                     C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def check(status: int):
    if status != 0:
        raise SpecError(status, load().spec_last_error().decode())
