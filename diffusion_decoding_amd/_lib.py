"""ctypes binding of libdg.so (argument marshalling only).

Every entry point of ``include/dg.h`` is exposed under the same name; each
raises ``DGError`` on a negative status.  Torch tensors provide device memory
and the current stream; no computation happens here.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_char_p, c_float, c_int32, c_uint8, c_uint32, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdg.so")

DG_DTYPE_FP32, DG_DTYPE_BF16, DG_DTYPE_FP8_E4M3, DG_DTYPE_MXFP4, DG_DTYPE_E8M0 = 0, 1, 2, 3, 4
DG_DTYPE_MXFP4_MXFP8 = 5
DG_STATUS_NONFINITE, DG_STATUS_TOKEN = 1, 2
DG_ERR_INVALID_ARG, DG_ERR_SHAPE, DG_ERR_NUMERIC = -1, -2, -6


class DGError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} returned {status} ({msg})")
        self.status = status


class dg_config(ctypes.Structure):
    _fields_ = [("n_layers", c_int32), ("d_model", c_int32), ("n_heads", c_int32),
                ("head_dim", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("d_expert", c_int32), ("d_shared", c_int32), ("vocab", c_int32),
                ("canvas_len", c_int32), ("max_steps", c_int32), ("rope_theta", c_float),
                ("rms_eps", c_float), ("commit_threshold", c_float), ("act_dtype", c_int32),
                ("expert_dtype", c_int32), ("mask_token", c_int32), ("self_condition", c_int32)]


class dg_layer_weights(ctypes.Structure):
    _fields_ = [("wqkv", c_void_p), ("wo", c_void_p), ("wr", c_void_p), ("w_gu", c_void_p),
                ("w_d", c_void_p), ("s_gu", c_void_p), ("s_d", c_void_p), ("ws_gu", c_void_p),
                ("ws_d", c_void_p), ("ss_gu", c_void_p), ("ss_d", c_void_p)]


class dg_weights(ctypes.Structure):
    _fields_ = [("embed", c_void_p), ("lm_head", c_void_p), ("layers", POINTER(dg_layer_weights))]


class dg_kv(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("batch", c_int32), ("capacity", c_int32),
                ("length", c_int32)]


class dg_canvas(ctypes.Structure):
    _fields_ = [("tokens", c_void_p), ("committed", c_void_p), ("batch", c_int32),
                ("step", c_int32), ("seed", c_uint64), ("block", c_uint32), ("prediction", c_void_p)]


class dg_step_out(ctypes.Structure):
    _fields_ = [("entropy", c_void_p), ("argmax", c_void_p), ("top2_gap", c_void_p),
                ("n_uncommitted", c_void_p), ("logits", c_void_p), ("hidden", c_void_p),
                ("status", c_void_p), ("expert_counts", c_void_p)]


DG_SEG_APPEND, DG_SEG_REFINE = 0, 1


class dg_segment(ctypes.Structure):
    _fields_ = [("kind", c_int32), ("n", c_int32), ("kv", POINTER(dg_kv)), ("tokens", c_void_p),
                ("canvas", POINTER(dg_canvas)), ("entropy", c_void_p), ("argmax", c_void_p),
                ("n_uncommitted", c_void_p), ("hidden", c_void_p)]


_SIGS = {
    "dg_model_create": [POINTER(dg_config), POINTER(dg_weights), c_int32, c_int32, c_int32,
                        POINTER(c_void_p)],
    "dg_model_destroy": [c_void_p],
    "dg_canvas_init": [c_void_p, POINTER(dg_canvas), c_void_p],
    "dg_canvas_prefill": [c_void_p, POINTER(dg_canvas), c_void_p, c_void_p, c_void_p],
    "dg_denoise_step": [c_void_p, POINTER(dg_canvas), POINTER(dg_kv), POINTER(dg_step_out),
                        c_void_p],
    "dg_generate_canvas": [c_void_p, POINTER(dg_canvas), POINTER(dg_kv), POINTER(c_int32),
                           c_void_p],
    "dg_commit_canvas": [c_void_p, c_void_p, c_int32, POINTER(dg_kv), c_void_p],
    "dg_mixed_step": [c_void_p, POINTER(dg_segment), c_int32, c_void_p, c_void_p],
    "dg_pack_experts": [c_void_p, c_void_p, ctypes.c_int64, c_int32, c_int32, c_int32, c_void_p],
    "dg_profile_kernel": [c_void_p, c_int32],
    "dg_profile_read": [c_void_p, POINTER(ctypes.c_double), POINTER(ctypes.c_int64)],
    "dg_test_philox": [c_uint64, c_uint32, c_uint32, c_uint32, c_uint32, c_uint32, c_int32,
                       c_void_p, c_void_p],
    "dg_test_lm_head": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
    "dg_test_fp4_decode": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p],
    "dg_test_mx8_quantize": [c_void_p, c_int32, c_int32, c_int32, ctypes.c_float, c_void_p, c_void_p,
                             c_void_p, c_void_p],
    "dg_test_commit": [c_void_p, POINTER(dg_canvas), c_void_p, c_void_p, c_void_p, c_void_p],
    "dg_test_qkv_rope": [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                         c_void_p, c_void_p],
    "dg_test_attention": [c_void_p, c_int32, c_void_p, POINTER(dg_kv), c_void_p, c_void_p, c_int32,
                          c_void_p, c_void_p],
    "dg_test_router": [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
    "dg_test_shared": [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p],
    "dg_test_moe": [c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                    c_void_p],
    "dg_test_force_routing": [c_void_p, c_void_p],
    "dg_lm_head_confidence_noalloc": [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p],
}
ENTRY_POINTS = ("dg_status_str", "dg_last_error", "dg_version", *_SIGS.keys())

_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libdg.so; raises if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m diffusion_decoding_amd.build`")
    lib = ctypes.CDLL(path)
    lib.dg_status_str.argtypes = [c_int32]
    lib.dg_status_str.restype = c_char_p
    lib.dg_last_error.argtypes = []
    lib.dg_last_error.restype = c_char_p
    lib.dg_version.argtypes = []
    lib.dg_version.restype = c_char_p
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = c_int32
    _lib = lib
    return lib


def _call(name, *args):
    lib = load()
    st = getattr(lib, name)(*args)
    if st != 0:
        raise DGError(name, st, f"{lib.dg_status_str(st).decode()}: {lib.dg_last_error().decode()}")
    return st


def dg_version() -> str:
    return load().dg_version().decode()


def dg_model_create(cfg, weights, max_batch, max_tokens, max_kv):
    h = c_void_p()
    _call("dg_model_create", byref(cfg), byref(weights), max_batch, max_tokens, max_kv, byref(h))
    return h


def dg_model_destroy(handle):
    _call("dg_model_destroy", handle)


def dg_canvas_init(handle, canvas, stream):
    _call("dg_canvas_init", handle, byref(canvas), stream)


def dg_canvas_prefill(handle, canvas, tokens_ptr, mask_ptr, stream):
    _call("dg_canvas_prefill", handle, byref(canvas), tokens_ptr, mask_ptr, stream)


def dg_denoise_step(handle, canvas, kv, out, stream):
    _call("dg_denoise_step", handle, byref(canvas), byref(kv), byref(out) if out else None, stream)


def dg_generate_canvas(handle, canvas, kv, stream) -> int:
    taken = c_int32(0)
    _call("dg_generate_canvas", handle, byref(canvas), byref(kv), byref(taken), stream)
    return taken.value


def dg_commit_canvas(handle, tokens_ptr, n, kv, stream):
    _call("dg_commit_canvas", handle, tokens_ptr, n, byref(kv), stream)


def dg_mixed_step(handle, segs, n_segs, status_ptr, stream):
    _call("dg_mixed_step", handle, segs, n_segs, status_ptr, stream)


def dg_pack_experts(src_ptr, dst_ptr, n_mats, rows, cols, dtype, stream):
    _call("dg_pack_experts", src_ptr, dst_ptr, n_mats, rows, cols, dtype, stream)


DG_PROF = {"none": 0, "attn": 1, "moe_gateup": 2, "moe_down": 3, "lm_head": 4, "qkv": 5,
           "shared": 6, "router": 7, "commit": 8}


def dg_profile_kernel(handle, kernel_id: int):
    _call("dg_profile_kernel", handle, kernel_id)


def dg_profile_read(handle):
    ms, n = ctypes.c_double(0.0), ctypes.c_int64(0)
    _call("dg_profile_read", handle, byref(ms), byref(n))
    return ms.value, n.value


def dg_test_philox(seed, pos0, tag, canvas, block, modulus, n, out_ptr, stream):
    _call("dg_test_philox", seed, pos0, tag, canvas, block, modulus, n, out_ptr, stream)


def dg_test_lm_head(handle, hf_ptr, T, ent_ptr, am_ptr, gap_ptr, stream):
    _call("dg_test_lm_head", handle, hf_ptr, T, ent_ptr, am_ptr, gap_ptr, stream)


def dg_test_commit(handle, canvas, ent_ptr, am_ptr, nunc_ptr, stream):
    _call("dg_test_commit", handle, byref(canvas), ent_ptr, am_ptr, nunc_ptr, stream)


def dg_test_qkv_rope(handle, layer, a_ptr, batch, n, pos0, q_ptr, k_ptr, v_ptr, stream):
    _call("dg_test_qkv_rope", handle, layer, a_ptr, batch, n, pos0, q_ptr, k_ptr, v_ptr, stream)


def dg_test_attention(handle, layer, q_ptr, kv, kc_ptr, vc_ptr, n, out_ptr, stream):
    _call("dg_test_attention", handle, layer, q_ptr, byref(kv), kc_ptr, vc_ptr, n, out_ptr, stream)


def dg_test_router(handle, layer, b_ptr, T, logits_ptr, ids_ptr, w_ptr, stream):
    _call("dg_test_router", handle, layer, b_ptr, T, logits_ptr, ids_ptr, w_ptr, stream)


def dg_test_shared(handle, layer, b_ptr, T, hs_ptr, ys_ptr, stream):
    _call("dg_test_shared", handle, layer, b_ptr, T, hs_ptr, ys_ptr, stream)


def dg_test_moe(handle, layer, b_ptr, T, ids_ptr, h_ptr, y_ptr, pos_ptr, stream):
    _call("dg_test_moe", handle, layer, b_ptr, T, ids_ptr, h_ptr, y_ptr, pos_ptr, stream)


def dg_test_force_routing(handle, ids_ptr):
    _call("dg_test_force_routing", handle, ids_ptr)


def dg_lm_head_confidence_noalloc(handle, hf_ptr, T, ent_ptr, am_ptr, gap_ptr, stream):
    _call("dg_lm_head_confidence_noalloc", handle, hf_ptr, T, ent_ptr, am_ptr, gap_ptr, stream)


def dg_test_fp4_decode(packed_ptr, scales_ptr, n_blocks, out_ptr, stream):
    _call("dg_test_fp4_decode", packed_ptr, scales_ptr, n_blocks, out_ptr, stream)


def dg_test_mx8_quantize(x_ptr, rows, d, norm, eps, y_ptr, codes_ptr, scales_ptr, stream):
    _call("dg_test_mx8_quantize", x_ptr, rows, d, norm, eps, y_ptr, codes_ptr, scales_ptr, stream)
