"""ctypes declarations of the C ABI in include/pn.h (argument marshalling only)."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpn.so")

PN_OK, PN_EINVAL, PN_ERANGE, PN_EUNSUPPORTED, PN_EHIP = 0, -1, -2, -3, -4
PN_F32, PN_BF16, PN_I8, PN_Q8_0, PN_Q4_0 = 0, 1, 2, 3, 4
(PN_K_EMBED, PN_K_QKV, PN_K_ATTN, PN_K_O, PN_K_GATEUP, PN_K_DOWN, PN_K_LMHEAD, PN_K_ARGMAX,
 PN_K_ROUTER, PN_K_MOE_GATEUP, PN_K_MOE_DOWN, PN_K_MOE_COMBINE, PN_K_COUNT) = range(13)
PN_OPT_ATTN_KEYS_PER_SPLIT = 1
PN_OPT_ATTN_KERNEL = 2
PN_OPT_ATTN_COMBINE = 3
PN_OPT_ATTN_WAVES = 4
PN_OPT_GEMM_PROLOGUE = 5
PN_OPT_WAVES_QKV, PN_OPT_WAVES_O, PN_OPT_WAVES_GATEUP, PN_OPT_WAVES_DOWN, PN_OPT_WAVES_LMHEAD = range(10, 15)

KERNEL_NAMES = ["embed", "qkv", "attn", "o", "gateup", "down", "lmhead", "argmax", "router",
                "moe_gateup", "moe_down", "moe_combine"]

i32, vp, sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t


class pn_config(ctypes.Structure):
    _fields_ = [("n_layer", i32), ("n_embd", i32), ("n_head", i32), ("n_kv_head", i32),
                ("head_dim", i32), ("n_ff", i32), ("n_vocab", i32), ("n_ctx", i32),
                ("n_expert", i32), ("n_expert_used", i32), ("sliding_window", i32),
                ("max_batch", i32), ("rope_theta", ctypes.c_float), ("rms_norm_eps", ctypes.c_float),
                ("w_dtype", i32), ("kv_dtype", i32), ("act_dtype", i32), ("rope_neox", i32),
                ("qkv_bias", i32), ("prefill_chunk", i32)]


class pn_layer_weights(ctypes.Structure):
    _fields_ = [(n, vp) for n in ("attn_norm", "ffn_norm", "wq", "wk", "wv", "wo", "w_gate", "w_up",
                                   "w_down", "w_router", "s_q", "s_k", "s_v", "s_o", "s_gate",
                                   "s_up", "s_down", "b_q", "b_k", "b_v")]


class pn_sampling_params(ctypes.Structure):
    _fields_ = [("temperature", ctypes.c_float), ("repeat_penalty", ctypes.c_float), ("top_k", i32),
                ("top_p", ctypes.c_float)]


class pn_weights(ctypes.Structure):
    _fields_ = [("tok_embd", vp), ("out_norm", vp), ("w_out", vp), ("s_out", vp),
                ("layers", ctypes.POINTER(pn_layer_weights))]


class PNError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (code %d)" % (msg, code))
        self.code = code


_lib = None


def lib():
    """Load libpn.so; fails loudly if the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("HIP library %s is not built; run __graft_entry__.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.POINTER
        sig = {
            "pn_config_default": (None, [P(pn_config)]),
            "pn_config_check": (ctypes.c_int, [P(pn_config)]),
            "pn_model_bytes": (sz, [P(pn_config)]),
            "pn_model_create": (ctypes.c_int, [P(pn_config), P(pn_weights), vp, sz, vp, P(vp)]),
            "pn_model_init": (ctypes.c_int, [P(pn_config), vp, sz, P(vp)]),
            "pn_model_load_globals": (ctypes.c_int, [vp, vp, vp, vp, vp, vp]),
            "pn_model_load_layer": (ctypes.c_int, [vp, i32, P(pn_layer_weights), vp]),
            "pn_model_free": (None, [vp]),
            "pn_state_bytes": (sz, [vp, i32]),
            "pn_state_new": (ctypes.c_int, [vp, i32, vp, sz, vp, P(vp)]),
            "pn_state_reset": (ctypes.c_int, [vp, vp]),
            "pn_state_set_kv": (ctypes.c_int, [vp, i32, i32, i32, vp, vp, vp]),
            "pn_state_set_page_table": (ctypes.c_int, [vp, P(i32), i32, vp]),
            "pn_state_pages": (i32, [vp]),
            "pn_page_size": (i32, []),
            "pn_state_set_pos": (ctypes.c_int, [vp, i32, vp]),
            "pn_pool_bytes": (sz, [vp, i32]),
            "pn_pool_new": (ctypes.c_int, [vp, i32, vp, sz, P(vp)]),
            "pn_pool_free_pages": (i32, [vp]),
            "pn_pool_free": (None, [vp]),
            "pn_state_bytes_pooled": (sz, [vp, i32]),
            "pn_state_new_pooled": (ctypes.c_int, [vp, vp, i32, vp, sz, vp, P(vp)]),
            "pn_state_pos": (i32, [vp]),
            "pn_state_max_ctx": (i32, [vp]),
            "pn_state_check": (ctypes.c_int, [vp, vp, P(i32)]),
            "pn_state_free": (None, [vp]),
            "pn_forward_step": (ctypes.c_int, [vp, vp, vp, vp, vp, vp]),
            "pn_forward_batch": (ctypes.c_int, [vp, P(vp), i32, vp, vp, vp, vp]),
            "pn_sample": (ctypes.c_int, [vp, vp, i32, P(pn_sampling_params), vp, i32, vp, vp, vp]),
            "pn_prefill": (ctypes.c_int, [vp, vp, vp, i32, vp, vp, vp]),
            "pn_model_set_option": (ctypes.c_int, [vp, i32, ctypes.c_int64]),
            "pn_profile_begin": (ctypes.c_int, [vp, i32]),
            "pn_profile_end": (ctypes.c_int, [vp, vp, P(ctypes.c_double), P(ctypes.c_int64)]),
            "pn_profile_replay": (ctypes.c_int, [vp, i32, i32, vp]),
            "pn_sample_noalloc": (ctypes.c_int, [vp, i32, i32, P(pn_sampling_params), vp, i32, vp, vp, vp]),
            "pn_model_route_log": (ctypes.c_int, [vp, vp, i32]),
            "pn_model_trace": (ctypes.c_int, [vp, vp]),
            "pn_stream_read": (ctypes.c_int, [vp, sz, vp, vp]),
            "pn_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


EXPORTS = ["pn_config_default", "pn_config_check", "pn_model_bytes", "pn_model_create",
           "pn_model_init", "pn_model_load_globals", "pn_model_load_layer", "pn_model_free",
           "pn_state_bytes", "pn_state_new", "pn_state_reset", "pn_state_set_kv",
           "pn_state_set_page_table", "pn_state_pages", "pn_page_size", "pn_state_set_pos",
           "pn_state_pos", "pn_state_max_ctx", "pn_state_check", "pn_state_free",
           "pn_pool_bytes", "pn_pool_new", "pn_pool_free_pages", "pn_pool_free", "pn_state_bytes_pooled",
           "pn_state_new_pooled",
           "pn_forward_step", "pn_forward_batch", "pn_prefill", "pn_sample", "pn_sample_noalloc", "pn_model_set_option", "pn_profile_begin",
           "pn_profile_end", "pn_profile_replay", "pn_model_route_log", "pn_model_trace", "pn_stream_read", "pn_last_error"]


def check(rc):
    """Raise PNError with pn_last_error() for a negative return code."""
    if rc != 0:
        raise PNError(rc, lib().pn_last_error().decode())
    return rc


def _fwd(name):
    def f(*args):
        return getattr(lib(), name)(*args)
    f.__name__ = name
    return f


for _n in EXPORTS:
    globals()[_n] = _fwd(_n)
