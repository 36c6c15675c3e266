"""ctypes declarations for libseqdecode.so (argument marshalling only)."""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libseqdecode.so")

P = ctypes.c_void_p
i32, i64, f32, f64, sz = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_size_t

# Every function declared in include/seqdecode.h, with its ctypes signature.
SIGNATURES = {
    "sd_status_string": ([i32], ctypes.c_char_p),
    "sd_abi_version": ([], i32),
    "sd_quantize_q8_act": ([P, i64, i32, i64, P, P, P], i32),
    "sd_qgemv_q8_0_batch": ([P, i64, i64, P, P, i32, P, P, i64, P], i32),
    "sd_qgemv_q8_0_batch_path": ([P, i64, i64, P, P, i32, P, P, i64, i32, P], i32),
    "sd_rope_posvec": ([P, i32, i32, i32, i64, i64, P, f64, i32, P], i32),
    "sd_kv_append_f16": ([P, P, i64, P, i32, i32, i32, P], i32),
    "sd_kv_append_q8_0": ([P, P, i64, P, i32, i32, i32, P], i32),
    "sd_decode_attn_workspace_bytes": ([P, i32, i32, i32], sz),
    "sd_decode_attn_multiseq": ([P, i64, P, i32, i32, i32, i32, f32, P, P, sz, P], i32),
    "sd_decode_attn_multiseq_noalloc": ([P, i64, P, i32, i32, i32, i32, f32, P, P], i32),
    "sd_decode_attn_verify_workspace_bytes": ([P, P, i32, i32, i32], sz),
    "sd_decode_attn_verify": ([P, i64, P, P, i32, i32, i32, i32, f32, P, P, sz, P], i32),
    "sd_rmsnorm_q8": ([P, i64, i32, i64, P, f32, P, P, P, P], i32),
    "sd_swiglu_q8": ([P, i64, i32, i64, P, P, P, P], i32),
    "sd_qgemv_q8_0_swiglu_q8": ([P, i64, i64, P, P, i32, P, P, P], i32),
    "sd_embed_f16": ([P, i64, i64, P, i32, P, P], i32),
    "sd_hbm_stream_read": ([P, sz, P, P], i32),
    "sd_argmax_workspace_bytes": ([i32, i64], sz),
    "sd_argmax_rows": ([P, i64, i32, i64, P, P, sz, P], i32),
    "sd_decode_step_workspace_bytes": ([P, i32, i32], sz),
    "sd_decode_step": ([P, P, P], i32),
}


class SeqView(ctypes.Structure):
    _fields_ = [("k", P), ("v", P), ("ctx_len", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("ld_tok", ctypes.c_int64), ("ld_head", ctypes.c_int64),
                ("window", ctypes.c_int32), ("ring", ctypes.c_int32),
                ("block_table", P), ("block_size", ctypes.c_int32), ("kv_type", ctypes.c_int32),
                ("k_q8", P), ("v_q8", P), ("k_d", P), ("v_d", P)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_qkv", P), ("w_o", P), ("w_gate_up", P), ("w_down", P),
                ("attn_norm", P), ("ffn_norm", P)]


class Model(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32), ("vocab", ctypes.c_int32),
                ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double),
                ("tok_embd", P), ("out_norm", P), ("w_lm_head", P), ("layers", P),
                ("n_rot", ctypes.c_int32), ("window", ctypes.c_int32)]


class StepSeq(ctypes.Structure):
    _fields_ = [("k_cache", P), ("v_cache", P), ("capacity", ctypes.c_int32),
                ("pos", ctypes.c_int32), ("n_new", ctypes.c_int32), ("ring", ctypes.c_int32),
                ("block_table", P), ("block_size", ctypes.c_int32), ("kv_type", ctypes.c_int32),
                ("k_q8", P), ("v_q8", P), ("k_d", P), ("v_d", P)]


class StepIO(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("seqs", P), ("tokens", P), ("positions", P),
                ("logits", P), ("next_tokens", P), ("ws", P), ("ws_bytes", ctypes.c_size_t)]


_lib = None


def load(path: str = LIB_PATH):
    """Loads the HIP library.  Raises if it has not been built: there is no
    other implementation to fall back to."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                " (or python sequence_decode_amd/build.py)")
        L = ctypes.CDLL(path)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib
