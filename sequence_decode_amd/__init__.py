"""Python binding of libseqdecode (include/seqdecode.h), one function per entry point.

Argument marshalling only: every operation runs in the library's HIP kernels on
the current torch CUDA stream.  torch provides device memory and streams.  If
the library is missing, every call raises; nothing falls back to another
implementation.
"""
import ctypes

from . import _lib
from ._lib import SeqView

__all__ = [
    "SdError", "load", "abi_version", "quantize_q8_act", "qgemv_q8_0_batch", "rope_posvec",
    "kv_append_f16", "seqview", "decode_attn_workspace_bytes", "decode_attn_multiseq",
    "decode_attn_multiseq_noalloc", "ATTN_SCRATCH_BYTES",
    "decode_attn_verify", "ATTN_MAX_NEW",
    "rmsnorm_q8", "swiglu_q8", "qgemv_q8_0_swiglu_q8", "embed_f16", "argmax_rows", "MAX_TOKENS", "MAX_SEQS",
    "ATTN_CHUNK", "ATTN_SMALL_CHUNK", "ATTN_SMALL_SPAN", "GEMV_AUTO", "GEMV_NARROW", "GEMV_MFMA", "seqview_q8", "seqview_quant", "kv_append_q8_0",
    "KV_F16", "KV_Q8_0", "KV_Q4_0", "KV_Q4_Q8", "KV_Q8_Q4", "kv_type_of",
]

MAX_TOKENS = 16
MAX_SEQS = 4
ATTN_CHUNK = 256
ATTN_SMALL_CHUNK = 64
ATTN_SMALL_SPAN = 2048
ATTN_MAX_NEW = 4
ATTN_SCRATCH_BYTES = 16 << 20
GEMV_AUTO, GEMV_NARROW, GEMV_MFMA = 0, 1, 2
KV_F16, KV_Q8_0, KV_Q4_0, KV_Q4_Q8, KV_Q8_Q4 = 0, 1, 2, 3, 4


def kv_type_of(k_type: str, v_type: str) -> int:
    """The sd_seqview kv_type of quantized K and V types ("q8_0" or "q4_0")."""
    types = {("q8_0", "q8_0"): KV_Q8_0, ("q4_0", "q4_0"): KV_Q4_0, ("q4_0", "q8_0"): KV_Q4_Q8,
             ("q8_0", "q4_0"): KV_Q8_Q4}
    if (k_type, v_type) not in types:
        raise ValueError(f"unknown K/V types {k_type}/{v_type}")
    return types[(k_type, v_type)]


class SdError(RuntimeError):
    def __init__(self, fn, status):
        msg = _lib.load().sd_status_string(status).decode()
        super().__init__(f"{fn}: {msg} ({status})")
        self.status = status


def load():
    return _lib.load()


def _check(fn, status):
    if status != 0:
        raise SdError(fn, status)


def _stream(stream=None):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")


def abi_version() -> int:
    return _lib.load().sd_abi_version()


def quantize_q8_act(x, xq=None, xd=None, stream=None):
    """x [n_tok][K] fp32 -> (xq int8 [n_tok][K], xd fp32 [n_tok][K/32])."""
    import torch
    _need(x, torch.float32, "x")
    n_tok, K = x.shape
    xq = torch.empty((n_tok, K), dtype=torch.int8, device=x.device) if xq is None else xq
    xd = torch.empty((n_tok, K // 32), dtype=torch.float32, device=x.device) if xd is None else xd
    _check("sd_quantize_q8_act", _lib.load().sd_quantize_q8_act(
        _p(x), K, n_tok, K, _p(xq), _p(xd), _stream(stream)))
    return xq, xd


def qgemv_q8_0_batch(w, N, K, xq, xd, residual=None, out=None, stream=None, path=None):
    """q8_0 GEMV for n_tok = xq.shape[0] rows -> y fp32 [n_tok][N].  path=None
    calls sd_qgemv_q8_0_batch; GEMV_AUTO / GEMV_NARROW / GEMV_MFMA call
    sd_qgemv_q8_0_batch_path with that kernel choice."""
    import torch
    _need(w, torch.uint8, "w")
    _need(xq, torch.int8, "xq")
    _need(xd, torch.float32, "xd")
    n_tok = xq.shape[0]
    y = torch.empty((n_tok, N), dtype=torch.float32, device=xq.device) if out is None else out
    if residual is not None:
        _need(residual, torch.float32, "residual")
    if path is None:
        _check("sd_qgemv_q8_0_batch", _lib.load().sd_qgemv_q8_0_batch(
            _p(w), N, K, _p(xq), _p(xd), n_tok, _p(residual), _p(y), y.shape[1], _stream(stream)))
    else:
        _check("sd_qgemv_q8_0_batch_path", _lib.load().sd_qgemv_q8_0_batch_path(
            _p(w), N, K, _p(xq), _p(xd), n_tok, _p(residual), _p(y), y.shape[1], int(path),
            _stream(stream)))
    return y


def rope_posvec(x, pos, theta, n_rot=None, stream=None):
    """In place on x [n_tok][n_heads][head_dim] fp32 with pos int32 [n_tok]."""
    import torch
    _need(x, torch.float32, "x")
    _need(pos, torch.int32, "pos")
    n_tok, n_heads, head_dim = x.shape
    n_rot = head_dim if n_rot is None else n_rot
    _check("sd_rope_posvec", _lib.load().sd_rope_posvec(
        _p(x), n_tok, n_heads, head_dim, n_heads * head_dim, head_dim, _p(pos), float(theta),
        n_rot, _stream(stream)))
    return x


def seqview(k, v, ctx_len, window=0, ring=False, block_table=None, block_size=0):
    """View of one sequence's caches k, v: [capacity][H_kv][D] fp16 (or int16
    bits).  window > 0: tokens attend to their last `window` positions; ring:
    position j lives in row j % capacity; block_table (int32 device tensor, kept
    alive by the caller): k, v are a pool of blocks of block_size rows and
    position j lives in row block_table[j // block_size] * block_size
    + j % block_size."""
    import torch
    cap, H_kv, D = k.shape
    bt = 0
    if block_table is not None:
        _need(block_table, torch.int32, "block_table")
        bt = block_table.data_ptr()
    return SeqView(k.data_ptr(), v.data_ptr(), int(ctx_len), int(cap), H_kv * D, D, int(window),
                   1 if ring else 0, bt, int(block_size), KV_F16)


def seqview_q8(kq, kd, vq, vd, ctx_len, window=0, ring=False, block_table=None, block_size=0):
    """View of one sequence's q8_0 caches: codes kq, vq [capacity][H_kv][D] int8
    and fp16 block scales kd, vd [capacity][H_kv][D/32] (or int16 bits); the
    other arguments as in seqview."""
    return seqview_quant(kq, kd, vq, vd, ctx_len, "q8_0", "q8_0", window, ring, block_table, block_size)


def seqview_quant(kq, kd, vq, vd, ctx_len, k_type="q8_0", v_type="q8_0", window=0, ring=False,
                  block_table=None, block_size=0):
    """View of one sequence's quantized caches, K and V each "q8_0" (codes int8
    [capacity][H_kv][D]) or "q4_0" (nibble pairs uint8 [capacity][H_kv][D/2]),
    with fp16 block scales kd, vd [capacity][H_kv][D/32] (or int16 bits); the
    other arguments as in seqview."""
    import torch
    kv_type = kv_type_of(k_type, v_type)
    cap, H_kv, nsc = kd.shape
    D = 32 * nsc
    for t, n, ty in ((kq, "kq", k_type), (vq, "vq", v_type)):
        _need(t, torch.int8 if ty == "q8_0" else torch.uint8, n)
        if tuple(t.shape) != (cap, H_kv, D if ty == "q8_0" else D // 2):
            raise TypeError(f"{n} has the wrong shape for {ty} codes")
    for t, n in ((kd, "kd"), (vd, "vd")):
        if t.dtype not in (torch.float16, torch.int16):
            raise TypeError(f"{n} must be float16 (or int16 bits)")
        if not t.is_cuda or not t.is_contiguous() or tuple(t.shape) != (cap, H_kv, D // 32):
            raise TypeError(f"{n} must be a contiguous CUDA tensor of shape {(cap, H_kv, D // 32)}")
    bt = 0
    if block_table is not None:
        _need(block_table, torch.int32, "block_table")
        bt = block_table.data_ptr()
    return SeqView(0, 0, int(ctx_len), int(cap), H_kv * D, D, int(window), 1 if ring else 0, bt,
                   int(block_size), kv_type, kq.data_ptr(), vq.data_ptr(), kd.data_ptr(),
                   vd.data_ptr())


def _views(views):
    arr = (SeqView * len(views))(*views)
    return arr


def kv_append_f16(k_new, v_new, views, stream=None):
    """Writes fp16(k_new[s]), fp16(v_new[s]) into row ctx_len-1 of each view."""
    import torch
    _need(k_new, torch.float32, "k_new")
    _need(v_new, torch.float32, "v_new")
    n_seq, H_kv, D = k_new.shape
    arr = _views(views)
    _check("sd_kv_append_f16", _lib.load().sd_kv_append_f16(
        _p(k_new), _p(v_new), H_kv * D, arr, len(views), H_kv, D, _stream(stream)))


def kv_append_q8_0(k_new, v_new, views, stream=None):
    """Writes the q8_0 blocks of k_new[s], v_new[s] into row ctx_len-1 of each
    q8_0 view."""
    import torch
    _need(k_new, torch.float32, "k_new")
    _need(v_new, torch.float32, "v_new")
    n_seq, H_kv, D = k_new.shape
    arr = _views(views)
    _check("sd_kv_append_q8_0", _lib.load().sd_kv_append_q8_0(
        _p(k_new), _p(v_new), H_kv * D, arr, len(views), H_kv, D, _stream(stream)))


def decode_attn_workspace_bytes(views, H_q, D):
    return _lib.load().sd_decode_attn_workspace_bytes(_views(views), len(views), H_q, D)


def decode_attn_multiseq(q, views, H_kv, scale, out=None, ws=None, stream=None):
    """q [n_seq][H_q][D] fp32 -> out [n_seq][H_q][D] fp32."""
    import torch
    _need(q, torch.float32, "q")
    n_seq, H_q, D = q.shape
    arr = _views(views)
    need = _lib.load().sd_decode_attn_workspace_bytes(arr, len(views), H_q, D)
    if ws is None:
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q) if out is None else out
    _check("sd_decode_attn_multiseq", _lib.load().sd_decode_attn_multiseq(
        _p(q), H_q * D, arr, len(views), H_q, H_kv, D, float(scale), _p(out), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return out


def decode_attn_multiseq_noalloc(q, views, H_kv, scale, out=None, stream=None):
    """decode_attn_multiseq with the partials in the library's static scratch
    array (no workspace; calls that overlap on one GPU race)."""
    import torch
    _need(q, torch.float32, "q")
    n_seq, H_q, D = q.shape
    out = torch.empty_like(q) if out is None else out
    _check("sd_decode_attn_multiseq_noalloc", _lib.load().sd_decode_attn_multiseq_noalloc(
        _p(q), H_q * D, _views(views), len(views), H_q, H_kv, D, float(scale), _p(out),
        _stream(stream)))
    return out


def decode_attn_verify(q, views, n_new, H_kv, scale, out=None, ws=None, stream=None):
    """q [rows][H_q][D] fp32 with rows = sum(n_new), packed by sequence; the
    n_new[s] newest positions of sequence s attend causally -> out like q."""
    import torch
    _need(q, torch.float32, "q")
    rows, H_q, D = q.shape
    if rows != sum(n_new):
        raise ValueError("q rows must equal sum(n_new)")
    arr = _views(views)
    nn = (ctypes.c_int32 * len(n_new))(*[int(v) for v in n_new])
    need = _lib.load().sd_decode_attn_verify_workspace_bytes(arr, nn, len(views), H_q, D)
    if ws is None:
        ws = torch.zeros(max(need, 16), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q) if out is None else out
    _check("sd_decode_attn_verify", _lib.load().sd_decode_attn_verify(
        _p(q), H_q * D, arr, nn, len(views), H_q, H_kv, D, float(scale), _p(out), _p(ws),
        ws.numel() * ws.element_size(), _stream(stream)))
    return out


def rmsnorm_q8(x, gamma, eps, want_y=False, stream=None):
    import torch
    _need(x, torch.float32, "x")
    _need(gamma, torch.float32, "gamma")
    n_tok, D = x.shape
    xq = torch.empty((n_tok, D), dtype=torch.int8, device=x.device)
    xd = torch.empty((n_tok, D // 32), dtype=torch.float32, device=x.device)
    y = torch.empty_like(x) if want_y else None
    _check("sd_rmsnorm_q8", _lib.load().sd_rmsnorm_q8(
        _p(x), D, n_tok, D, _p(gamma), float(eps), _p(xq), _p(xd), _p(y), _stream(stream)))
    return (xq, xd, y) if want_y else (xq, xd)


def swiglu_q8(gu, F, want_y=False, stream=None):
    import torch
    _need(gu, torch.float32, "gu")
    n_tok = gu.shape[0]
    xq = torch.empty((n_tok, F), dtype=torch.int8, device=gu.device)
    xd = torch.empty((n_tok, F // 32), dtype=torch.float32, device=gu.device)
    y = torch.empty((n_tok, F), dtype=torch.float32, device=gu.device) if want_y else None
    _check("sd_swiglu_q8", _lib.load().sd_swiglu_q8(
        _p(gu), gu.shape[1], n_tok, F, _p(xq), _p(xd), _p(y), _stream(stream)))
    return (xq, xd, y) if want_y else (xq, xd)


def qgemv_q8_0_swiglu_q8(w, F, K, xq, xd, stream=None):
    """gate|up projection (w: 2F q8_0 rows of K) and SwiGLU in one launch ->
    (xq_out int8 [n_tok][F], xd_out fp32 [n_tok][F/32]); bitwise equal to
    qgemv_q8_0_batch followed by swiglu_q8."""
    import torch
    _need(w, torch.uint8, "w")
    _need(xq, torch.int8, "xq")
    _need(xd, torch.float32, "xd")
    n_tok = xq.shape[0]
    oq = torch.empty((n_tok, F), dtype=torch.int8, device=xq.device)
    od = torch.empty((n_tok, F // 32), dtype=torch.float32, device=xq.device)
    _check("sd_qgemv_q8_0_swiglu_q8", _lib.load().sd_qgemv_q8_0_swiglu_q8(
        _p(w), F, K, _p(xq), _p(xd), n_tok, _p(oq), _p(od), _stream(stream)))
    return oq, od


def embed_f16(table, tokens, stream=None):
    import torch
    _need(tokens, torch.int32, "tokens")
    V, H = table.shape
    x = torch.empty((tokens.numel(), H), dtype=torch.float32, device=tokens.device)
    _check("sd_embed_f16", _lib.load().sd_embed_f16(
        _p(table), V, H, _p(tokens), tokens.numel(), _p(x), _stream(stream)))
    return x


def argmax_rows(logits, stream=None):
    import torch
    _need(logits, torch.float32, "logits")
    n_tok, V = logits.shape
    out = torch.empty(n_tok, dtype=torch.int32, device=logits.device)
    need = _lib.load().sd_argmax_workspace_bytes(n_tok, V)
    ws = torch.empty(max(need, 4), dtype=torch.uint8, device=logits.device)
    _check("sd_argmax_rows", _lib.load().sd_argmax_rows(
        _p(logits), V, n_tok, V, _p(out), _p(ws), ws.numel(), _stream(stream)))
    return out
