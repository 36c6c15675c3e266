"""Plain CPU oracle for the exact multi-sequence decode step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
(``sequence_decode_amd``) never imports it, and this package never imports the
product library: the two meet only on seeded inputs.

The arithmetic lives in ``oracle.c`` (plain loops; see its header for the page
passages each function follows).  This module holds ctypes wrappers taking
numpy arrays, plus the few steps that are a single numpy library call
(fp32 -> fp16 rounding, gather, argmax) and the composition of the decode step.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    """Loads liboracle.so, compiling it first when it is missing or stale."""
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oracle_num_threads.restype = i32
        L.oracle_set_num_threads.argtypes = [i32]
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = f64
        L.oracle_f16_decode.argtypes = [P, i64, P]
        L.oracle_quantize_q8_act.argtypes = [P, i64, i32, i64, P, P]
        L.oracle_quantize_q8_act.restype = i32
        L.oracle_quantize_kv_q4_0.argtypes = [P, i64, i64, P, P]
        L.oracle_quantize_kv_q4_0.restype = i32
        L.oracle_qgemv_q8_0.argtypes = [P, i64, i64, P, i64, P, i64, i32, P, i64,
                                        P, i64, P, P, P, i64]
        L.oracle_rope_posvec.argtypes = [P, i32, i32, i32, i64, i64, P, f64, i32]
        L.oracle_attn_decode_one.argtypes = [P, P, P, i64, i64, i32, i32, i32, i32,
                                             f64, P]
        L.oracle_attn_decode_one_f64.argtypes = [P, P, P, i64, i64, i32, i32, i32, i32,
                                                 f64, P]
        L.oracle_rmsnorm.argtypes = [P, i64, i32, i64, P, f64, P, i64]
        L.oracle_swiglu.argtypes = [P, P, i64, P]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _req(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    """Thread count of the oracle's parallel loops (for timing on fewer cores)."""
    lib().oracle_set_num_threads(int(n))


def f16_decode(bits: np.ndarray) -> np.ndarray:
    """fp16 bit patterns (uint16) -> float64 values, decoded field by field."""
    bits = _req(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().oracle_f16_decode(_ptr(bits), bits.size, _ptr(out))
    return out


def quantize_q8_act(x: np.ndarray):
    """Per-token q8 activation blocks: returns (xq int8 [n][K], xd fp32 [n][K/32])."""
    x = _req(x, np.float32)
    n_tok, K = x.shape
    xq = np.empty((n_tok, K), np.int8)
    xd = np.empty((n_tok, K // 32), np.float32)
    rc = lib().oracle_quantize_q8_act(_ptr(x), K, n_tok, K, _ptr(xq), _ptr(xd))
    if rc != 0:
        raise ValueError("oracle quantize: K must be a multiple of 32 and x finite")
    return xq, xd


def qgemv_q8_0(w: np.ndarray, N: int, K: int, xq: np.ndarray, xd: np.ndarray,
               residual=None, rows=None, want_terms=False):
    """y[t][n] = residual + sum_b fl(fl(dw*dx)*isum) (fp32, block order).

    ``w`` is the packed weight blob (uint8, N*(K/32)*34 bytes).  ``rows``
    selects a subset of output rows (the result then has len(rows) columns).
    With ``want_terms`` also returns (shadow fp64 sum, sum of |s_b|).
    """
    w = _req(w, np.uint8).reshape(-1)
    assert w.size == N * (K // 32) * 34
    xq = _req(xq, np.int8)
    xd = _req(xd, np.float32)
    n_tok = xq.shape[0]
    assert xq.shape == (n_tok, K) and xd.shape == (n_tok, K // 32)
    if rows is not None:
        rows = _req(rows, np.int64)
        ncol = rows.size
    else:
        ncol = N
    y = np.empty((n_tok, ncol), np.float32)
    sh = np.empty((n_tok, ncol), np.float64) if want_terms else None
    ab = np.empty((n_tok, ncol), np.float64) if want_terms else None
    r = None
    if residual is not None:
        r = _req(residual, np.float32)
        assert r.shape == (n_tok, N)
    lib().oracle_qgemv_q8_0(_ptr(w), N, K, _ptr(xq), K, _ptr(xd), K // 32, n_tok,
                            _ptr(r), N if r is not None else 0, _ptr(y), ncol,
                            _ptr(sh), _ptr(ab), _ptr(rows),
                            0 if rows is None else rows.size)
    if want_terms:
        return y, sh, ab
    return y


def rope_posvec(x: np.ndarray, pos, theta: float, n_rot=None) -> np.ndarray:
    """x [n_tok][n_heads][head_dim] fp32 -> rotated copy (fp64 math)."""
    x = np.array(x, dtype=np.float32, copy=True, order="C")
    n_tok, n_heads, head_dim = x.shape
    n_rot = head_dim if n_rot is None else n_rot
    pos = _req(pos, np.int32)
    assert pos.shape == (n_tok,)
    lib().oracle_rope_posvec(_ptr(x), n_tok, n_heads, head_dim, n_heads * head_dim,
                             head_dim, _ptr(pos), float(theta), n_rot)
    return x


def attn_decode_one(q: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                    ctx_len: int, scale: float) -> np.ndarray:
    """One sequence: q [H_q][D] fp32, caches [cap][H_kv][D] fp16 bits -> [H_q][D].

    ``scale`` is an fp32 value (the library takes it as float); it is rounded to
    fp32 here before the fp64 arithmetic uses it.
    """
    q = _req(q, np.float32)
    H_q, D = q.shape
    assert D <= 1024
    k_bits = _req(k_bits, np.uint16)
    v_bits = _req(v_bits, np.uint16)
    cap, H_kv, Dk = k_bits.shape
    assert Dk == D and v_bits.shape == k_bits.shape and 1 <= ctx_len <= cap
    assert H_q % H_kv == 0
    out = np.empty((H_q, D), np.float32)
    lib().oracle_attn_decode_one(_ptr(q), _ptr(k_bits), _ptr(v_bits), H_kv * D, D,
                                 ctx_len, H_q, H_kv, D, float(np.float32(scale)), _ptr(out))
    return out


def quantize_kv_q8_0(x: np.ndarray):
    """q8_0 blocks of cache rows x [..., D] fp32 (the "int8 KV" cache of "#1209
    Speed up concurrent generation, fix QFUSE, and improve prefill monitoring",
    "What changed and why"): per run of 32 dims, d = amax / 127 and codes
    round-half-away(x / d) clamped to +-127, as the activation quantizer; the
    stored scale is fp16(d), nearest even.  Returns (codes int8 [..., D],
    scale bits uint16 [..., D/32])."""
    x = _req(x, np.float32)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    codes, d = quantize_q8_act(flat)
    return codes.reshape(x.shape), f32_to_f16_bits(d).reshape(x.shape[:-1] + (D // 32,))


def dequant_kv_q8_0(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """The values d * c of q8_0 cache rows, in fp64 (exact)."""
    codes = np.asarray(codes, np.int8)
    d = np.asarray(scale_bits, np.uint16).view(np.float16).astype(np.float64)
    return codes.astype(np.float64) * np.repeat(d, 32, axis=-1)


def quantize_kv_q4_0(x: np.ndarray):
    """q4_0 blocks of cache rows x [..., D] fp32 (the Q4 cache type of the Q4/Q8
    and Q8/Q4 cases in "feat(qwen36): complete concurrent serving implementation
    with speculation", "Validation"): per run of 32 dims, d = amax / 7 and codes
    c = round-half-away(x / d) in [-8, 7], stored as nibbles c + 8, two per byte
    (low nibble: the even dim); the stored scale is fp16(d), nearest even.
    Returns (packed uint8 [..., D/2], scale bits uint16 [..., D/32])."""
    x = _req(x, np.float32)
    D = x.shape[-1]
    flat = x.reshape(-1, D)
    packed = np.empty((flat.shape[0], D // 2), np.uint8)
    d = np.empty((flat.shape[0], D // 32), np.float32)
    rc = lib().oracle_quantize_kv_q4_0(_ptr(flat), flat.shape[0], D, _ptr(packed), _ptr(d))
    if rc != 0:
        raise ValueError("quantize_kv_q4_0: D must be a multiple of 32 and x finite")
    return (packed.reshape(x.shape[:-1] + (D // 2,)),
            f32_to_f16_bits(d).reshape(x.shape[:-1] + (D // 32,)))


def dequant_kv_q4_0(packed: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """The values d * (n - 8) of q4_0 cache rows, in fp64 (exact)."""
    packed = np.asarray(packed, np.uint8)
    n = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), np.int64)
    n[..., 0::2] = packed & 0x0F
    n[..., 1::2] = packed >> 4
    d = np.asarray(scale_bits, np.uint16).view(np.float16).astype(np.float64)
    return (n - 8).astype(np.float64) * np.repeat(d, 32, axis=-1)


def dequant_kv(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """dequant_kv_q8_0 for int8 codes [..., D], dequant_kv_q4_0 for packed
    uint8 nibbles [..., D/2]."""
    if np.asarray(codes).dtype == np.uint8:
        return dequant_kv_q4_0(codes, scale_bits)
    return dequant_kv_q8_0(codes, scale_bits)


def attn_decode_one_f64(q: np.ndarray, k: np.ndarray, v: np.ndarray, ctx_len: int,
                        scale: float) -> np.ndarray:
    """attn_decode_one over fp64 keys and values [cap][H_kv][D]."""
    q = _req(q, np.float32)
    H_q, D = q.shape
    assert D <= 1024
    k = _req(k, np.float64)
    v = _req(v, np.float64)
    cap, H_kv, Dk = k.shape
    assert Dk == D and v.shape == k.shape and 1 <= ctx_len <= cap
    assert H_q % H_kv == 0
    out = np.empty((H_q, D), np.float32)
    lib().oracle_attn_decode_one_f64(_ptr(q), _ptr(k), _ptr(v), H_kv * D, D, ctx_len, H_q, H_kv,
                                     D, float(np.float32(scale)), _ptr(out))
    return out


def attn_decode_multiseq(q: np.ndarray, caches, ctx_lens, scale: float) -> np.ndarray:
    """q [n_seq][H_q][D]; caches = [(k_bits, v_bits)] per sequence."""
    return np.stack([attn_decode_one(q[s], caches[s][0], caches[s][1], ctx_lens[s], scale)
                     for s in range(q.shape[0])])


def attn_verify(q_rows: np.ndarray, caches, ctx_lens, n_new, scale: float, window: int = 0,
                rings=None, tables=None, block_size: int = 0) -> np.ndarray:
    """Several query tokens per sequence, packed by sequence (the verification of
    proposed tokens in "feat(qwen36): complete concurrent serving implementation
    with speculation"): the n_new[s] newest positions of sequence s, token i at
    position p = ctx_lens[s] - n_new[s] + i.  A token attends to positions
    lo..p, lo = max(0, p - window + 1) with a window, else 0; it is the one-token
    decode attention over exactly those keys.  rings[s] true: the cache is a
    ring (ds4 pull request 604, "Commit walkthrough / CUDA kernels": each
    sequence attends to its own KV ring), position j stored in row j % capacity.
    tables[s] not None: the cache is a pool of blocks of block_size rows shared
    through per-sequence block tables ("feat(qwen36): complete concurrent serving
    implementation with speculation", "Summary"), position j stored in row
    tables[s][j // block_size] * block_size + j % block_size.
    caches[s] = (k_bits, v_bits) of an fp16 cache, or (kq, kd_bits, vq, vd_bits)
    of a quantized cache, attended over its dequantized values; K and V each
    q8_0 (int8 codes [..., D]) or q4_0 (uint8 nibbles [..., D/2]), so mixed
    Q4/Q8 and Q8/Q4 caches too.
    q_rows [sum(n_new)][H_q][D] -> same shape."""
    out = []
    r = 0
    for s, T in enumerate(n_new):
        if len(caches[s]) == 4:
            kq, kd, vq, vd = caches[s]
            k_bits, v_bits = dequant_kv(kq, kd), dequant_kv(vq, vd)
            one = attn_decode_one_f64
        else:
            k_bits, v_bits = caches[s]
            one = attn_decode_one
        cap = k_bits.shape[0]
        for i in range(T):
            p = ctx_lens[s] - T + i
            lo = max(0, p - window + 1) if window else 0
            rows = np.arange(lo, p + 1)
            if rings is not None and rings[s]:
                rows = rows % cap
            if tables is not None and tables[s] is not None:
                rows = np.asarray(tables[s], np.int64)[rows // block_size] * block_size \
                    + rows % block_size
            out.append(one(q_rows[r], k_bits[rows], v_bits[rows], p + 1 - lo, scale))
            r += 1
    return np.stack(out)


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    x = _req(x, np.float32)
    n_tok, D = x.shape
    gamma = _req(gamma, np.float32)
    y = np.empty_like(x)
    lib().oracle_rmsnorm(_ptr(x), D, n_tok, D, _ptr(gamma), float(np.float32(eps)), _ptr(y), D)
    return y


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _req(g, np.float32)
    u = _req(u, np.float32)
    assert g.shape == u.shape
    y = np.empty_like(g)
    lib().oracle_swiglu(_ptr(g), _ptr(u), g.size, _ptr(y))
    return y


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """IEEE round-to-nearest-even fp32 -> fp16 (numpy's conversion), as bits."""
    with np.errstate(over="ignore"):
        return np.asarray(x, np.float32).astype(np.float16).view(np.uint16)


def argmax_rows(logits: np.ndarray) -> np.ndarray:
    """Greedy token per row; numpy returns the lowest index among equal maxima."""
    return np.argmax(logits, axis=1).astype(np.int32)
