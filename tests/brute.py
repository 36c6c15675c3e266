"""Independent brute-force references used to pin the oracle on tiny inputs.

These never call the oracle.  They evaluate the same definitions by other
means: exact integers, Python Fractions, 50-digit Decimals, and fp32 single
operations emulated in fp64.  The emulation is exact: a product of two fp32
values (or of an fp32 value and an integer below 2^29) is exact in fp64, and
for +, -, *, / rounding first to fp64 and then to fp32 gives the correctly
rounded fp32 result, because fp64 carries more than 2*24+2 significand bits
(Figueroa, "When is double rounding innocuous?", 1995).
"""
from decimal import Decimal, getcontext
from fractions import Fraction
import cmath
import math

import numpy as np

getcontext().prec = 50

f32 = np.float32
f64 = np.float64


def f32_div(a, b):
    return f32(f64(f32(a)) / f64(f32(b)))


def f32_mul(a, b):
    return f32(f64(f32(a)) * f64(f32(b)))


def f32_add(a, b):
    return f32(f64(f32(a)) + f64(f32(b)))


def round_half_away(v: float) -> int:
    """Nearest integer, ties away from zero, of an exactly representable value."""
    fr = Fraction(v)
    n = math.floor(abs(fr) + Fraction(1, 2))
    return n if fr >= 0 else -n


def quantize_block(xb):
    """One block of 32 fp32 values -> (codes list, fp32 scale), exact semantics."""
    amax = f32(0.0)
    for v in xb:
        a = f32(abs(f32(v)))
        if a > amax:
            amax = a
    d = f32_div(amax, f32(127.0))
    if d == 0:
        return [0] * len(xb), d
    codes = []
    for v in xb:
        r = round_half_away(float(f32_div(v, d)))
        codes.append(max(-127, min(127, r)))
    return codes, d


def quantize_rows_vectorized(x: np.ndarray):
    """Vectorized exact-semantics quantizer for large random samples."""
    n, K = x.shape
    xb = x.reshape(n, K // 32, 32).astype(np.float32)
    amax = np.abs(xb).max(axis=2)
    d = (amax.astype(np.float64) / 127.0).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (xb.astype(np.float64) / d[:, :, None].astype(np.float64)).astype(np.float32)
    aq = np.floor(np.abs(quot).astype(np.float64) + 0.5)  # exact for fp32 inputs
    q = np.where(quot < 0, -aq, aq)
    q = np.clip(q, -127, 127)
    q = np.where(d[:, :, None] == 0, 0, q)
    return q.astype(np.int8).reshape(n, K), d


def f16_bits_to_fraction(bits: int) -> Fraction:
    s = (bits >> 15) & 1
    e = (bits >> 10) & 31
    m = bits & 1023
    assert e != 31
    if e == 0:
        v = Fraction(m, 1 << 24)
    else:
        v = Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))
    return -v if s else v


def qgemv_exact(codes, scale_bits, xq, xd, residual=None):
    """y[t][n] with fp32 single-op semantics in block order (Python loops)."""
    N, K = codes.shape
    nb = K // 32
    n_tok = xq.shape[0]
    y = np.zeros((n_tok, N), np.float32)
    for t in range(n_tok):
        for n in range(N):
            acc = f32(0.0)
            for b in range(nb):
                isum = 0
                for i in range(32):
                    isum += int(codes[n, b * 32 + i]) * int(xq[t, b * 32 + i])
                dw = f32(float(f16_bits_to_fraction(int(scale_bits[n, b]))))
                s = f32_mul(f32_mul(dw, xd[t, b]), f32(isum))
                acc = f32_add(acc, s)
            if residual is not None:
                acc = f32_add(residual[t, n], acc)
            y[t, n] = acc
    return y


def D(v) -> Decimal:
    return Decimal(float(v))


def dexp(v: Decimal) -> Decimal:
    return v.exp()


def attn_decimal(q, k, v, ctx_len, scale, G):
    """q [H_q][D] float, k/v [ctx][H_kv][D] float values; 50-digit softmax."""
    H_q, Dd = q.shape
    out = np.zeros((H_q, Dd), np.float64)
    sc = D(scale)
    for h in range(H_q):
        g = h // G
        z = []
        for j in range(ctx_len):
            acc = Decimal(0)
            for d in range(Dd):
                acc += D(q[h, d]) * D(k[j, g, d])
            z.append(acc * sc)
        m = max(z)
        p = [dexp(zj - m) for zj in z]
        den = sum(p, Decimal(0))
        for d in range(Dd):
            num = sum((p[j] * D(v[j, g, d]) for j in range(ctx_len)), Decimal(0))
            out[h, d] = float(num / den)
    return out


def rmsnorm_decimal(x, gamma, eps):
    n, Dd = x.shape
    out = np.zeros((n, Dd), np.float64)
    for t in range(n):
        ss = sum((D(v) * D(v) for v in x[t]), Decimal(0))
        r = Decimal(1) / (ss / Decimal(Dd) + D(eps)).sqrt()
        for i in range(Dd):
            out[t, i] = float(D(x[t, i]) * r * D(gamma[i]))
    return out


def swiglu_decimal(g, u):
    out = np.zeros(g.shape, np.float64)
    for i, (gv, uv) in enumerate(zip(g.reshape(-1), u.reshape(-1))):
        G_ = D(gv)
        out.reshape(-1)[i] = float(G_ / (Decimal(1) + dexp(-G_)) * D(uv))
    return out


def ulp32(v):
    return np.spacing(np.abs(np.asarray(v, np.float32)).astype(np.float32))


# ------------------------------------------------------------ step composition

def unpack_q8_0(blob, N, K):
    """(codes int8 [N][K], fp16 scale bits uint16 [N][K/32]) of a q8_0 blob:
    each 34-byte block is a little-endian fp16 scale then 32 int8 codes."""
    b = np.asarray(blob, np.uint8).reshape(N, K // 32, 34)
    bits = b[:, :, 0].astype(np.uint16) | (b[:, :, 1].astype(np.uint16) << 8)
    codes = b[:, :, 2:].copy().view(np.int8).reshape(N, K)
    return codes, bits


def qgemv_exact_vec(codes, scale_bits, xq, xd, residual=None):
    """qgemv_exact vectorized over rows and tokens: exact int64 block sums, then
    emulated fp32 single operations in block order (same semantics)."""
    N, K = codes.shape
    nb = K // 32
    n_tok = xq.shape[0]
    c = codes.astype(np.int64).reshape(N, nb, 32)
    x = xq.astype(np.int64).reshape(n_tok, nb, 32)
    isum = np.einsum("nbi,tbi->tnb", c, x)              # exact integers
    dw = scale_bits.view(np.float16).astype(np.float64)  # [N][nb], exact
    acc = np.zeros((n_tok, N), np.float32)
    for b in range(nb):
        sc = (dw[None, :, b] * xd[:, b, None].astype(np.float64)).astype(np.float32)
        s = (sc.astype(np.float64) * isum[:, :, b].astype(np.float64)).astype(np.float32)
        acc = (acc.astype(np.float64) + s.astype(np.float64)).astype(np.float32)
    if residual is not None:
        acc = (residual.astype(np.float64) + acc.astype(np.float64)).astype(np.float32)
    return acc


def rope_complex(x, pos, theta, n_rot):
    """x [n][H][D] -> copy whose last n_rot dims of every head are rotated:
    dims (off + i, off + i + n_rot/2) form the complex number a + ib, multiplied
    by e^{i pos theta^(-2i/n_rot)} (Python complex arithmetic), rounded to fp32."""
    x = np.array(x, np.float32, copy=True)
    n, H, Dd = x.shape
    off, half = Dd - n_rot, n_rot // 2
    for t in range(n):
        for h in range(H):
            for i in range(half):
                ang = float(pos[t]) * float(theta) ** (-2.0 * i / n_rot)
                z = complex(float(x[t, h, off + i]), float(x[t, h, off + i + half])) * cmath.exp(1j * ang)
                x[t, h, off + i], x[t, h, off + i + half] = np.float32(z.real), np.float32(z.imag)
    return x
