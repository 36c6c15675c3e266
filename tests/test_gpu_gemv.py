"""GPU parity and batch invariance of the q8 quantizer and the q8_0 GEMV.

Oracle parity: the quantizer bitwise; the GEMV bitwise where the sum has one or
two nonzero terms, else within 1e-5 * sum|s_b| per element.  Invariance (GPU
vs GPU, bitwise): a token row's output is the same for every batch size 1..16,
row order, duplicated rows and changes to the other rows.
"""
import itertools

import numpy as np
import pytest

import oracle
from helpers import bits, dev, gemv_tolerance, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu


def _case(seed, N, K, n_tok, lo=1e-3, hi=1e-2):
    g = synth.rng(seed)
    blob, codes, sbits = synth.q8_0_weights(g, N, K, lo, hi)
    x = synth.activations(g, n_tok, K)
    return blob, x


def _gpu_quant(sd, x):
    xq, xd = sd.quantize_q8_act(dev(x))
    return xq, xd


# ------------------------------------------------------------------ quantizer

@pytest.mark.parametrize("n_tok,K", [(1, 32), (4, 4096), (16, 14336), (3, 1056)])
def test_quantize_bitwise(sd, n_tok, K):
    say(f"quantize n_tok={n_tok} K={K}")
    x = synth.rng(100 + K).standard_normal((n_tok, K), dtype=np.float32)
    x[0, :32] = 0.0                         # zero block
    if K >= 128:
        x[0, 32:64] *= np.float32(1e-40)    # denormal magnitudes
        x[0, 64:96] = np.float32(-3.5)      # every value equal to -amax
    xq, xd = _gpu_quant(sd, x)
    rq, rd = oracle.quantize_q8_act(x)
    assert np.array_equal(host(xq), rq)
    assert np.array_equal(bits(host(xd)), bits(rd))


def test_quantize_tie_cases_bitwise(sd):
    say("quantize ties")
    vals = np.array([0.5, -0.5, 1.5, 2.5, -2.5, 3.5, 4.5, 126.5, -126.5,
                     np.float32(0.49999997), np.float32(-0.49999997), np.float32(1.4999999)],
                    np.float32)
    x = np.zeros((1, 64), np.float32)
    x[0, 0] = 127.0
    x[0, 1:1 + vals.size] = vals
    x[0, 32] = -127.0
    x[0, 33:33 + vals.size] = vals[::-1]
    xq, xd = _gpu_quant(sd, x)
    rq, rd = oracle.quantize_q8_act(x)
    assert np.array_equal(host(xq), rq) and np.array_equal(host(xd), rd)


# ------------------------------------------------------------------ GEMV parity

def _run_gemv(sd, blob_dev, N, K, xq, xd, residual=None):
    y = sd.qgemv_q8_0_batch(blob_dev, N, K, xq, xd, residual=residual)
    return host(y)


def test_gemv_single_and_two_block_terms_bitwise(sd):
    """P1/P2: with one or two nonzero blocks the sum is one exact add."""
    say("gemv P1/P2")
    N, K = 33, 512
    blob, x = _case(200, N, K, 4)
    rq, rd = oracle.quantize_q8_act(x)
    for keep in ([0], [3], [0, 15], [7, 8], [1, 14]):
        xq = np.zeros_like(rq)
        for b in keep:
            xq[:, b * 32:(b + 1) * 32] = rq[:, b * 32:(b + 1) * 32]
        y = _run_gemv(sd, dev(blob), N, K, dev(xq), dev(rd))
        ref = oracle.qgemv_q8_0(blob, N, K, xq, rd)
        assert np.array_equal(bits(y), bits(ref)), keep


@pytest.mark.parametrize("N,K,n_tok", [
    (1, 256, 1), (7, 256, 3), (1000, 512, 4), (257, 768, 2), (513, 4096, 5),
    (96, 1280, 16), (130, 14336, 4), (64, 14336, 16), (1024, 4096, 8), (300, 2304, 12),
    (300, 8192, 3), (77, 6144, 7), (5000, 4352, 4),
])
def test_gemv_parity_small(sd, N, K, n_tok):
    say(f"gemv parity N={N} K={K} n_tok={n_tok}")
    blob, x = _case(300 + N + K + n_tok, N, K, n_tok)
    rq, rd = oracle.quantize_q8_act(x)
    y = _run_gemv(sd, dev(blob), N, K, dev(rq), dev(rd))
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, want_terms=True)
    assert np.all(np.abs(y - ref) <= gemv_tolerance(ab))
    assert np.all(np.abs(y.astype(np.float64) - sh) <= gemv_tolerance(ab))


def test_gemv_subnormal_scales_and_residual(sd):
    say("gemv subnormal scales + residual")
    N, K = 200, 1024
    blob, x = _case(400, N, K, 3, lo=1e-7, hi=5e-5)   # fp16 subnormal scales
    rq, rd = oracle.quantize_q8_act(x)
    r = synth.rng(401).standard_normal((3, N), dtype=np.float32)
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, residual=r, want_terms=True)
    rdev = dev(r)
    y = _run_gemv(sd, dev(blob), N, K, dev(rq), dev(rd), residual=rdev)
    assert np.all(np.abs(y - ref) <= gemv_tolerance(ab) + np.spacing(np.abs(r)))
    # in place: y = y + W x with residual == out
    ydev = dev(r)
    sd.qgemv_q8_0_batch(dev(blob), N, K, dev(rq), dev(rd), residual=ydev, out=ydev)
    assert np.array_equal(bits(host(ydev)), bits(y))


CONFIG_SHAPES = [  # (N, K): O proj, QKV, gate+up (fused rows), down
    (4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336)]


@pytest.mark.parametrize("N,K", CONFIG_SHAPES)
def test_gemv_parity_full_shapes(sd, N, K):
    say(f"gemv full N={N} K={K}")
    blob, x = _case(500 + N, N, K, 4)
    rq, rd = oracle.quantize_q8_act(x)
    bdev = dev(blob)
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, want_terms=True)
    for n_tok in (1, 2, 3, 4):
        y = _run_gemv(sd, bdev, N, K, dev(rq[:n_tok]), dev(rd[:n_tok]))
        assert np.all(np.abs(y - ref[:n_tok]) <= gemv_tolerance(ab[:n_tok])), n_tok


def test_gemv_lm_head_sampled_rows(sd):
    say("gemv LM head 151936x4096 sampled")
    N, K = 151936, 4096
    g = synth.rng(600)
    blob, _, _ = synth.q8_0_weights(g, N, K)
    x = synth.activations(g, 4, K)
    rq, rd = oracle.quantize_q8_act(x)
    y = _run_gemv(sd, dev(blob), N, K, dev(rq), dev(rd))
    rows = np.unique(np.concatenate([g.integers(0, N, 3000), [0, 1, N - 2, N - 1]])).astype(np.int64)
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, rows=rows, want_terms=True)
    assert np.all(np.abs(y[:, rows] - ref) <= gemv_tolerance(ab))


# ------------------------------------------------------------------ invariance

def test_gemv_width_invariance_1_to_16(sd):
    """Row t's bits are the same for every n_tok (the width-invariance gate)."""
    say("gemv width invariance")
    for (N, K) in ((1000, 4096), (260, 14336)):
        blob, x = _case(700 + K, N, K, 16)
        xq, xd = _gpu_quant(sd, x)
        bdev = dev(blob)
        full = _run_gemv(sd, bdev, N, K, xq, xd)
        for n in range(1, 17):
            y = _run_gemv(sd, bdev, N, K, xq[:n].contiguous(), xd[:n].contiguous())
            assert np.array_equal(bits(y), bits(full[:n])), (N, K, n)
        for t in range(16):
            solo = _run_gemv(sd, bdev, N, K, xq[t:t + 1].contiguous(), xd[t:t + 1].contiguous())
            assert np.array_equal(bits(solo[0]), bits(full[t])), (N, K, t)


def test_gemv_identical_rows_permutation_isolation(sd):
    say("gemv identical/permutation/isolation")
    N, K = 777, 4096
    blob, x = _case(800, N, K, 4)
    bdev = dev(blob)
    same = np.repeat(x[:1], 4, axis=0)
    xq, xd = _gpu_quant(sd, same)
    y = _run_gemv(sd, bdev, N, K, xq, xd)
    for t in range(1, 4):
        assert np.array_equal(bits(y[t]), bits(y[0]))
    xq, xd = _gpu_quant(sd, x)
    base = _run_gemv(sd, bdev, N, K, xq, xd)
    for perm in itertools.permutations(range(4)):
        p = list(perm)
        yp = _run_gemv(sd, bdev, N, K, xq[p].contiguous(), xd[p].contiguous())
        assert np.array_equal(bits(yp), bits(base[p]))
    x2 = x.copy()
    x2[1:] = synth.rng(801).standard_normal((3, K), dtype=np.float32)
    xq2, xd2 = _gpu_quant(sd, x2)
    y2 = _run_gemv(sd, bdev, N, K, xq2, xd2)
    assert np.array_equal(bits(y2[0]), bits(base[0]))


def test_gemv_batch_layouts(sd):
    """All ordered selections of 1..4 rows from a pool of 8 (2,080 layouts)
    against each row's solo output, plus 2,000 seeded layouts of 5..16 rows."""
    say("gemv layouts")
    N, K = 64, 512
    blob, x = _case(900, N, K, 8)
    bdev = dev(blob)
    xq, xd = _gpu_quant(sd, x)
    solo = np.stack([_run_gemv(sd, bdev, N, K, xq[t:t + 1].contiguous(),
                               xd[t:t + 1].contiguous())[0] for t in range(8)])
    count = 0
    for n in range(1, 5):
        for sel in itertools.permutations(range(8), n):
            s = list(sel)
            y = _run_gemv(sd, bdev, N, K, xq[s].contiguous(), xd[s].contiguous())
            assert np.array_equal(bits(y), bits(solo[s])), s
            count += 1
    assert count == 2080
    g = synth.rng(901)
    for _ in range(2000):
        n = int(g.integers(5, 17))
        s = list(g.integers(0, 8, n))
        y = _run_gemv(sd, bdev, N, K, xq[s].contiguous(), xd[s].contiguous())
        assert np.array_equal(bits(y), bits(solo[s])), s


def test_gemv_repeat_determinism(sd):
    say("gemv repeat determinism")
    N, K = 4096, 4096
    blob, x = _case(950, N, K, 4)
    bdev = dev(blob)
    xq, xd = _gpu_quant(sd, x)
    first = _run_gemv(sd, bdev, N, K, xq, xd)
    for _ in range(50):
        assert np.array_equal(bits(_run_gemv(sd, bdev, N, K, xq, xd)), bits(first))


@pytest.mark.parametrize("F,K", [(32, 256), (800, 1024), (768, 512), (14336, 4096)])
def test_gemv_swiglu_fused_equals_chain(sd, F, K):
    """The gate|up projection with SwiGLU in one launch gives exactly the codes
    and scales of the projection followed by sd_swiglu_q8, at every width the
    fused kernel takes (1 unit, ragged unit counts over the grid, the FFN)."""
    say(f"gemv+swiglu F={F} K={K}")
    blob, x = _case(900 + F + K, 2 * F, K, 8)
    rq, rd = oracle.quantize_q8_act(x)
    bdev = dev(blob)
    for n in range(1, 9):
        xq, xd = dev(rq[:n]), dev(rd[:n])
        oq, od = sd.qgemv_q8_0_swiglu_q8(bdev, F, K, xq, xd)
        gu = sd.qgemv_q8_0_batch(bdev, 2 * F, K, xq, xd)
        cq, cd = sd.swiglu_q8(gu, F)
        assert np.array_equal(host(oq), host(cq)), n
        assert np.array_equal(bits(host(od)), bits(host(cd))), n

