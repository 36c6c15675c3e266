"""The widened verify batch: n_tok up to 16 on both q8_0 GEMV kernels.

The v_dot4 ("narrow") kernels and the matrix-core kernel (v_mfma_i32_16x16x32_i8)
form the same cells in the same fixed order, so their outputs must agree
bitwise for every shape and width; both are also held to the oracle (1e-5 of
sum|s_b| per element).  Shapes cover ragged N (not a multiple of the 16-row
tile), K whose last 64-pair chunk is partial, and the decode projections and
LM head at n_tok = 8, 12, 16 (several proposed tokens per sequence checked
together).
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, gemv_tolerance, host, say
from sequence_decode_amd import synth, GEMV_AUTO, GEMV_NARROW, GEMV_MFMA

pytestmark = pytest.mark.gpu


def _case(seed, N, K, n_tok):
    g = synth.rng(seed)
    blob, _, _ = synth.q8_0_weights(g, N, K)
    x = synth.activations(g, n_tok, K)
    return blob, x


def _y(sd, bdev, N, K, xq, xd, path, residual=None, out=None):
    return host(sd.qgemv_q8_0_batch(bdev, N, K, xq, xd, residual=residual, out=out, path=path))


@pytest.mark.parametrize("N,K", [(1, 256), (17, 512), (33, 1280), (250, 4352), (130, 14336),
                                 (1000, 4096), (48, 16384), (77, 16640)])
def test_mfma_equals_narrow_every_width(sd, N, K):
    say(f"mfma vs narrow N={N} K={K}")
    blob, x = _case(1100 + N + K, N, K, 16)
    rq, rd = oracle.quantize_q8_act(x)
    bdev = dev(blob)
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, want_terms=True)
    for n in range(1, 17):
        xq, xd = dev(rq[:n]), dev(rd[:n])
        ym = _y(sd, bdev, N, K, xq, xd, GEMV_MFMA)
        yn = _y(sd, bdev, N, K, xq, xd, GEMV_NARROW)
        ya = _y(sd, bdev, N, K, xq, xd, GEMV_AUTO)
        assert np.array_equal(bits(ym), bits(yn)), (N, K, n)
        assert np.array_equal(bits(ya), bits(yn)), (N, K, n)
        assert np.all(np.abs(ym - ref[:n]) <= gemv_tolerance(ab[:n])), (N, K, n)


CONFIG_SHAPES = [(4096, 4096), (6144, 4096), (28672, 4096), (4096, 14336)]


@pytest.mark.parametrize("N,K", CONFIG_SHAPES)
def test_verify_widths_full_shapes(sd, N, K):
    say(f"verify widths full N={N} K={K}")
    blob, x = _case(1200 + N, N, K, 16)
    rq, rd = oracle.quantize_q8_act(x)
    bdev = dev(blob)
    g = synth.rng(1201 + N)
    rows = np.unique(np.concatenate([g.integers(0, N, 1500), [0, 15, 16, N - 1]])).astype(np.int64)
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, rows=rows, want_terms=True)
    for n in (8, 12, 16):
        xq, xd = dev(rq[:n]), dev(rd[:n])
        ym = _y(sd, bdev, N, K, xq, xd, GEMV_MFMA)
        yn = _y(sd, bdev, N, K, xq, xd, GEMV_NARROW)
        assert np.array_equal(bits(ym), bits(yn)), (N, K, n)
        assert np.all(np.abs(ym[:, rows] - ref[:n]) <= gemv_tolerance(ab[:n])), (N, K, n)


def test_verify_width_lm_head_sampled(sd):
    say("verify width LM head 151936x4096, n_tok 16")
    N, K = 151936, 4096
    blob, x = _case(1300, N, K, 16)
    rq, rd = oracle.quantize_q8_act(x)
    bdev = dev(blob)
    ym = _y(sd, bdev, N, K, dev(rq), dev(rd), GEMV_MFMA)
    yn = _y(sd, bdev, N, K, dev(rq), dev(rd), GEMV_NARROW)
    assert np.array_equal(bits(ym), bits(yn))
    g = synth.rng(1301)
    rows = np.unique(np.concatenate([g.integers(0, N, 2000), [0, N - 1]])).astype(np.int64)
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, rq, rd, rows=rows, want_terms=True)
    assert np.all(np.abs(ym[:, rows] - ref) <= gemv_tolerance(ab))


def test_mfma_residual_in_place_and_isolation(sd):
    say("mfma residual / in place / row isolation")
    N, K = 300, 14336
    blob, x = _case(1400, N, K, 12)
    rq, rd = oracle.quantize_q8_act(x)
    bdev = dev(blob)
    r = synth.rng(1401).standard_normal((12, N), dtype=np.float32)
    ym = _y(sd, bdev, N, K, dev(rq), dev(rd), GEMV_MFMA, residual=dev(r))
    yn = _y(sd, bdev, N, K, dev(rq), dev(rd), GEMV_NARROW, residual=dev(r))
    assert np.array_equal(bits(ym), bits(yn))
    ydev = dev(r)
    sd.qgemv_q8_0_batch(bdev, N, K, dev(rq), dev(rd), residual=ydev, out=ydev, path=GEMV_MFMA)
    assert np.array_equal(bits(host(ydev)), bits(ym))
    # a token row is the same alone (narrow, width 1) as inside a permuted width-12 batch
    perm = synth.rng(1402).permutation(12)
    yp = _y(sd, bdev, N, K, dev(rq[perm]), dev(rd[perm]), GEMV_MFMA)
    for i, t in enumerate(perm):
        solo = _y(sd, bdev, N, K, dev(rq[t:t + 1]), dev(rd[t:t + 1]), GEMV_NARROW)
        assert np.array_equal(bits(yp[i]), bits(solo[0])), t
