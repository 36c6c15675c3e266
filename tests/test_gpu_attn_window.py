"""Sliding-window attention and ring caches (each sequence attends to its own
KV ring): parity with the oracle, ring == plain bitwise, burst tokens equal to
one-token calls over their own windows, and the append into a ring row.
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu

H_Q, H_KV, D = 32, 8, 128
SCALE = np.float32(1.0) / np.sqrt(np.float32(D))


def _kv(seed, n):
    g = synth.rng(seed)
    return synth.kv_cache(g, n, H_KV, D), synth.kv_cache(g, n, H_KV, D)


def _ring_of(k, v, ctx, cap):
    """The last `cap` positions of a plain cache, stored at row j % cap."""
    rk, rv = np.zeros((cap,) + k.shape[1:], k.dtype), np.zeros((cap,) + v.shape[1:], v.dtype)
    for j in range(max(0, ctx - cap), ctx):
        rk[j % cap], rv[j % cap] = k[j], v[j]
    return rk, rv


def _run(sd, q, kvs, lens, news, window, ring):
    import torch
    devs = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kvs]
    views = [sd.seqview(k, v, L, window=window, ring=ring) for (k, v), L in zip(devs, lens)]
    return host(sd.decode_attn_verify(dev(q), views, news, H_KV, SCALE))


def _check_parity(o, ref):
    assert np.max(np.abs(o - ref)) <= 2e-3
    rel = np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert rel <= 1e-4, rel


@pytest.mark.parametrize("window", [1, 100, 256, 257, 1000, 5000])
def test_window_parity_plain_and_ring(sd, window):
    say(f"window {window}")
    lens, news = [3000, 700, 4100, 300], [4, 1, 2, 3]
    kvs = [_kv(3000 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(3100 + window), sum(news), H_Q, D)
    o = _run(sd, q, kvs, lens, news, window, False)
    ref = oracle.attn_verify(q, kvs, lens, news, SCALE, window=window)
    _check_parity(o, ref)
    caps = [min(L, window + T - 1) + 5 for L, T in zip(lens, news)]
    rings = [_ring_of(k, v, L, cap) for (k, v), L, cap in zip(kvs, lens, caps)]
    orr = _run(sd, q, rings, lens, news, window, True)
    assert np.array_equal(bits(orr), bits(o))
    # each burst token equals a one-token call over its own window
    r = 0
    for s, (L, T) in enumerate(zip(lens, news)):
        for i in range(T):
            one = _run(sd, q[r:r + 1], [kvs[s]], [L - T + i + 1], [1], window, False)
            assert np.array_equal(bits(one[0]), bits(o[r])), (s, i)
            r += 1


@pytest.mark.parametrize("window", [60, 100, 2047])
def test_window_across_the_grid_edge(sd, window):
    """Windows that start among the 64-key chunks below position 2048 and end
    among the 256-key ones: oracle parity, ring == plain, burst token == its
    one-token call."""
    say(f"window {window} across the chunk grid edge")
    lens, news = [2100, 2049, 2400, 70], [4, 2, 3, 1]
    kvs = [_kv(3300 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(3400 + window), sum(news), H_Q, D)
    o = _run(sd, q, kvs, lens, news, window, False)
    ref = oracle.attn_verify(q, kvs, lens, news, SCALE, window=window)
    _check_parity(o, ref)
    caps = [min(L, window + T - 1) + 5 for L, T in zip(lens, news)]
    rings = [_ring_of(k, v, L, cap) for (k, v), L, cap in zip(kvs, lens, caps)]
    assert np.array_equal(bits(_run(sd, q, rings, lens, news, window, True)), bits(o))
    r = 0
    for s, (L, T) in enumerate(zip(lens, news)):
        for i in range(T):
            one = _run(sd, q[r:r + 1], [kvs[s]], [L - T + i + 1], [1], window, False)
            assert np.array_equal(bits(one[0]), bits(o[r])), (s, i)
            r += 1


def test_ring_wrapping_inside_a_chunk_and_small_ring(sd):
    """A ring smaller than a chunk (window 40, 43 rows), positions far past the
    ring size, so the rows of one chunk wrap."""
    say("small ring")
    lens, news, window = [10000, 77], [4, 2], 40
    kvs = [_kv(3200 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(3201), sum(news), H_Q, D)
    ref = oracle.attn_verify(q, kvs, lens, news, SCALE, window=window)
    rings = [_ring_of(k, v, L, window + 3) for (k, v), L in zip(kvs, lens)]
    o = _run(sd, q, rings, lens, news, window, True)
    _check_parity(o, ref)
    assert np.array_equal(bits(o), bits(_run(sd, q, kvs, lens, news, window, False)))


def test_kv_append_into_ring_row(sd):
    import torch
    say("kv append ring")
    cap, ctx = 50, 1234
    k = dev(np.zeros((cap, H_KV, D), np.uint16), torch.float16)
    v = dev(np.zeros((cap, H_KV, D), np.uint16), torch.float16)
    kn = synth.rng(3300).standard_normal((1, H_KV, D), dtype=np.float32)
    vn = synth.rng(3301).standard_normal((1, H_KV, D), dtype=np.float32)
    sd.kv_append_f16(dev(kn), dev(vn), [sd.seqview(k, v, ctx, window=cap, ring=True)])
    kh, vh = host(k), host(v)
    row = (ctx - 1) % cap
    assert np.array_equal(kh[row], oracle.f32_to_f16_bits(kn[0]))
    assert np.array_equal(vh[row], oracle.f32_to_f16_bits(vn[0]))
    others = np.delete(np.arange(cap), row)
    assert not kh[others].any() and not vh[others].any()
