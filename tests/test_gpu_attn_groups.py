"""Decode attention for any number of query heads per KV head (H_q % H_kv == 0).

A workgroup takes a head group: hpw query heads of one KV head, hpw the largest
divisor of G = H_q / H_kv up to 4 (G = 1, 2, 3, 4 take one group per KV head;
G = 5, 6, 8 take 5, 2, 2 groups, each reading the KV head's keys and values).
Against the oracle (2e-3 absolute, 1e-4 normwise) on ragged contexts with
verify bursts, fp16, q8_0 and mixed q4_0/q8_0 caches and windows; bitwise:
burst tokens equal one-token calls over their prefixes, a sequence alone
equals it inside the batch, the allocation-free entry point equals the
workspace one, and ring and paged storage equal plain storage.
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu

D = 128
SCALE = np.float32(1.0) / np.sqrt(np.float32(D))
GROUPS = [(8, 8), (16, 8), (12, 4), (10, 2), (24, 4), (32, 4)]  # G = 1, 2, 3, 5, 6, 8


def _check_parity(o, ref):
    assert np.max(np.abs(o - ref)) <= 2e-3
    rel = np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert rel <= 1e-4, rel


def _fp16_caches(seed, lens, H_kv):
    g = synth.rng(seed)
    return [(synth.kv_cache(g, L + 2, H_kv, D), synth.kv_cache(g, L + 2, H_kv, D)) for L in lens]


@pytest.mark.parametrize("H_q,H_kv", GROUPS)
def test_groups_fp16_parity_prefix_and_solo(sd, H_q, H_kv):
    import torch
    say(f"attention head groups H_q={H_q} H_kv={H_kv}")
    lens, news = [2050, 65, 4097, 300], [4, 1, 3, 2]
    kv = _fp16_caches(7000 + H_q * 10 + H_kv, lens, H_kv)
    dkv = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kv]
    views = [sd.seqview(k, v, L) for (k, v), L in zip(dkv, lens)]
    q = synth.queries(synth.rng(7100 + H_q), sum(news), H_q, D)
    o = host(sd.decode_attn_verify(dev(q), views, news, H_kv, SCALE))
    _check_parity(o, oracle.attn_verify(q, kv, lens, news, SCALE))
    # each burst token: a one-token call over its own prefix
    r = 0
    for s, (L, n) in enumerate(zip(lens, news)):
        for i in range(n):
            p = L - n + i
            one = host(sd.decode_attn_multiseq(dev(q[r][None]), [sd.seqview(dkv[s][0], dkv[s][1], p + 1)],
                                               H_kv, SCALE))[0]
            assert np.array_equal(bits(o[r]), bits(one)), (s, i)
            r += 1
    # one token per sequence: batched == alone == the allocation-free entry point
    q1 = synth.queries(synth.rng(7200 + H_q), len(lens), H_q, D)
    ob = host(sd.decode_attn_multiseq(dev(q1), views, H_kv, SCALE))
    _check_parity(ob, oracle.attn_decode_multiseq(q1, kv, lens, SCALE))
    on = host(sd.decode_attn_multiseq_noalloc(dev(q1), views, H_kv, SCALE))
    assert np.array_equal(bits(ob), bits(on))
    for s in range(len(lens)):
        solo = host(sd.decode_attn_multiseq(dev(q1[s][None]), [views[s]], H_kv, SCALE))[0]
        assert np.array_equal(bits(ob[s]), bits(solo)), s


@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (32, 4)])
def test_groups_q8_parity(sd, H_q, H_kv):
    import torch
    say(f"q8 attention head groups H_q={H_q} H_kv={H_kv}")
    lens, news = [2051, 700, 17], [2, 4, 1]
    g = synth.rng(7300 + H_q)
    caches, views, keep = [], [], []
    for L in lens:
        kq, kd = synth.kv_cache_q8(g, L, H_kv, D)
        vq, vd = synth.kv_cache_q8(g, L, H_kv, D)
        caches.append((kq, kd, vq, vd))
        t = [dev(kq), dev(kd, torch.float16), dev(vq), dev(vd, torch.float16)]
        keep += t
        views.append(sd.seqview_q8(t[0], t[1], t[2], t[3], L))
    q = synth.queries(synth.rng(7400 + H_q), sum(news), H_q, D)
    o = host(sd.decode_attn_verify(dev(q), views, news, H_kv, SCALE))
    _check_parity(o, oracle.attn_verify(q, caches, lens, news, SCALE))


def test_groups_of_four_unchanged(sd):
    """G = 4 keeps one head group per KV head: a 32/8 call equals the same call
    split into its four 8/2 quarters (heads 8k .. 8k+7 over KV heads 2k, 2k+1)."""
    import torch
    say("attention G=4 quarters")
    lens = [2050, 3000]
    kv = _fp16_caches(7500, lens, 8)
    dkv = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kv]
    views = [sd.seqview(k, v, L) for (k, v), L in zip(dkv, lens)]
    q = synth.queries(synth.rng(7501), len(lens), 32, D)
    full = host(sd.decode_attn_multiseq(dev(q), views, 8, SCALE))
    for k in range(4):
        sub = [(dev(np.ascontiguousarray(c[0][:, 2 * k:2 * k + 2]), torch.float16),
                dev(np.ascontiguousarray(c[1][:, 2 * k:2 * k + 2]), torch.float16)) for c in kv]
        sv = [sd.seqview(a, b, L) for (a, b), L in zip(sub, lens)]
        part = host(sd.decode_attn_multiseq(dev(np.ascontiguousarray(q[:, 8 * k:8 * k + 8])), sv, 2, SCALE))
        assert np.array_equal(bits(part), bits(full[:, 8 * k:8 * k + 8])), k


def _ring_of(k, v, ctx, cap):
    """The last `cap` positions of a plain cache, stored at row j % cap."""
    rk, rv = np.zeros((cap,) + k.shape[1:], k.dtype), np.zeros((cap,) + v.shape[1:], v.dtype)
    for j in range(max(0, ctx - cap), ctx):
        rk[j % cap], rv[j % cap] = k[j], v[j]
    return rk, rv


def _pool_of(kvs, lens, bs, H_kv, seed, spare=3):
    """Every sequence's positions in blocks of bs rows at shuffled places of
    one pool, noise in the spare blocks.  Returns (pool_k, pool_v, tables)."""
    g = synth.rng(seed)
    nb = [(L + bs - 1) // bs for L in lens]
    n_pool = sum(nb) + spare
    place = g.permutation(n_pool)
    pk = synth.kv_cache(g, n_pool * bs, H_kv, D)
    pv = synth.kv_cache(g, n_pool * bs, H_kv, D)
    tables, nxt = [], 0
    for (k, v), L, n in zip(kvs, lens, nb):
        tab = place[nxt:nxt + n].astype(np.int32)
        nxt += n
        for j in range(L):
            r = tab[j // bs] * bs + j % bs
            pk[r], pv[r] = k[j], v[j]
        tables.append(tab)
    return pk, pv, tables


def _verify(sd, q, views, news, H_kv):
    return host(sd.decode_attn_verify(dev(q), views, news, H_kv, SCALE))


@pytest.mark.parametrize("H_q,H_kv", [(8, 8), (16, 8), (24, 4)])  # G = 1, 2, 6
def test_groups_window_ring_paged(sd, H_q, H_kv):
    """Head groups over windowed, ring and paged storage: windowed parity with
    the oracle, ring == plain and paged == plain bitwise."""
    import torch
    say(f"head groups window/ring/paged H_q={H_q} H_kv={H_kv}")
    lens, news, window, bs = [3000, 700, 4100, 300], [4, 1, 2, 3], 257, 64
    g = synth.rng(7600 + H_q + H_kv)
    kvs = [(synth.kv_cache(g, L, H_kv, D), synth.kv_cache(g, L, H_kv, D)) for L in lens]
    q = synth.queries(synth.rng(7700 + H_q), sum(news), H_q, D)
    keep = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kvs]
    plain_w = _verify(sd, q, [sd.seqview(k, v, L, window=window) for (k, v), L in zip(keep, lens)], news, H_kv)
    _check_parity(plain_w, oracle.attn_verify(q, kvs, lens, news, SCALE, window=window))
    caps = [min(L, window + T - 1) + 5 for L, T in zip(lens, news)]
    rings = [_ring_of(k, v, L, cap) for (k, v), L, cap in zip(kvs, lens, caps)]
    rdev = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in rings]
    ring_w = _verify(sd, q, [sd.seqview(k, v, L, window=window, ring=True) for (k, v), L in zip(rdev, lens)],
                     news, H_kv)
    assert np.array_equal(bits(ring_w), bits(plain_w))
    plain = _verify(sd, q, [sd.seqview(k, v, L) for (k, v), L in zip(keep, lens)], news, H_kv)
    pk, pv, tabs = _pool_of(kvs, lens, bs, H_kv, 7800 + H_q)
    dpk, dpv = dev(pk, torch.float16), dev(pv, torch.float16)
    dt = [dev(t) for t in tabs]
    paged = _verify(sd, q, [sd.seqview(dpk, dpv, L, block_table=t, block_size=bs) for t, L in zip(dt, lens)],
                    news, H_kv)
    assert np.array_equal(bits(paged), bits(plain))
    _check_parity(plain, oracle.attn_verify(q, kvs, lens, news, SCALE))


@pytest.mark.parametrize("kt,vt", [("q4_0", "q8_0"), ("q8_0", "q4_0")])
@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (32, 4)])  # G = 2, 8
def test_groups_mixed_quant_parity_and_prefix(sd, H_q, H_kv, kt, vt):
    """Head groups over the mixed q4_0 / q8_0 caches: parity with the oracle over
    the dequantized caches, and each burst token equal to a one-token call."""
    import torch
    say(f"head groups {kt}/{vt} H_q={H_q} H_kv={H_kv}")
    lens, news = [2051, 700, 17], [3, 4, 1]
    g = synth.rng(7900 + H_q + H_kv)
    half = lambda n, ty: synth.kv_cache_q4(g, n, H_kv, D) if ty == "q4_0" else synth.kv_cache_q8(g, n, H_kv, D)
    caches, views, keep = [], [], []
    for L in lens:
        kq, kd = half(L, kt)
        vq, vd = half(L, vt)
        caches.append((kq, kd, vq, vd))
        t = [dev(kq), dev(kd, torch.float16), dev(vq), dev(vd, torch.float16)]
        keep.append(t)
        views.append(sd.seqview_quant(t[0], t[1], t[2], t[3], L, kt, vt))
    q = synth.queries(synth.rng(7950 + H_q), sum(news), H_q, D)
    o = _verify(sd, q, views, news, H_kv)
    _check_parity(o, oracle.attn_verify(q, caches, lens, news, SCALE))
    r = 0
    for s, (L, T) in enumerate(zip(lens, news)):
        t = keep[s]
        for i in range(T):
            v1 = sd.seqview_quant(t[0], t[1], t[2], t[3], L - T + i + 1, kt, vt)
            one = _verify(sd, q[r:r + 1], [v1], [1], H_kv)
            assert np.array_equal(bits(one[0]), bits(o[r])), (s, i)
            r += 1


@pytest.mark.parametrize("H_q,H_kv", [(16, 8), (32, 4), (12, 4)])  # G = 2, 8, 3
def test_groups_batch_order(sd, H_q, H_kv):
    """The same sequences in reversed order give the same rows, bit for bit
    (one-token and verify calls)."""
    import torch
    say(f"head groups batch order H_q={H_q} H_kv={H_kv}")
    lens, news = [2050, 65, 4097, 300], [4, 1, 3, 2]
    kv = _fp16_caches(8100 + H_q + H_kv, lens, H_kv)
    dkv = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kv]
    views = [sd.seqview(k, v, L) for (k, v), L in zip(dkv, lens)]
    rev = views[::-1]
    q1 = synth.queries(synth.rng(8200 + H_q), len(lens), H_q, D)
    a = host(sd.decode_attn_multiseq(dev(q1), views, H_kv, SCALE))
    b = host(sd.decode_attn_multiseq(dev(np.ascontiguousarray(q1[::-1])), rev, H_kv, SCALE))
    assert np.array_equal(bits(a), bits(b[::-1]))
    q = synth.queries(synth.rng(8300 + H_q), sum(news), H_q, D)
    starts = np.cumsum([0] + news[:-1])
    qr = np.concatenate([q[s:s + n] for s, n in zip(starts[::-1], news[::-1])])
    o = host(sd.decode_attn_verify(dev(q), views, news, H_kv, SCALE))
    orv = host(sd.decode_attn_verify(dev(qr), rev, news[::-1], H_kv, SCALE))
    back = np.concatenate([orv[s:s + n] for s, n in zip(np.cumsum([0] + news[::-1][:-1])[::-1], news)])
    assert np.array_equal(bits(o), bits(back))
