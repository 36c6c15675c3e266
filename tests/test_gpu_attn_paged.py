"""Paged KV caches (a shared pool in blocks of 64, 128 or 256 rows, placed by
per-sequence block tables): parity with the oracle, paged == plain bitwise for
the same positions (one-token, verify and windowed calls), shared blocks,
clamped table entries, and the append into a paged row.
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


def _pool_of(kvs, lens, bs, seed, spare=3, share=0):
    """A pool holding every sequence's positions in blocks of bs rows at
    shuffled places, noise in the spare blocks.  share > 0: the sequences after
    the first use the first sequence's first `share` blocks (their caches must
    agree there).  Returns (pool_k, pool_v, tables)."""
    g = synth.rng(seed)
    nb = [(L + bs - 1) // bs for L in lens]
    n_pool = sum(nb) - share * (len(lens) - 1) + spare
    place = g.permutation(n_pool)
    pk = synth.kv_cache(g, n_pool * bs, H_KV, D)
    pv = synth.kv_cache(g, n_pool * bs, H_KV, D)
    tables, nxt = [], 0
    for s, ((k, v), L) in enumerate(zip(kvs, lens)):
        tab = np.empty(nb[s], np.int32)
        for b in range(nb[s]):
            if s > 0 and b < share:
                tab[b] = tables[0][b]
                continue
            tab[b] = place[nxt]
            nxt += 1
        for j in range(L):
            r = tab[j // bs] * bs + j % bs
            pk[r], pv[r] = k[j], v[j]
        tables.append(tab)
    return pk, pv, tables


def _run_plain(sd, q, kvs, lens, news, window=0):
    import torch
    devs = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kvs]
    views = [sd.seqview(k, v, L, window=window) for (k, v), L in zip(devs, lens)]
    return host(sd.decode_attn_verify(dev(q), views, news, H_KV, SCALE))


def _run_paged(sd, q, pool, tables, bs, lens, news, window=0, multiseq=False):
    import torch
    pk, pv = dev(pool[0], torch.float16), dev(pool[1], torch.float16)
    tabs = [dev(t) for t in tables]
    views = [sd.seqview(pk, pv, L, window=window, block_table=t, block_size=bs)
             for t, L in zip(tabs, lens)]
    if multiseq:
        return host(sd.decode_attn_multiseq(dev(q), views, H_KV, SCALE))
    return host(sd.decode_attn_verify(dev(q), views, news, H_KV, SCALE))


def _check_parity(o, ref):
    assert np.max(np.abs(o - ref)) <= 2e-3
    rel = np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert rel <= 1e-4, rel


@pytest.mark.parametrize("bs", [64, 128, 256])
def test_paged_parity_and_plain_bits(sd, bs):
    say(f"paged bs {bs}")
    lens, news = [1, 300, 2050, 777], [1, 4, 2, 3]
    kvs = [_kv(4000 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(4100 + bs), sum(news), H_Q, D)
    pool = _pool_of(kvs, lens, bs, 4200 + bs)
    o = _run_paged(sd, q, pool[:2], pool[2], bs, lens, news)
    ref = oracle.attn_verify(q, [pool[:2]] * 4, lens, news, SCALE, tables=pool[2], block_size=bs)
    _check_parity(o, ref)
    assert np.array_equal(bits(o), bits(_run_plain(sd, q, kvs, lens, news)))


def test_paged_one_token_entry(sd):
    say("paged multiseq")
    lens, bs = [5000, 64, 65, 1000], 128
    kvs = [_kv(4300 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(4301), len(lens), H_Q, D)
    pool = _pool_of(kvs, lens, bs, 4302)
    o = _run_paged(sd, q, pool[:2], pool[2], bs, lens, [1] * 4, multiseq=True)
    assert np.array_equal(bits(o), bits(_run_plain(sd, q, kvs, lens, [1] * 4)))


@pytest.mark.parametrize("window", [1, 100, 1000])
def test_paged_window_with_stale_entries(sd, window):
    """Blocks wholly below every query's window may hold any table entry:
    out-of-range values are clamped into the pool and never enter a sum."""
    say(f"paged window {window}")
    lens, news, bs = [3000, 700, 4100, 300], [4, 1, 2, 3], 64
    kvs = [_kv(4400 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(4401 + window), sum(news), H_Q, D)
    pk, pv, tables = _pool_of(kvs, lens, bs, 4402)
    for s, (L, T) in enumerate(zip(lens, news)):
        lo = max(0, L - T - window + 1)
        for b in range(lo // bs):
            tables[s][b] = [-7, 1 << 30, 3][b % 3]
    o = _run_paged(sd, q, (pk, pv), tables, bs, lens, news, window=window)
    assert np.array_equal(bits(o), bits(_run_plain(sd, q, kvs, lens, news, window=window)))
    _check_parity(o, oracle.attn_verify(q, kvs, lens, news, SCALE, window=window))


def test_paged_shared_prefix_blocks(sd):
    """Four sequences reading the same first four blocks of the pool."""
    say("paged shared prefix")
    lens, news, bs = [1100, 600, 2050, 257], [2, 4, 1, 3], 64
    base_k, base_v = _kv(4500, 4 * bs)
    kvs = []
    for i, L in enumerate(lens):
        k, v = _kv(4510 + i, L)
        k[:4 * bs], v[:4 * bs] = base_k, base_v
        kvs.append((k, v))
    q = synth.queries(synth.rng(4520), sum(news), H_Q, D)
    pool = _pool_of(kvs, lens, bs, 4521, share=4)
    assert all(np.array_equal(t[:4], pool[2][0][:4]) for t in pool[2])
    o = _run_paged(sd, q, pool[:2], pool[2], bs, lens, news)
    assert np.array_equal(bits(o), bits(_run_plain(sd, q, kvs, lens, news)))


def test_paged_long_context(sd):
    """A 32768-position sequence in 256-row blocks beside short ones."""
    say("paged 32768")
    lens, news, bs = [32768, 100, 4097, 1], [1, 2, 4, 1], 256
    kvs = [_kv(4600 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(4601), sum(news), H_Q, D)
    pool = _pool_of(kvs, lens, bs, 4602, spare=8)
    o = _run_paged(sd, q, pool[:2], pool[2], bs, lens, news)
    assert np.array_equal(bits(o), bits(_run_plain(sd, q, kvs, lens, news)))
    # sampled rows against the oracle (the last token of each sequence)
    r = np.cumsum(news) - 1
    ref = oracle.attn_verify(q[r], kvs, lens, [1] * 4, SCALE)
    _check_parity(o[r], ref)


def test_kv_append_into_paged_row(sd):
    import torch
    say("kv append paged")
    bs, n_pool, ctx = 64, 6, 200
    k = dev(np.zeros((n_pool * bs, H_KV, D), np.uint16), torch.float16)
    v = dev(np.zeros((n_pool * bs, H_KV, D), np.uint16), torch.float16)
    tab = np.array([4, 0, 5, 2], np.int32)
    kn = synth.rng(4700).standard_normal((1, H_KV, D), dtype=np.float32)
    vn = synth.rng(4701).standard_normal((1, H_KV, D), dtype=np.float32)
    t = dev(tab)
    sd.kv_append_f16(dev(kn), dev(vn), [sd.seqview(k, v, ctx, block_table=t, block_size=bs)])
    kh, vh = host(k), host(v)
    row = tab[(ctx - 1) // bs] * bs + (ctx - 1) % bs
    assert np.array_equal(kh[row], oracle.f32_to_f16_bits(kn[0]))
    assert np.array_equal(vh[row], oracle.f32_to_f16_bits(vn[0]))
    others = np.delete(np.arange(n_pool * bs), row)
    assert not kh[others].any() and not vh[others].any()
