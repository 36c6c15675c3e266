"""q4_0 KV caches and the mixed Q4/Q8, Q8/Q4 caches ("feat(qwen36): complete
concurrent serving implementation with speculation", "Validation": the Q4/Q8
and Q8/Q4 attention cases): the append against the oracle's quantizers
(bitwise), attention against the oracle over the dequantized caches, burst
tokens equal to one-token calls, batch invariance, and ring / paged storage
equal to plain storage bitwise.
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu

H_Q, H_KV, D = 32, 8, 128
SCALE = np.float32(1.0) / np.sqrt(np.float32(D))
TYPES = [("q4_0", "q8_0"), ("q8_0", "q4_0"), ("q4_0", "q4_0")]


def _half(g, n, ty):
    return synth.kv_cache_q4(g, n, H_KV, D) if ty == "q4_0" else synth.kv_cache_q8(g, n, H_KV, D)


def _kv(seed, n, kt, vt):
    g = synth.rng(seed)
    kq, kd = _half(g, n, kt)
    vq, vd = _half(g, n, vt)
    return kq, kd, vq, vd


def _views(sd, caches, lens, kt, vt, window=0, ring=False, tables=None, bs=0):
    import torch
    views, keep = [], []
    for i, ((kq, kd, vq, vd), L) in enumerate(zip(caches, lens)):
        t = [dev(kq), dev(kd, torch.float16), dev(vq), dev(vd, torch.float16)]
        bt = None if tables is None else dev(tables[i])
        keep += t + [bt]
        views.append(sd.seqview_quant(t[0], t[1], t[2], t[3], L, kt, vt, window=window, ring=ring,
                                      block_table=bt, block_size=bs))
    return views, keep


def _run(sd, q, caches, lens, news, kt, vt, **kw):
    views, keep = _views(sd, caches, lens, kt, vt, **kw)
    return host(sd.decode_attn_verify(dev(q), views, news, H_KV, SCALE))


def _check_parity(o, ref):
    assert np.max(np.abs(o - ref)) <= 2e-3
    rel = np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert rel <= 1e-4, rel


@pytest.mark.parametrize("kt,vt", TYPES)
@pytest.mark.parametrize("lens,news", [([1, 2, 63, 64], [1, 1, 1, 1]),
                                       ([65, 255, 256, 257], [1, 4, 2, 3]),
                                       ([2047, 2048, 2049, 2051], [1, 4, 2, 4])])
def test_q4_mixed_attention_parity_and_prefix(sd, kt, vt, lens, news):
    say(f"{kt}/{vt} attn {lens} {news}")
    caches = [_kv(6000 + i + sum(lens), L, kt, vt) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(6100 + sum(lens)), sum(news), H_Q, D)
    o = _run(sd, q, caches, lens, news, kt, vt)
    _check_parity(o, oracle.attn_verify(q, caches, lens, news, SCALE))
    # each burst token equals a one-token call over its own prefix
    r = 0
    for s, (L, T) in enumerate(zip(lens, news)):
        for i in range(T):
            one = _run(sd, q[r:r + 1], [caches[s]], [L - T + i + 1], [1], kt, vt)
            assert np.array_equal(bits(one[0]), bits(o[r])), (s, i)
            r += 1


@pytest.mark.parametrize("kt,vt", TYPES)
def test_q4_mixed_full_contexts_and_invariance(sd, kt, vt):
    """The decode contexts 2050, 3072, 16384, 32768: sampled rows against the
    oracle; each sequence alone, in any order, and with others gives the same
    bits."""
    lens = [2050, 3072, 16384, 32768]
    say(f"{kt}/{vt} attn full {lens}")
    caches = [_kv(6200 + i, L, kt, vt) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(6201), 4, H_Q, D)
    o = _run(sd, q, caches, lens, [1] * 4, kt, vt)
    for s in (0, 3):
        ref = oracle.attn_verify(q[s:s + 1], [caches[s]], [lens[s]], [1], SCALE)
        _check_parity(o[s:s + 1], ref)
    for s in range(4):
        solo = _run(sd, q[s:s + 1], [caches[s]], [lens[s]], [1], kt, vt)
        assert np.array_equal(bits(solo[0]), bits(o[s])), s
    perm = [3, 1, 0, 2]
    op = _run(sd, q[perm], [caches[i] for i in perm], [lens[i] for i in perm], [1] * 4, kt, vt)
    assert np.array_equal(bits(op), bits(o[perm]))


@pytest.mark.parametrize("kt,vt", TYPES[:2])
def test_q4_mixed_window_ring_and_paged_equal_plain(sd, kt, vt):
    lens, news, bs, window = [3000, 700, 4100, 300], [4, 1, 2, 3], 64, 100
    say(f"{kt}/{vt} window {window}: ring, paged")
    caches = [_kv(6300 + i, L, kt, vt) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(6301), sum(news), H_Q, D)
    o = _run(sd, q, caches, lens, news, kt, vt, window=window)
    _check_parity(o, oracle.attn_verify(q, caches, lens, news, SCALE, window=window))
    rings = []
    for c, L, T in zip(caches, lens, news):
        cap = min(L, window + T - 1) + 5
        ring = [np.zeros((cap,) + a.shape[1:], a.dtype) for a in c]
        for j in range(max(0, L - cap), L):
            for dst, src in zip(ring, c):
                dst[j % cap] = src[j]
        rings.append(tuple(ring))
    orr = _run(sd, q, rings, lens, news, kt, vt, window=window, ring=True)
    assert np.array_equal(bits(orr), bits(o))
    g = synth.rng(6302)
    nb = [(L + bs - 1) // bs for L in lens]
    place = g.permutation(sum(nb) + 2)
    pool = [np.zeros(((sum(nb) + 2) * bs,) + a.shape[1:], a.dtype) for a in caches[0]]
    tables, at = [], 0
    for c, L, n in zip(caches, lens, nb):
        tab = place[at:at + n].astype(np.int32)
        at += n
        rows = tab[np.arange(L) // bs] * bs + np.arange(L) % bs
        for dst, src in zip(pool, c):
            dst[rows] = src
        tables.append(tab)
    op = _run(sd, q, [tuple(pool)] * 4, lens, news, kt, vt, window=window, tables=tables, bs=bs)
    assert np.array_equal(bits(op), bits(o))


@pytest.mark.parametrize("kt,vt", TYPES)
def test_q4_mixed_single_key(sd, kt, vt):
    """One key: the output is that key's dequantized value (weight exactly 1)."""
    say(f"{kt}/{vt} single key")
    kq, kd, vq, vd = _kv(6400, 1, kt, vt)
    q = synth.queries(synth.rng(6401), 1, H_Q, D)
    o = _run(sd, q, [(kq, kd, vq, vd)], [1], [1], kt, vt)
    val = oracle.dequant_kv(vq, vd).astype(np.float32)
    for h in range(H_Q):
        assert np.array_equal(o[0, h], val[0, h // 4]), h


@pytest.mark.parametrize("kt,vt", TYPES)
def test_kv_append_q4_and_mixed_bitwise(sd, kt, vt):
    """Codes and fp16 scales of each half equal the oracle's quantizer of its
    type bit for bit (including an all-zero block and a block of ties), in plain,
    ring and paged rows; no other row changes."""
    import torch
    say(f"kv append {kt}/{vt}")
    cap, n_seq = 192, 3
    g = synth.rng(6500)
    k_new = g.standard_normal((n_seq, H_KV, D), dtype=np.float32) * 3
    v_new = g.standard_normal((n_seq, H_KV, D), dtype=np.float32)
    k_new[0, 0, :32] = 0.0
    # x / d = k + 1/2 exactly for a q4_0 block with amax 7 (d = 1), and for q8_0 too
    ties = (np.arange(32, dtype=np.float32) % 14) - np.float32(6.5)
    ties[0] = 7.0
    v_new[1, 2, 32:64] = ties
    k_new[2, 1, 64:96] = ties

    def zeros(ty):
        shape = (cap, H_KV, D // 2) if ty == "q4_0" else (cap, H_KV, D)
        return dev(np.zeros(shape, np.uint8 if ty == "q4_0" else np.int8))

    bufs = [[zeros(kt), dev(np.zeros((cap, H_KV, D // 32), np.uint16), torch.float16),
             zeros(vt), dev(np.zeros((cap, H_KV, D // 32), np.uint16), torch.float16)]
            for _ in range(n_seq)]
    tab = dev(np.array([2, 0, 1], np.int32))
    ctx = [100, 1000, 150]
    views = [sd.seqview_quant(*bufs[0], ctx[0], kt, vt),
             sd.seqview_quant(*bufs[1], ctx[1], kt, vt, window=cap, ring=True),
             sd.seqview_quant(*bufs[2], ctx[2], kt, vt, block_table=tab, block_size=64)]
    sd.kv_append_q8_0(dev(k_new), dev(v_new), views)
    rows = [ctx[0] - 1, (ctx[1] - 1) % cap, 1 * 64 + (ctx[2] - 1) % 64]
    quant = {"q4_0": oracle.quantize_kv_q4_0, "q8_0": oracle.quantize_kv_q8_0}
    for s in range(n_seq):
        kq, kd = quant[kt](k_new[s])
        vq, vd = quant[vt](v_new[s])
        got = [host(b) for b in bufs[s]]
        for a, want in zip(got, (kq, kd, vq, vd)):
            assert np.array_equal(a[rows[s]], want), s
            others = np.delete(np.arange(cap), rows[s])
            assert not a[others].any()
    assert not host(bufs[0][1])[rows[0], 0, 0]  # the all-zero block has scale +0
