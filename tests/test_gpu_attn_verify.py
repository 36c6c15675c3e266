"""Multi-token verify attention: the newest n_new positions of each sequence
attend causally (several proposed tokens per sequence checked together).

Oracle parity per token (2e-3 absolute, 1e-4 normwise).  Bitwise (GPU vs GPU):
burst token i equals a one-token call over its own prefix of p_i + 1 keys, so a
burst row is the same whatever the burst length, the other tokens, the other
sequences and their order.  Bursts that straddle chunk boundaries and bursts
covering the whole context are included.
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu

H_Q, H_KV, D = 32, 8, 128
SCALE = np.float32(1.0) / np.sqrt(np.float32(D))


def _seq(seed, cap):
    g = synth.rng(seed)
    return synth.kv_cache(g, cap, H_KV, D), synth.kv_cache(g, cap, H_KV, D)


def _upload(kv):
    import torch
    return dev(kv[0], torch.float16), dev(kv[1], torch.float16)


def _verify(sd, q_rows, devkv, lens, news):
    views = [sd.seqview(k, v, L) for (k, v), L in zip(devkv, lens)]
    return host(sd.decode_attn_verify(dev(q_rows), views, news, H_KV, SCALE))


def _single(sd, q, devkv, L):
    return host(sd.decode_attn_multiseq(dev(q[None]), [sd.seqview(devkv[0], devkv[1], L)], H_KV, SCALE))[0]


def _check_parity(o, ref):
    assert np.max(np.abs(o - ref)) <= 2e-3
    rel = np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert rel <= 1e-4, rel


CASES = [
    ([258, 3], [4, 3]),                    # burst straddles the 256-key chunk boundary; burst = context
    ([2050, 3072, 16384, 300], [4, 2, 3, 1]),
    ([1, 513, 256, 257], [1, 4, 4, 2]),
    ([2049, 2051, 66, 2300], [4, 4, 3, 2]),  # bursts across the 64 -> 256-key grid edge at 2048
    # a 256-key chunk with 66 keys below ctx_len (four waves) whose earlier
    # tokens see at most 64 of them (one wave in their one-token calls)
    ([2114, 2370, 130], [4, 4, 2]),
    # the newest token at 4096 has 41 chunks, the one before it 40: the merge
    # loads them in different numbers of rounds, with the same sums
    ([4097, 4095], [4, 2]),
]


@pytest.mark.parametrize("lens,news", CASES)
def test_verify_parity_and_prefix_equality(sd, lens, news):
    say(f"verify lens={lens} news={news}")
    kv = [_seq(2000 + i + L, L + 5) for i, L in enumerate(lens)]
    dkv = [_upload(x) for x in kv]
    q = synth.queries(synth.rng(2100 + sum(lens)), sum(news), H_Q, D)
    o = _verify(sd, q, dkv, lens, news)
    ref = oracle.attn_verify(q, kv, lens, news, SCALE)
    _check_parity(o, ref)
    r = 0
    for s, (L, T) in enumerate(zip(lens, news)):
        for i in range(T):
            p = L - T + i
            one = _single(sd, q[r], dkv[s], p + 1)
            assert np.array_equal(bits(o[r]), bits(one)), (s, i)
            r += 1


def test_verify_one_token_equals_multiseq(sd):
    say("verify n_new=1 == multiseq")
    lens = [2050, 17, 4000]
    kv = [_seq(2200 + i, L) for i, L in enumerate(lens)]
    dkv = [_upload(x) for x in kv]
    q = synth.queries(synth.rng(2201), 3, H_Q, D)
    o = _verify(sd, q, dkv, lens, [1, 1, 1])
    views = [sd.seqview(k, v, L) for (k, v), L in zip(dkv, lens)]
    m = host(sd.decode_attn_multiseq(dev(q), views, H_KV, SCALE))
    assert np.array_equal(bits(o), bits(m))


def test_verify_order_and_isolation(sd):
    say("verify order / isolation")
    lens, news = [700, 1500, 90], [3, 4, 2]
    kv = [_seq(2300 + i, L) for i, L in enumerate(lens)]
    dkv = [_upload(x) for x in kv]
    qs = [synth.queries(synth.rng(2310 + s), T, H_Q, D) for s, T in enumerate(news)]
    base = _verify(sd, np.concatenate(qs), dkv, lens, news)
    rows = np.cumsum([0] + news)
    for order in ([2, 0, 1], [1, 2, 0]):
        o = _verify(sd, np.concatenate([qs[s] for s in order]), [dkv[s] for s in order],
                    [lens[s] for s in order], [news[s] for s in order])
        r = 0
        for s in order:
            assert np.array_equal(bits(o[r:r + news[s]]), bits(base[rows[s]:rows[s + 1]]))
            r += news[s]
    # other sequences' queries and caches replaced: sequence 0 unchanged
    kv2 = [_seq(2400 + i, L) for i, L in enumerate(lens)]
    dkv2 = [dkv[0]] + [_upload(x) for x in kv2[1:]]
    q2 = np.concatenate([qs[0]] + [synth.queries(synth.rng(2410 + s), news[s], H_Q, D) for s in (1, 2)])
    o2 = _verify(sd, q2, dkv2, lens, news)
    assert np.array_equal(bits(o2[:news[0]]), bits(base[:news[0]]))
