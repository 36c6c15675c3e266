"""GPU parity and batch invariance of multi-sequence decode attention.

Oracle parity: |o_gpu - o_oracle| <= 2e-3 absolute (fp32 online softmax vs the
fp64 oracle), and additionally a normwise relative error <= 1e-4.  Bitwise
(GPU vs GPU): a sequence's output is the same alone, in any batch, in any
order, and when the other sequences' data change.  ctx = 1 gives v_0 exactly.
"""
import itertools

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


def _gpu(sd, q, devkv, lens):
    views = [sd.seqview(k, v, L) for (k, v), L in zip(devkv, lens)]
    return host(sd.decode_attn_multiseq(dev(q), views, H_KV, SCALE))


def _check_parity(o, ref):
    assert np.max(np.abs(o - ref)) <= 2e-3
    rel = np.linalg.norm((o - ref).ravel()) / np.linalg.norm(ref.ravel())
    assert rel <= 1e-4, rel


@pytest.mark.parametrize("lens", [[1], [5], [255, 256, 257], [511, 512, 513, 1],
                                  [2050, 2051], [300, 17, 4000, 9],
                                  [63, 64, 65, 129],          # 64-key chunk edges
                                  [2047, 2048, 2049, 2305]])  # the 64 -> 256-key grid edge
def test_attention_parity_small(sd, lens):
    say(f"attention parity lens={lens}")
    kv = [_seq(1000 + i + L, L + 3) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(1100 + sum(lens)), len(lens), H_Q, D)
    o = _gpu(sd, q, [_upload(x) for x in kv], lens)
    ref = oracle.attn_decode_multiseq(q, kv, lens, SCALE)
    _check_parity(o, ref)


def test_attention_parity_sharpened(sd):
    say("attention parity sharpened q*4")
    lens = [700, 1500]
    kv = [_seq(1200 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(1201), 2, H_Q, D) * 4.0
    o = _gpu(sd, q, [_upload(x) for x in kv], lens)
    ref = oracle.attn_decode_multiseq(q, kv, lens, SCALE)
    _check_parity(o, ref)


def test_attention_single_key_is_exact(sd):
    say("attention ctx=1 exact")
    kv = [_seq(1300, 4)]
    q = synth.queries(synth.rng(1301), 1, H_Q, D)
    o = _gpu(sd, q, [_upload(kv[0])], [1])
    v0 = kv[0][1][0].view(np.float16).astype(np.float32)
    for h in range(H_Q):
        assert np.array_equal(bits(o[0, h]), bits(v0[h // 4]))


def test_attention_full_config_contexts(sd):
    """Four sequences at the ragged contexts {2050, 3072, 16384, 32768}."""
    say("attention full config")
    lens = [2050, 3072, 16384, 32768]
    kv = [_seq(1400 + i, L) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(1401), 4, H_Q, D)
    devkv = [_upload(x) for x in kv]
    o = _gpu(sd, q, devkv, lens)
    ref = oracle.attn_decode_multiseq(q, kv, lens, SCALE)
    _check_parity(o, ref)
    # each sequence alone gives the same bits
    for s in range(4):
        solo = _gpu(sd, q[s:s + 1], [devkv[s]], [lens[s]])
        assert np.array_equal(bits(solo[0]), bits(o[s])), s


def test_attention_invariance_permutation_isolation(sd):
    say("attention invariance")
    lens = [257, 1000, 2051, 40]
    kv = [_seq(1500 + i, L + 1) for i, L in enumerate(lens)]
    q = synth.queries(synth.rng(1501), 4, H_Q, D)
    devkv = [_upload(x) for x in kv]
    base = _gpu(sd, q, devkv, lens)
    for perm in itertools.permutations(range(4)):
        p = list(perm)
        o = _gpu(sd, q[p], [devkv[i] for i in p], [lens[i] for i in p])
        assert np.array_equal(bits(o), bits(base[p]))
    for n in (1, 2, 3):
        for sel in itertools.combinations(range(4), n):
            s = list(sel)
            o = _gpu(sd, q[s], [devkv[i] for i in s], [lens[i] for i in s])
            assert np.array_equal(bits(o), bits(base[s]))
    # changing the other sequences' queries, caches and lengths leaves sequence 0 unchanged
    kv2 = [_seq(1600 + i, 3000) for i in range(3)]
    q2 = q.copy()
    q2[1:] = synth.queries(synth.rng(1601), 3, H_Q, D)
    o = _gpu(sd, q2, [devkv[0]] + [_upload(x) for x in kv2], [lens[0], 2999, 12, 2048])
    assert np.array_equal(bits(o[0]), bits(base[0]))
    # identical sequences give identical rows
    o = _gpu(sd, np.repeat(q[:1], 4, axis=0), [devkv[0]] * 4, [lens[0]] * 4)
    for s in range(4):
        assert np.array_equal(bits(o[s]), bits(base[0]))


def test_workspace_reuse_across_shapes(sd):
    """One workspace serves successive calls of different shapes, and the
    results are those of calls on fresh workspaces (nothing carries over)."""
    import torch
    say("attention workspace reuse")
    cases = [([2050, 3072, 16384, 32768], [1, 1, 1, 1]), ([1, 300], [1, 1]), ([700, 65, 5000], [4, 2, 3])]
    size = 0
    prepared = []
    for i, (lens, news) in enumerate(cases):
        kv = [_seq(6000 + 10 * i + j, L) for j, L in enumerate(lens)]
        devkv = [_upload(x) for x in kv]
        views = [sd.seqview(k, v, L) for (k, v), L in zip(devkv, lens)]
        q = dev(synth.queries(synth.rng(6100 + i), sum(news), H_Q, D))
        need = sd._lib.load().sd_decode_attn_verify_workspace_bytes(
            sd._views(views), (__import__("ctypes").c_int32 * len(news))(*news), len(views), H_Q, D)
        size = max(size, need)
        prepared.append((views, news, q, devkv))
    ws = torch.zeros(size, dtype=torch.uint8, device="cuda")
    for rnd in range(2):
        for i, (views, news, q, _) in enumerate(prepared):
            shared = host(sd.decode_attn_verify(q, views, news, H_KV, SCALE, ws=ws))
            fresh = host(sd.decode_attn_verify(q, views, news, H_KV, SCALE))
            assert np.array_equal(bits(shared), bits(fresh)), (rnd, i)


def test_attention_maximum_context(sd):
    """The largest supported span, SD_MAX_CTX = 524288 keys (2072 chunks), in
    one sequence beside a short one: sampled heads against the oracle, and the
    long sequence alone gives the same bits."""
    import torch
    L_max = 2048 * 256
    say(f"attention at the maximum context {L_max}")
    g = torch.Generator(device="cuda")
    g.manual_seed(6200)
    k = torch.randn((L_max, H_KV, D), generator=g, device="cuda").half()
    v = torch.randn((L_max, H_KV, D), generator=g, device="cuda").half()
    ks, vs = _upload(_seq(6201, 300))
    q = synth.queries(synth.rng(6202), 2, H_Q, D)
    views = [sd.seqview(k, v, L_max), sd.seqview(ks, vs, 300)]
    o = host(sd.decode_attn_multiseq(dev(q), views, H_KV, SCALE))
    kh, vh = host(k), host(v)
    for gi in (0, 3, 7):  # KV heads 0, 3, 7 and their four query heads each
        ref = oracle.attn_decode_one(q[0][gi * 4:gi * 4 + 4], np.ascontiguousarray(kh[:, gi:gi + 1]),
                                     np.ascontiguousarray(vh[:, gi:gi + 1]), L_max, SCALE)
        _check_parity(o[0][gi * 4:gi * 4 + 4], ref)
    solo = host(sd.decode_attn_multiseq(dev(q[:1]), views[:1], H_KV, SCALE))
    assert np.array_equal(bits(solo[0]), bits(o[0]))
    # one key more than the maximum span is refused
    too_long = sd.SeqView(k.data_ptr(), v.data_ptr(), L_max + 1, L_max + 1, H_KV * D, D)
    with pytest.raises(sd.SdError):
        sd.decode_attn_multiseq(dev(q[:1]), [too_long], H_KV, SCALE, ws=torch.zeros(16, dtype=torch.uint8, device="cuda"))
