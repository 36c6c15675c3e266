"""The fused decode step on the GPU: bitwise batch invariance (the hard gate)
and end-to-end agreement with the oracle's step.

Batch invariance, bitwise: each sequence's logits, next token and cache rows
are those of a step holding it alone, for 1..4 sequences, any order, over a
64-step soak that feeds tokens back, and across a cancel/reset/reuse of one
slot.  Against the oracle: requantization between layers makes the end-to-end
result discontinuous (one activation code can flip when an input moves by an
ulp), so the check is normwise (logits within 1e-3 relative) and on tokens
whose top-2 margin is clear.
"""
import numpy as np
import pytest

import oracle
from oracle import step as ostep
from helpers import bits, dev, host, say
from sequence_decode_amd import synth
from sequence_decode_amd.step import DecodeModel, SeqCache, StepRunner

pytestmark = pytest.mark.gpu

DIMS = dict(n_layers=2, hidden=512, n_heads=4, n_kv_heads=1, head_dim=128, ffn=768, vocab=1000)
CAP = 320


@pytest.fixture(scope="module")
def model_host():
    return synth.model_host(3000, **DIMS)


@pytest.fixture(scope="module")
def model(sd, model_host):
    return DecodeModel.from_host(model_host)


def _caches_host(n, seed=3001):
    g = synth.rng(seed)
    return [synth.prefilled_cache(g, DIMS["n_layers"], CAP, DIMS["n_kv_heads"], DIMS["head_dim"])
            for _ in range(n)]


def _run(model, caches_h, tokens, pos):
    """One GPU step on fresh device copies; returns logits, tokens, device caches."""
    caches = [SeqCache.from_host(k, v) for k, v in caches_h]
    r = StepRunner(model, caches, max_ctx=CAP)
    r.tokens.copy_(dev(np.asarray(tokens, np.int32)))
    r.set_positions(pos)
    r.step()
    return host(r.logits), host(r.next_tokens), [(host(c.k), host(c.v)) for c in caches]


def test_step_batched_equals_solo(sd, model):
    say("step batched == solo")
    ch = _caches_host(4)
    toks, pos = [11, 222, 333, 999], [0, 130, 256, 319]
    lg, nt, cs = _run(model, ch, toks, pos)
    for s in range(4):
        l1, n1, c1 = _run(model, [ch[s]], [toks[s]], [pos[s]])
        assert np.array_equal(bits(l1[0]), bits(lg[s])), s
        assert n1[0] == nt[s]
        assert np.array_equal(c1[0][0], cs[s][0]) and np.array_equal(c1[0][1], cs[s][1])
    perm = [2, 0, 3, 1]
    lp, npm, _ = _run(model, [ch[i] for i in perm], [toks[i] for i in perm], [pos[i] for i in perm])
    assert np.array_equal(bits(lp), bits(lg[perm])) and np.array_equal(npm, nt[perm])
    for n in (2, 3):
        ln, nn, _ = _run(model, ch[:n], toks[:n], pos[:n])
        assert np.array_equal(bits(ln), bits(lg[:n]))


def test_step_soak_64_steps_and_slot_reuse(sd, model):
    """Four sequences decode 64 steps batched; every step equals the solo runs.
    At step 20 slot 1 is cancelled, reset to a new sequence and reused."""
    import torch
    say("step soak 64")
    ch = _caches_host(5, seed=3100)
    start = [3, 40, 100, 250]
    first = [5, 6, 7, 8]
    steps = 64
    # batched run with a reset of slot 1 at step 20 (new cache = ch[4], new start 0)
    caches = [SeqCache.from_host(*ch[s]) for s in range(4)]
    r = StepRunner(model, caches, max_ctx=CAP)
    pos = list(start)
    tok = list(first)
    hist = [[] for _ in range(4)]
    for i in range(steps):
        if i == 20:
            fresh = SeqCache.from_host(*ch[4])
            caches[1].k.copy_(fresh.k)
            caches[1].v.copy_(fresh.v)
            pos[1], tok[1] = 0, 42
        r.tokens.copy_(torch.tensor(tok, dtype=torch.int32))
        r.set_positions(pos)
        r.step()
        lg = host(r.logits)
        nt = host(r.next_tokens)
        for s in range(4):
            hist[s].append((lg[s].copy(), int(nt[s])))
        tok = [int(t) for t in nt]
        pos = [p + 1 for p in pos]
    # solo reference runs
    def solo(cache_h, p0, t0, n_steps):
        c = SeqCache.from_host(*cache_h)
        rr = StepRunner(model, [c], max_ctx=CAP)
        out, p, t = [], p0, t0
        for _ in range(n_steps):
            rr.tokens.copy_(torch.tensor([t], dtype=torch.int32))
            rr.set_positions([p])
            rr.step()
            l1 = host(rr.logits)[0].copy()
            t = int(host(rr.next_tokens)[0])
            out.append((l1, t))
            p += 1
        return out
    for s in (0, 2, 3):
        ref = solo(ch[s], start[s], first[s], steps)
        for i in range(steps):
            assert np.array_equal(bits(ref[i][0]), bits(hist[s][i][0])), (s, i)
            assert ref[i][1] == hist[s][i][1]
    ref1a = solo(ch[1], start[1], first[1], 20)
    for i in range(20):
        assert np.array_equal(bits(ref1a[i][0]), bits(hist[1][i][0]))
    ref1b = solo(ch[4], 0, 42, steps - 20)
    for i in range(steps - 20):
        assert np.array_equal(bits(ref1b[i][0]), bits(hist[1][20 + i][0]))


def test_step_matches_oracle_end_to_end(sd, model, model_host):
    say("step vs oracle")
    h = model_host
    m = ostep.Model(h["hidden"], h["n_heads"], h["n_kv_heads"], h["head_dim"], h["ffn"],
                    h["vocab"], h["eps"], h["theta"], h["tok_embd_bits"], h["out_norm"],
                    h["w_lm"], h["layers"])
    ch = _caches_host(4, seed=3200)
    toks, pos = [1, 2, 500, 998], [7, 64, 255, 300]
    lg, nt, cs = _run(model, ch, toks, pos)
    ocache = [(k.copy(), v.copy()) for k, v in ch]
    olg, ont = ostep.decode_step(m, ocache, toks, pos)
    rel = np.linalg.norm(lg - olg) / np.linalg.norm(olg)
    say(f"  logits normwise relative error vs oracle: {rel:.3e}")
    assert rel <= 1e-3
    for s in range(4):
        top = np.sort(olg[s])[-2:]
        if top[1] - top[0] > 1e-3 * abs(top[1]):
            assert nt[s] == ont[s]
        for L in range(DIMS["n_layers"]):
            gk = cs[s][0][L, pos[s]].view(np.float16).astype(np.float32)
            ok = ocache[s][0][L, pos[s]].view(np.float16).astype(np.float32)
            assert np.max(np.abs(gk - ok)) <= 2e-2 * max(1.0, np.max(np.abs(ok)))


def test_verify_step_equals_one_token_steps(sd, model, model_host):
    """A verify step (several tokens per sequence through the whole model, causal
    within each sequence) gives, for every token row, bitwise the logits of
    one-token steps of that sequence alone run one after another over the same
    tokens, and leaves the same caches.  Bursts straddle a 256-key chunk edge."""
    import torch
    say("verify step == sequential one-token steps")
    ch = _caches_host(3, seed=3300)
    news, pos = [4, 2, 3], [10, 255, 100]
    toks = [[5, 17, 333, 2], [999, 0], [41, 42, 43]]
    caches = [SeqCache.from_host(*c) for c in ch]
    r = StepRunner(model, caches, max_ctx=CAP, n_new=news)
    r.tokens.copy_(torch.tensor(sum(toks, []), dtype=torch.int32))
    r.set_positions(pos)
    r.step()
    lg, nt = host(r.logits), host(r.next_tokens)
    row = 0
    for s in range(3):
        c1 = SeqCache.from_host(*ch[s])
        rr = StepRunner(model, [c1], max_ctx=CAP)
        for i in range(news[s]):
            rr.tokens.copy_(torch.tensor([toks[s][i]], dtype=torch.int32))
            rr.set_positions([pos[s] + i])
            rr.step()
            assert np.array_equal(bits(host(rr.logits)[0]), bits(lg[row])), (s, i)
            assert int(host(rr.next_tokens)[0]) == int(nt[row])
            row += 1
        assert np.array_equal(host(c1.k), host(caches[s].k)) and np.array_equal(host(c1.v), host(caches[s].v))
    # and against the oracle's sequential steps for the first sequence
    h = model_host
    m = ostep.Model(h["hidden"], h["n_heads"], h["n_kv_heads"], h["head_dim"], h["ffn"],
                    h["vocab"], h["eps"], h["theta"], h["tok_embd_bits"], h["out_norm"],
                    h["w_lm"], h["layers"])
    oc = [(ch[0][0].copy(), ch[0][1].copy())]
    for i in range(news[0]):
        olg, _ = ostep.decode_step(m, oc, [toks[0][i]], [pos[0] + i])
        rel = np.linalg.norm(lg[i] - olg[0]) / np.linalg.norm(olg[0])
        assert rel <= 1e-3, (i, rel)


@pytest.mark.parametrize("n_rot", [64, 128])
def test_window_rope_tail_step_vs_oracle_and_ring(sd, n_rot):
    """A model with a 100-position attention window and RoPE on the last n_rot
    of 128 head dims (64: the separate RoPE/KV launch; 128: RoPE and the K/V
    write in the QKV projection's epilogue): the step agrees with the oracle's
    step, and the same steps on ring caches of window + 3 rows give bitwise the
    plain-cache logits, for one-token steps and for a verify step."""
    import torch
    say(f"window + rope (n_rot {n_rot}) step, ring == plain")
    h = synth.model_host(3400, **DIMS)
    h["n_rot"], h["window"] = n_rot, 100
    model = DecodeModel.from_host(h)
    m = ostep.Model(h["hidden"], h["n_heads"], h["n_kv_heads"], h["head_dim"], h["ffn"],
                    h["vocab"], h["eps"], h["theta"], h["tok_embd_bits"], h["out_norm"],
                    h["w_lm"], h["layers"], n_rot=n_rot, window=100)
    ch = _caches_host(2, seed=3401)
    toks, pos = [3, 700], [150, 290]
    lg, nt, cs = _run(model, ch, toks, pos)
    ocache = [(k.copy(), v.copy()) for k, v in ch]
    olg, ont = ostep.decode_step(m, ocache, toks, pos)
    rel = np.linalg.norm(lg - olg) / np.linalg.norm(olg)
    say(f"  logits normwise relative error vs oracle: {rel:.3e}")
    assert rel <= 1e-3
    # ring caches: each layer keeps the last 103 positions at row j % 103
    cap = 103
    rings = []
    for k, v in ch:
        rk = np.zeros((k.shape[0], cap) + k.shape[2:], k.dtype)
        rings.append((rk, np.zeros_like(rk)))
    for s in range(2):
        k, v = ch[s]
        for j in range(pos[s] - cap + 1, pos[s]):
            rings[s][0][:, j % cap], rings[s][1][:, j % cap] = k[:, j], v[:, j]
    plain = [SeqCache.from_host(*c) for c in ch]
    ring = [SeqCache.from_host(*c) for c in rings]
    rp = StepRunner(model, plain, max_ctx=CAP)
    rr = StepRunner(model, ring, max_ctx=CAP, ring=True)
    t = list(toks)
    for step in range(6):
        for r_ in (rp, rr):
            r_.tokens.copy_(torch.tensor(t, dtype=torch.int32))
            r_.set_positions([p + step for p in pos])
            r_.step()
        assert np.array_equal(bits(host(rp.logits)), bits(host(rr.logits))), step
        t = [int(x) for x in host(rp.next_tokens)]
    # a verify step of 3 tokens per sequence on both
    vp = StepRunner(model, plain, max_ctx=CAP, n_new=[3, 3])
    vr = StepRunner(model, ring, max_ctx=CAP, n_new=[3, 3], ring=True)
    for r_ in (vp, vr):
        r_.tokens.copy_(torch.tensor([9, 8, 7, 6, 5, 4], dtype=torch.int32))
        r_.set_positions([p + 6 for p in pos])
        r_.step()
    assert np.array_equal(bits(host(vp.logits)), bits(host(vr.logits)))


def test_paged_pool_step_equals_plain(sd, model):
    """Three sequences whose caches live in one shared pool of 64-row blocks at
    shuffled places: one-token steps (crossing a block edge) and a verify step
    give bitwise the plain-cache logits, and the pool rows the step wrote hold
    the plain caches' new rows."""
    import torch
    say("paged pool step == plain")
    bs = 64
    ch = _caches_host(3, seed=3500)
    nb = CAP // bs
    n_pool = 3 * nb + 2
    place = synth.rng(3501).permutation(n_pool)
    tables = [place[s * nb:(s + 1) * nb].astype(np.int32) for s in range(3)]
    L_, _, Hkv, Dh = ch[0][0].shape
    pk = np.zeros((L_, n_pool * bs, Hkv, Dh), np.uint16)
    pv = np.zeros_like(pk)
    rows = [tables[s][np.arange(CAP) // bs] * bs + np.arange(CAP) % bs for s in range(3)]
    for s, (k, v) in enumerate(ch):
        pk[:, rows[s]], pv[:, rows[s]] = k, v
    plain = [SeqCache.from_host(*c) for c in ch]
    pool = SeqCache.from_host(pk, pv)
    tabs = [dev(t) for t in tables]
    rp = StepRunner(model, plain, max_ctx=CAP)
    rq = StepRunner(model, [pool] * 3, max_ctx=CAP, block_tables=tabs, block_size=bs)
    toks, pos = [5, 17, 901], [62, 200, 250]
    t = list(toks)
    for step in range(4):
        for r_ in (rp, rq):
            r_.tokens.copy_(torch.tensor(t, dtype=torch.int32))
            r_.set_positions([p + step for p in pos])
            r_.step()
        assert np.array_equal(bits(host(rp.logits)), bits(host(rq.logits))), step
        t = [int(x) for x in host(rp.next_tokens)]
    vp = StepRunner(model, plain, max_ctx=CAP, n_new=[3, 1, 2])
    vq = StepRunner(model, [pool] * 3, max_ctx=CAP, n_new=[3, 1, 2], block_tables=tabs,
                    block_size=bs)
    for r_ in (vp, vq):
        r_.tokens.copy_(torch.tensor([9, 8, 7, 6, 5, 4], dtype=torch.int32))
        r_.set_positions([p + 4 for p in pos])
        r_.step()
    assert np.array_equal(bits(host(vp.logits)), bits(host(vq.logits)))
    pkh, pvh = host(pool.k), host(pool.v)
    for s, c in enumerate(plain):
        kh, vh = host(c.k), host(c.v)
        assert np.array_equal(pkh[:, rows[s]], kh) and np.array_equal(pvh[:, rows[s]], vh), s


def _q8_caches_host(n, seed, kt="q8_0", vt="q8_0"):
    """Quantized caches [n_layers][CAP][H_kv][D] codes (q8_0) or [..][D/2] nibble
    pairs (q4_0), K and V each, and [..][D/32] fp16 scale bits."""
    g = synth.rng(seed)
    L_, Hkv, Dh = DIMS["n_layers"], DIMS["n_kv_heads"], DIMS["head_dim"]
    half = lambda ty: synth.kv_cache_q4 if ty == "q4_0" else synth.kv_cache_q8
    out = []
    for _ in range(n):
        kq, kd = half(kt)(g, L_ * CAP, Hkv, Dh)
        vq, vd = half(vt)(g, L_ * CAP, Hkv, Dh)
        out.append(tuple(a.reshape((L_, CAP) + a.shape[1:]) for a in (kq, kd, vq, vd)))
    return out


@pytest.mark.parametrize("kt,vt", [("q8_0", "q8_0"), ("q4_0", "q8_0"), ("q8_0", "q4_0")])
def test_q8_kv_step_oracle_invariance_and_verify(sd, model, model_host, kt, vt):
    """Steps over quantized caches (q8_0, and the mixed Q4/Q8 and Q8/Q4 types of
    "feat(qwen36): complete concurrent serving implementation with speculation",
    "Validation"): agreement with the oracle's step over the same caches; each
    sequence alone gives the batched bits (logits and cache rows); a verify step
    equals the sequential one-token steps."""
    import torch
    from sequence_decode_amd.step import SeqCacheQ8
    say(f"{kt}/{vt} KV step")
    h = model_host
    m = ostep.Model(h["hidden"], h["n_heads"], h["n_kv_heads"], h["head_dim"], h["ffn"],
                    h["vocab"], h["eps"], h["theta"], h["tok_embd_bits"], h["out_norm"],
                    h["w_lm"], h["layers"])
    ch = _q8_caches_host(4, 3600, kt, vt)
    toks, pos = [4, 77, 600, 999], [0, 63, 256, 319]

    def run(caches_h, tokens, positions, n_new=None):
        cs = [SeqCacheQ8.from_host(*c) for c in caches_h]
        r = StepRunner(model, cs, max_ctx=CAP, n_new=n_new)
        r.tokens.copy_(torch.tensor(tokens, dtype=torch.int32))
        r.set_positions(positions)
        r.step()
        return host(r.logits), host(r.next_tokens), [tuple(host(t) for t in (c.kq, c.kd, c.vq, c.vd)) for c in cs]

    lg, nt, cs = run(ch, toks, pos)
    ocache = [tuple(a.copy() for a in c) for c in ch]
    olg, ont = ostep.decode_step(m, ocache, toks, pos)
    rel = np.linalg.norm(lg - olg) / np.linalg.norm(olg)
    say(f"  {kt}/{vt} logits normwise relative error vs oracle: {rel:.3e}")
    assert rel <= 1e-3
    for s in range(4):
        l1, n1, c1 = run([ch[s]], [toks[s]], [pos[s]])
        assert np.array_equal(bits(l1[0]), bits(lg[s])) and n1[0] == nt[s], s
        for a, b in zip(c1[0], cs[s]):
            assert np.array_equal(a, b), s
    # verify step of 3 + 2 tokens against sequential one-token steps
    news, vpos, vt = [3, 2], [100, 255], [[5, 6, 7], [8, 9]]
    lv, nv, cv = run(ch[:2], vt[0] + vt[1], vpos, n_new=news)
    row = 0
    for s in range(2):
        c = [SeqCacheQ8.from_host(*ch[s])]
        rr = StepRunner(model, c, max_ctx=CAP)
        for i in range(news[s]):
            rr.tokens.copy_(torch.tensor([vt[s][i]], dtype=torch.int32))
            rr.set_positions([vpos[s] + i])
            rr.step()
            assert np.array_equal(bits(host(rr.logits)[0]), bits(lv[row])), (s, i)
            row += 1
        for a, b in zip((c[0].kq, c[0].kd, c[0].vq, c[0].vd), cv[s]):
            assert np.array_equal(host(a), b), s
