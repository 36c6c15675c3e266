"""The decode step for other numbers of query heads per KV head (n_heads %
n_kv_heads == 0): G = 1, 2 and 8 on a 2-layer model.  Bitwise: batched equals
solo, and a verify step equals one-token steps run one after another;
against the oracle's step: logits within 1e-3 normwise (as for G = 4)."""
import numpy as np
import pytest

from oracle import step as ostep
from helpers import bits, dev, host, say
from sequence_decode_amd import synth
from sequence_decode_amd.step import DecodeModel, SeqCache, StepRunner

pytestmark = pytest.mark.gpu

CAP = 300


def _dims(n_heads, n_kv):
    return dict(n_layers=2, hidden=512, n_heads=n_heads, n_kv_heads=n_kv, head_dim=128, ffn=768, vocab=1000)


def _run(model, caches_h, tokens, pos, news=None):
    import torch
    caches = [SeqCache.from_host(k, v) for k, v in caches_h]
    r = StepRunner(model, caches, max_ctx=CAP, n_new=news)
    r.tokens.copy_(torch.tensor(np.asarray(tokens, np.int32).ravel(), dtype=torch.int32))
    r.set_positions(pos)
    r.step()
    return host(r.logits), host(r.next_tokens), [(host(c.k), host(c.v)) for c in caches]


@pytest.mark.parametrize("n_heads,n_kv", [(4, 4), (4, 2), (8, 1)])
def test_step_head_groups(sd, n_heads, n_kv):
    say(f"step head groups n_heads={n_heads} n_kv={n_kv}")
    dims = _dims(n_heads, n_kv)
    h = synth.model_host(3900 + 10 * n_heads + n_kv, **dims)
    model = DecodeModel.from_host(h)
    g = synth.rng(3901 + n_heads)
    ch = [synth.prefilled_cache(g, dims["n_layers"], CAP, n_kv, 128) for _ in range(3)]
    toks, pos = [5, 600, 999], [3, 129, 270]
    lg, nt, cs = _run(model, ch, toks, pos)
    for s in range(3):
        l1, n1, c1 = _run(model, [ch[s]], [toks[s]], [pos[s]])
        assert np.array_equal(bits(l1[0]), bits(lg[s])), s
        assert np.array_equal(c1[0][0], cs[s][0]) and np.array_equal(c1[0][1], cs[s][1]), s
    m = ostep.Model(h["hidden"], h["n_heads"], h["n_kv_heads"], h["head_dim"], h["ffn"], h["vocab"], h["eps"],
                    h["theta"], h["tok_embd_bits"], h["out_norm"], h["w_lm"], h["layers"])
    oc = [(k.copy(), v.copy()) for k, v in ch]
    olg, _ = ostep.decode_step(m, oc, toks, pos)
    rel = np.linalg.norm(lg - olg) / np.linalg.norm(olg)
    say(f"  logits normwise relative error vs oracle: {rel:.3e}")
    assert rel <= 1e-3
    # a verify step of 3 tokens equals three one-token steps
    vt = [7, 8, 9]
    lv, _, cv = _run(model, [ch[1]], [vt], [100], news=[3])
    seq = [(ch[1][0].copy(), ch[1][1].copy())]
    for i in range(3):
        l1, _, seq = _run(model, seq, [vt[i]], [100 + i])
        assert np.array_equal(bits(l1[0]), bits(lv[i])), i
    assert np.array_equal(seq[0][0], cv[0][0]) and np.array_equal(seq[0][1], cv[0][1])
