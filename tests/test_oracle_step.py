"""Pins of the oracle's decode-step composition (CPU only)."""
import numpy as np

from sequence_decode_amd import synth
import oracle
from oracle import step as ostep

DIMS = dict(n_layers=2, hidden=256, n_heads=4, n_kv_heads=2, head_dim=64, ffn=512, vocab=96)


def _model(seed=70, **over):
    d = dict(DIMS, **over)
    h = synth.model_host(seed, **d)
    m = ostep.Model(h["hidden"], h["n_heads"], h["n_kv_heads"], h["head_dim"], h["ffn"],
                    h["vocab"], h["eps"], h["theta"], h["tok_embd_bits"], h["out_norm"],
                    h["w_lm"], h["layers"])
    return h, m


def _caches(n, cap, seed=71):
    g = synth.rng(seed)
    return [synth.prefilled_cache(g, DIMS["n_layers"], cap, DIMS["n_kv_heads"], DIMS["head_dim"])
            for _ in range(n)]


def test_zero_layers_copy_the_input_token():
    """All-zero layer weights make every layer the identity on the residual
    stream; an LM head whose row r holds sign(embedding[r]) with unit scales then
    scores the input token's own row highest (sum of |codes| beats any other row)."""
    h, m = _model()
    for L in m.layers:
        for key in ("w_qkv", "w_o", "w_gu", "w_down"):
            blob = L[key].reshape(-1, 34).copy()
            blob[:, 2:] = 0
            L[key] = blob.reshape(-1)
    V, H = m.vocab, m.hidden
    emb = m.tok_embd_bits.view(np.float16).astype(np.float32)
    codes = np.where(emb >= 0, 1, -1).astype(np.int8)
    m.w_lm = synth.pack_q8_0(codes, np.full((V, H // 32), 0x3C00, np.uint16))
    m.out_norm = np.ones(H, np.float32)
    toks = np.array([5, 17, 90, 33])
    caches = _caches(4, 40)
    _, nxt = ostep.decode_step(m, caches, toks, [10, 20, 30, 39])
    assert list(nxt) == list(toks)
    for s, p in enumerate([10, 20, 30, 39]):
        # rotated zeros may carry a negative sign; the values are zero
        assert np.all(caches[s][0][:, p].view(np.float16) == 0)
        assert np.all(caches[s][1][:, p].view(np.float16) == 0)


def test_step_writes_only_the_current_rows_and_is_per_sequence():
    h, m = _model(72)
    pos = [3, 17, 25]
    toks = np.array([1, 2, 3])
    c_batch = _caches(3, 32, seed=73)
    before = [(k.copy(), v.copy()) for k, v in c_batch]
    lg, nxt = ostep.decode_step(m, c_batch, toks, pos)
    for s, p in enumerate(pos):
        k0, v0 = before[s]
        k1, v1 = c_batch[s]
        mask = np.ones(k0.shape[1], bool)
        mask[p] = False
        assert np.array_equal(k0[:, mask], k1[:, mask]) and np.array_equal(v0[:, mask], v1[:, mask])
        assert not np.array_equal(k0[:, p], k1[:, p])
    # each sequence alone gives the same logits, cache rows and token
    for s, p in enumerate(pos):
        c_solo = [(before[s][0].copy(), before[s][1].copy())]
        lg1, nx1 = ostep.decode_step(m, c_solo, toks[s:s + 1], [p])
        assert np.array_equal(lg1[0], lg[s]) and nx1[0] == nxt[s]
        assert np.array_equal(c_solo[0][0], c_batch[s][0])


def test_first_layer_key_row_is_rotated_projection():
    """The cached key of layer 0 equals fp16(rope(W_k rmsnorm(embed))) - the
    projection rows Hq*D .. (Hq+Hkv)*D of w_qkv, rotated at the token's position."""
    h, m = _model(74, n_layers=1)
    pos, tok = 9, 7
    caches = [synth.prefilled_cache(synth.rng(75), 1, 16, DIMS["n_kv_heads"], DIMS["head_dim"])]
    ostep.decode_step(m, caches, [tok], [pos])
    x = oracle.f16_decode(m.tok_embd_bits[[tok]]).astype(np.float32)
    a = oracle.rmsnorm(x, m.layers[0]["attn_norm"], m.eps)
    aq, ad = oracle.quantize_q8_act(a)
    Hq, Hkv, D = m.n_heads, m.n_kv_heads, m.head_dim
    rows = np.arange(Hq * D, (Hq + Hkv) * D)
    kproj = oracle.qgemv_q8_0(m.layers[0]["w_qkv"], (Hq + 2 * Hkv) * D, m.hidden, aq, ad, rows=rows)
    k = oracle.rope_posvec(kproj.reshape(1, Hkv, D), [pos], m.theta)
    assert np.array_equal(caches[0][0][0, pos], oracle.f32_to_f16_bits(k[0]))
