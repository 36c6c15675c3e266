"""Teacher-forced parity of the decode step, op by op, layer by layer.

Each layer runs on the GPU one C-ABI call at a time (rmsnorm_q8, GEMV, RoPE,
KV append, attention, quantize, GEMV + residual, rmsnorm_q8, GEMV, swiglu_q8,
GEMV + residual), and every op's output is checked against the oracle's op
applied to the GPU's own input of that op, so no error carries from one op to
the next: GEMV within 1e-5 of the sum of |terms|, attention within 2e-3
absolute (1e-4 normwise), RMSNorm 2e-6 relative, SwiGLU 8 ulp, RoPE 4 ulp of
the pair, and every quantization, fp16 rounding and argmax bitwise (each taken
in fp32 on the GPU's own values on both sides).  Then the same chain is shown
to be exactly the fused sd_decode_step: logits, tokens and cache rows bitwise.
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, gemv_tolerance, host, say
from sequence_decode_amd import synth
from sequence_decode_amd.step import DecodeModel, SeqCache, StepRunner

pytestmark = pytest.mark.gpu

DIMS = dict(n_layers=2, hidden=512, n_heads=8, n_kv_heads=2, head_dim=128, ffn=768, vocab=1000)
# the real head shape: QKV 6144 x 4096 (768 RoPE pair groups, 3 per workgroup
# of the fused launch), FFN 14336, the full 151,936-row LM head
REAL = dict(n_layers=1, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
            vocab=151936)
CAP = 600


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return np.spacing(np.maximum(x, np.float32(1e-30)))


def _check_gemv(y, blob, N, K, xq, xd, residual=None):
    ref, sh, ab = oracle.qgemv_q8_0(blob, N, K, xq, xd, residual=residual, want_terms=True)
    if residual is not None:  # the fp64 shadow sum is over the block terms only
        sh = sh + residual.astype(np.float64)
        ab = ab + np.abs(residual)
    assert np.all(np.abs(y.astype(np.float64) - sh) <= gemv_tolerance(ab) + 1e-30), (N, K)


def _check_quant(xq, xd, y):
    rq, rd = oracle.quantize_q8_act(y)
    assert np.array_equal(xq, rq) and np.array_equal(bits(xd), bits(rd))


@pytest.mark.parametrize("dims", [DIMS, REAL], ids=["small", "real_heads"])
def test_layer_ops_teacher_forced_and_fused_step(sd, dims):
    import torch
    say(f"teacher-forced step ops {dims}")
    h = synth.model_host(3700, **dims)
    model = DecodeModel.from_host(h)
    H, Hq, Hkv, Dh, F, V = (dims[k] for k in ("hidden", "n_heads", "n_kv_heads", "head_dim", "ffn",
                                             "vocab"))
    QKV = (Hq + 2 * Hkv) * Dh
    eps, theta = np.float32(h["eps"]), h["theta"]
    scale = np.float32(1.0) / np.sqrt(np.float32(Dh))
    g = synth.rng(3701)
    caches = [synth.prefilled_cache(g, dims["n_layers"], CAP, Hkv, Dh) for _ in range(3)]
    toks = np.array([17, 999, 3], np.int32)
    pos = np.array([0, 257, 599], np.int32)
    n = len(toks)
    ctx = [int(p) + 1 for p in pos]

    # fused step on its own copies
    fused = [SeqCache.from_host(k.copy(), v.copy()) for k, v in caches]
    r = StepRunner(model, fused, max_ctx=CAP)
    r.tokens.copy_(dev(toks))
    r.set_positions(pos.tolist())
    r.step()
    lg_fused, nt_fused = host(r.logits), host(r.next_tokens)

    # the same step op by op, every op checked against the oracle on its GPU input
    chain = [SeqCache.from_host(k.copy(), v.copy()) for k, v in caches]
    x = sd.embed_f16(model.tok_embd, dev(toks))
    assert np.array_equal(bits(host(x)), bits(oracle.f16_decode(h["tok_embd_bits"][toks]).astype(np.float32)))
    pos_d = dev(pos)
    for li, L in enumerate(h["layers"]):
        DL = model.layers[li]
        xh = host(x)
        aq, ad, y = sd.rmsnorm_q8(x, DL["attn_norm"], float(eps), want_y=True)
        ref = oracle.rmsnorm(xh, L["attn_norm"], float(eps))
        assert np.all(np.abs(host(y) - ref) <= 2e-6 * np.abs(ref) + 1e-30)
        _check_quant(host(aq), host(ad), host(y))
        qkv = sd.qgemv_q8_0_batch(DL["w_qkv"], QKV, H, aq, ad)
        _check_gemv(host(qkv), L["w_qkv"], QKV, H, host(aq), host(ad))
        q = qkv[:, :Hq * Dh].reshape(n, Hq, Dh).contiguous()
        k = qkv[:, Hq * Dh:(Hq + Hkv) * Dh].reshape(n, Hkv, Dh).contiguous()
        v = qkv[:, (Hq + Hkv) * Dh:].reshape(n, Hkv, Dh).contiguous()
        qh, kh = host(q), host(k)
        sd.rope_posvec(q, pos_d, theta)
        sd.rope_posvec(k, pos_d, theta)
        for got, src in ((host(q), qh), (host(k), kh)):
            ref = oracle.rope_posvec(src, pos, theta)
            half = Dh // 2
            pair = np.maximum(np.abs(ref[..., :half]), np.abs(ref[..., half:]))
            tol = 4 * _ulp32(np.concatenate([pair, pair], axis=-1))
            assert np.all(np.abs(got - ref) <= tol)
        views = [sd.seqview(c.k[li], c.v[li], L_) for c, L_ in zip(chain, ctx)]
        sd.kv_append_f16(k, v, views)
        for s in range(n):
            assert np.array_equal(host(chain[s].k[li])[pos[s]], oracle.f32_to_f16_bits(host(k)[s]))
            assert np.array_equal(host(chain[s].v[li])[pos[s]], oracle.f32_to_f16_bits(host(v)[s]))
        o = sd.decode_attn_multiseq(q, views, Hkv, scale)
        ref = oracle.attn_verify(host(q), [(host(c.k[li]), host(c.v[li])) for c in chain], ctx,
                                 [1] * n, scale)
        oh = host(o)
        assert np.max(np.abs(oh - ref)) <= 2e-3
        assert np.linalg.norm((oh - ref).ravel()) / np.linalg.norm(ref.ravel()) <= 1e-4
        oq, od = sd.quantize_q8_act(o.reshape(n, Hq * Dh))
        _check_quant(host(oq), host(od), oh.reshape(n, Hq * Dh))
        x_in = host(x)
        hx = sd.qgemv_q8_0_batch(DL["w_o"], H, Hq * Dh, oq, od, residual=x)
        _check_gemv(host(hx), L["w_o"], H, Hq * Dh, host(oq), host(od), residual=x_in)
        nq, nd, ny = sd.rmsnorm_q8(hx, DL["ffn_norm"], float(eps), want_y=True)
        ref = oracle.rmsnorm(host(hx), L["ffn_norm"], float(eps))
        assert np.all(np.abs(host(ny) - ref) <= 2e-6 * np.abs(ref) + 1e-30)
        _check_quant(host(nq), host(nd), host(ny))
        gu = sd.qgemv_q8_0_batch(DL["w_gu"], 2 * F, H, nq, nd)
        _check_gemv(host(gu), L["w_gu"], 2 * F, H, host(nq), host(nd))
        mq, md, my = sd.swiglu_q8(gu, F, want_y=True)
        guh = host(gu)
        ref = oracle.swiglu(guh[:, :F], guh[:, F:])
        assert np.all(np.abs(host(my) - ref) <= 8 * _ulp32(ref) + 1e-45)
        _check_quant(host(mq), host(md), host(my))
        h_in = host(hx)
        x = sd.qgemv_q8_0_batch(DL["w_down"], H, F, mq, md, residual=hx)
        _check_gemv(host(x), L["w_down"], H, F, host(mq), host(md), residual=h_in)
    fq, fd, fy = sd.rmsnorm_q8(x, model.out_norm, float(eps), want_y=True)
    ref = oracle.rmsnorm(host(x), h["out_norm"], float(eps))
    assert np.all(np.abs(host(fy) - ref) <= 2e-6 * np.abs(ref) + 1e-30)
    _check_quant(host(fq), host(fd), host(fy))
    lg = sd.qgemv_q8_0_batch(model.w_lm, V, H, fq, fd)
    _check_gemv(host(lg), h["w_lm"], V, H, host(fq), host(fd))
    nt = sd.argmax_rows(lg)
    assert np.array_equal(host(nt), oracle.argmax_rows(host(lg)))

    # the fused step is this chain, bit for bit
    assert np.array_equal(bits(host(lg)), bits(lg_fused))
    assert np.array_equal(host(nt), nt_fused)
    for c1, c2 in zip(chain, fused):
        assert np.array_equal(host(c1.k), host(c2.k)) and np.array_equal(host(c1.v), host(c2.v))
