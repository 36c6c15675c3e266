"""GPU parity of pos-vector RoPE, the KV append and the step glue kernels."""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu


def _ulp(a):
    return np.spacing(np.abs(a).astype(np.float32))


# ------------------------------------------------------------------ RoPE

@pytest.mark.parametrize("n_tok,n_heads,head_dim,n_rot", [
    (4, 32, 128, 128), (4, 8, 128, 128), (16, 3, 64, 64), (2, 4, 128, 64), (1, 1, 8, 2)])
def test_rope_parity(sd, n_tok, n_heads, head_dim, n_rot):
    say(f"rope parity {n_tok} {n_heads} {head_dim} {n_rot}")
    g = synth.rng(2000 + head_dim + n_rot)
    x = g.standard_normal((n_tok, n_heads, head_dim), dtype=np.float32)
    pos = np.array(([2049, 3071, 16383, 32767] * 4)[:n_tok], np.int32)
    pos[0] = 0 if n_tok > 4 else pos[0]
    xd = dev(x)
    sd.rope_posvec(xd, dev(pos), 1e6, n_rot)
    y = host(xd)
    ref = oracle.rope_posvec(x, pos, 1e6, n_rot)
    off, half = head_dim - n_rot, n_rot // 2
    assert np.array_equal(bits(y[:, :, :off]), bits(x[:, :, :off]))
    pair_max = np.maximum(np.abs(x[:, :, off:off + half]), np.abs(x[:, :, off + half:]))
    tol = 4 * _ulp(pair_max)
    assert np.all(np.abs(y[:, :, off:off + half] - ref[:, :, off:off + half]) <= tol)
    assert np.all(np.abs(y[:, :, off + half:] - ref[:, :, off + half:]) <= tol)


def test_rope_position_zero_and_single_token_equivalence(sd):
    say("rope pos0 + posvec == single")
    g = synth.rng(2100)
    x = g.standard_normal((4, 32, 128), dtype=np.float32)
    z = dev(x)
    sd.rope_posvec(z, dev(np.zeros(4, np.int32)), 1e6)
    assert np.array_equal(bits(host(z)), bits(x))
    pos = np.array([2049, 3071, 16383, 32767], np.int32)
    full = dev(x)
    sd.rope_posvec(full, dev(pos), 1e6)
    yf = host(full)
    for t in range(4):
        one = dev(x[t:t + 1])
        sd.rope_posvec(one, dev(pos[t:t + 1]), 1e6)
        assert np.array_equal(bits(host(one)[0]), bits(yf[t]))


# ------------------------------------------------------------------ KV append

def test_kv_append_bitwise_and_rows_untouched(sd):
    import torch
    say("kv append")
    g = synth.rng(2200)
    caps, lens = [16, 40, 8], [3, 40, 1]
    ks = [synth.kv_cache(g, c, 8, 128) for c in caps]
    vs = [synth.kv_cache(g, c, 8, 128) for c in caps]
    kn = g.standard_normal((3, 8, 128), dtype=np.float32) * 300
    vn = g.standard_normal((3, 8, 128), dtype=np.float32)
    kn[0, 0, :4] = [70000.0, -1e-7, 6e-8, 65519.0]       # overflow, subnormal, tie, max
    kd = [dev(k, torch.float16) for k in ks]
    vd = [dev(v, torch.float16) for v in vs]
    views = [sd.seqview(kd[s], vd[s], lens[s]) for s in range(3)]
    sd.kv_append_f16(dev(kn), dev(vn), views)
    for s in range(3):
        K, V = host(kd[s]), host(vd[s])
        row = lens[s] - 1
        assert np.array_equal(K[row], oracle.f32_to_f16_bits(kn[s]))
        assert np.array_equal(V[row], oracle.f32_to_f16_bits(vn[s]))
        mask = np.arange(caps[s]) != row
        assert np.array_equal(K[mask], ks[s][mask]) and np.array_equal(V[mask], vs[s][mask])


# ------------------------------------------------------------------ glue

def test_rmsnorm_q8_parity_and_quantizer_consistency(sd):
    say("rmsnorm_q8")
    g = synth.rng(2300)
    for n, D in ((4, 4096), (1, 32), (16, 14336), (3, 800)):
        x = g.standard_normal((n, D), dtype=np.float32) * 3
        gamma = synth.uniform_f32(g, D, 0.5, 1.5)
        xq, xd, y = sd.rmsnorm_q8(dev(x), dev(gamma), 1e-6, want_y=True)
        yh = host(y)
        ref = oracle.rmsnorm(x, gamma, 1e-6)
        # fp32 sums of D squares (per-thread runs of D/256, then a 8-level tree)
        # plus sqrt, divide and two products: well inside 2e-6 relative
        assert np.all(np.abs(yh - ref) <= 2e-6 * np.abs(ref) + 1e-30)
        # the fused quantization equals the standalone quantizer on the same row
        q2, d2 = sd.quantize_q8_act(y)
        assert np.array_equal(host(xq), host(q2)) and np.array_equal(host(xd), host(d2))


def test_swiglu_q8_parity_and_quantizer_consistency(sd):
    say("swiglu_q8")
    g = synth.rng(2400)
    for n, F in ((4, 14336), (1, 32), (16, 512)):
        gu = g.standard_normal((n, 2 * F), dtype=np.float32) * 4
        gu[0, :8] = [0.0, -0.0, 88.0, -88.0, 100.0, -100.0, 1e-30, -1e-30]
        xq, xd, y = sd.swiglu_q8(dev(gu), F, want_y=True)
        yh = host(y)
        ref = oracle.swiglu(gu[:, :F], gu[:, F:])
        assert np.all(np.abs(yh - ref) <= 8 * _ulp(ref) + 1e-37)
        q2, d2 = sd.quantize_q8_act(y)
        assert np.array_equal(host(xq), host(q2)) and np.array_equal(host(xd), host(d2))


def test_embed_and_argmax(sd):
    import torch
    say("embed + argmax")
    g = synth.rng(2500)
    table = g.standard_normal((1000, 256), dtype=np.float32).astype(np.float16)
    toks = np.array([0, 999, 17, 17], np.int32)
    x = host(sd.embed_f16(dev(table.view(np.uint16), torch.float16), dev(toks)))
    assert np.array_equal(bits(x), bits(table[toks].astype(np.float32)))
    logits = g.standard_normal((5, 151936), dtype=np.float32)
    logits[1, 5] = logits[1, 99] = logits[1, 151935] = 50.0   # ties -> lowest index
    logits[2, :] = -1.0
    logits[3, 151935] = 1e30
    got = host(sd.argmax_rows(dev(logits)))
    assert np.array_equal(got, oracle.argmax_rows(logits))
    assert got[1] == 5 and got[2] == 0 and got[3] == 151935


def test_stream_read_runs_and_writes_nothing(sd):
    """The streaming-read reference kernel reads a buffer (no output beyond the
    sink word it writes only for one magic fold value) and leaves the buffer
    untouched."""
    import torch
    say("stream read")
    buf = torch.arange(1 << 18, dtype=torch.int32, device="cuda")   # 1 MiB, fold != magic
    before = buf.clone()
    sink = torch.full((64,), 7, dtype=torch.int32, device="cuda")
    lib = sd._lib.load()
    import ctypes
    rc = lib.sd_hbm_stream_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * 4,
                                ctypes.c_void_p(sink.data_ptr()), None)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(buf, before) and torch.all(sink == 7)
