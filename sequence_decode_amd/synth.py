"""Seeded synthetic inputs shared by the HIP path's tests and the oracle.

This module only draws random numbers and lays them out in the documented
input formats; it holds none of the method's arithmetic.  Distributions:

* q8_0 weights: int8 codes uniform on {-127, ..., 127}; one fp16 scale per
  block of 32, drawn in fp64 uniform on [lo, hi] and rounded to fp16 (RNE).
  A row of K weights is K/32 consecutive 34-byte blocks: 2 bytes of scale
  (little-endian fp16 bits) followed by the 32 codes.
* activations: fp32 standard normal.
* K/V caches: fp32 standard normal rounded to fp16 (RNE), layout
  [capacity][H_kv][D].
* q8_0 K/V caches: int8 codes uniform on {-127, ..., 127}, layout
  [capacity][H_kv][D]; one fp16 scale per 32 dims, drawn uniform on
  [2/127, 3/127] (the scale of a block of N(0,1) values, whose maximum of 32 is
  about 2 to 3) and rounded to fp16, layout [capacity][H_kv][D/32].
* queries: fp32 standard normal.

Host generators use numpy's PCG64; the device generators (large benchmark
inputs) use torch's generator on the GPU with the same distributions.
"""
import numpy as np

BLOCK = 32
BLOCK_BYTES = 34


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def pack_q8_0(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Lays out codes int8 [N][K] and fp16 scale bits uint16 [N][K/32] as q8_0 bytes."""
    N, K = codes.shape
    nb = K // BLOCK
    assert scale_bits.shape == (N, nb)
    out = np.empty((N, nb, BLOCK_BYTES), np.uint8)
    out[:, :, 0:2] = scale_bits.astype("<u2").view(np.uint8).reshape(N, nb, 2)
    out[:, :, 2:] = codes.reshape(N, nb, BLOCK).view(np.uint8)
    return out.reshape(-1)


def q8_0_weights(g: np.random.Generator, N: int, K: int, lo: float = 1e-3, hi: float = 1e-2):
    """Returns (blob uint8 [N*(K/32)*34], codes int8 [N][K], scale_bits uint16 [N][K/32])."""
    assert K % BLOCK == 0
    codes = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    scales = g.uniform(lo, hi, size=(N, K // BLOCK))
    scale_bits = scales.astype(np.float16).view(np.uint16)
    return pack_q8_0(codes, scale_bits), codes, scale_bits


def activations(g: np.random.Generator, n_tok: int, K: int) -> np.ndarray:
    return g.standard_normal(size=(n_tok, K), dtype=np.float32)


def kv_cache(g: np.random.Generator, capacity: int, H_kv: int, D: int) -> np.ndarray:
    """fp16 bit patterns [capacity][H_kv][D] of N(0,1) values."""
    x = g.standard_normal(size=(capacity, H_kv, D), dtype=np.float32)
    return x.astype(np.float16).view(np.uint16)


def kv_cache_q8(g: np.random.Generator, capacity: int, H_kv: int, D: int):
    """(codes int8 [capacity][H_kv][D], fp16 scale bits [capacity][H_kv][D/32])."""
    codes = g.integers(-127, 128, size=(capacity, H_kv, D), dtype=np.int8)
    d = g.uniform(2.0 / 127.0, 3.0 / 127.0, size=(capacity, H_kv, D // BLOCK))
    return codes, d.astype(np.float16).view(np.uint16)


def kv_cache_q4(g: np.random.Generator, capacity: int, H_kv: int, D: int):
    """(nibble pairs uint8 [capacity][H_kv][D/2], fp16 scale bits
    [capacity][H_kv][D/32]): nibbles uniform on 1..15 (codes -7..7), scales
    those of N(0,1) blocks under amax / 7."""
    packed = g.integers(1, 16, size=(capacity, H_kv, D // 2), dtype=np.uint8)
    packed |= g.integers(1, 16, size=(capacity, H_kv, D // 2), dtype=np.uint8) << 4
    d = g.uniform(2.0 / 7.0, 3.0 / 7.0, size=(capacity, H_kv, D // BLOCK))
    return packed, d.astype(np.float16).view(np.uint16)


def queries(g: np.random.Generator, n_seq: int, H_q: int, D: int) -> np.ndarray:
    return g.standard_normal(size=(n_seq, H_q, D), dtype=np.float32)


def uniform_f32(g: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    return g.uniform(lo, hi, size=shape).astype(np.float32)


# ---------------------------------------------------------------- device side

def torch_q8_0_weights(gen, N: int, K: int, device, lo: float = 1e-3, hi: float = 1e-2):
    """Device q8_0 blob (uint8 tensor) with the same distributions, drawn by torch."""
    import torch
    nb = K // BLOCK
    out = torch.empty((N, nb, BLOCK_BYTES), dtype=torch.uint8, device=device)
    chunk = max(1, (1 << 26) // (nb * BLOCK_BYTES))  # ~64 MB of output per piece
    for r0 in range(0, N, chunk):
        r1 = min(N, r0 + chunk)
        codes = torch.randint(-127, 128, (r1 - r0, nb, BLOCK), dtype=torch.int8,
                              device=device, generator=gen)
        sc = torch.rand((r1 - r0, nb), dtype=torch.float64, device=device, generator=gen)
        sc = (sc * (hi - lo) + lo).to(torch.float16)
        out[r0:r1, :, 0:2] = sc.view(torch.uint8).view(r1 - r0, nb, 2)
        out[r0:r1, :, 2:] = codes.view(torch.uint8)
    return out.reshape(-1)


def torch_normal_f16(gen, shape, device):
    import torch
    return torch.randn(shape, dtype=torch.float32, device=device, generator=gen).to(torch.float16)


# ------------------------------------------------------------ synthetic model

def unit_gain_scale_range(K: int):
    """Scale range giving a q8_0 projection of fan-in K roughly unit gain.

    Codes uniform on +-127 have standard deviation ~73.3, so a scale near
    1/(73.3 sqrt(K)) keeps the output of a unit-RMS input near unit RMS.
    """
    c = 1.0 / (73.3 * np.sqrt(K))
    return 0.5 * c, 1.5 * c


def model_host(seed: int, n_layers: int, hidden: int, n_heads: int, n_kv_heads: int,
               head_dim: int, ffn: int, vocab: int):
    """Random-init dense model as host arrays (dict); layout matches the library's.

    Per layer: w_qkv [(Hq+2Hkv)D][hidden] (q rows, then k rows, then v rows),
    w_o [hidden][Hq D], w_gu [2 ffn][hidden] (gate rows, then up rows),
    w_down [hidden][ffn], all q8_0; attn_norm and ffn_norm fp32 uniform
    [0.5, 1.5].  tok_embd fp16 N(0,1) bits [vocab][hidden], out_norm fp32,
    w_lm q8_0 [vocab][hidden].
    """
    g = rng(seed)
    qkv_rows = (n_heads + 2 * n_kv_heads) * head_dim
    layers = []
    for _ in range(n_layers):
        L = {}
        L["w_qkv"] = q8_0_weights(g, qkv_rows, hidden, *unit_gain_scale_range(hidden))[0]
        L["w_o"] = q8_0_weights(g, hidden, n_heads * head_dim,
                                *unit_gain_scale_range(n_heads * head_dim))[0]
        L["w_gu"] = q8_0_weights(g, 2 * ffn, hidden, *unit_gain_scale_range(hidden))[0]
        L["w_down"] = q8_0_weights(g, hidden, ffn, *unit_gain_scale_range(ffn))[0]
        L["attn_norm"] = uniform_f32(g, hidden, 0.5, 1.5)
        L["ffn_norm"] = uniform_f32(g, hidden, 0.5, 1.5)
        layers.append(L)
    tok = g.standard_normal(size=(vocab, hidden), dtype=np.float32).astype(np.float16)
    return {
        "n_layers": n_layers, "hidden": hidden, "n_heads": n_heads,
        "n_kv_heads": n_kv_heads, "head_dim": head_dim, "ffn": ffn, "vocab": vocab,
        "eps": 1e-6, "theta": 1e6,
        "tok_embd_bits": tok.view(np.uint16),
        "out_norm": uniform_f32(g, hidden, 0.5, 1.5),
        "w_lm": q8_0_weights(g, vocab, hidden, *unit_gain_scale_range(hidden))[0],
        "layers": layers,
    }


def prefilled_cache(g: np.random.Generator, n_layers: int, capacity: int, n_kv_heads: int,
                    head_dim: int):
    """(k, v) fp16 bits [n_layers][capacity][H_kv][D], every row N(0,1).

    Rows below a sequence's position stand for its earlier context; the step
    overwrites the row at the position itself.
    """
    k = np.stack([kv_cache(g, capacity, n_kv_heads, head_dim) for _ in range(n_layers)])
    v = np.stack([kv_cache(g, capacity, n_kv_heads, head_dim) for _ in range(n_layers)])
    return k, v
