"""Oracle composition of one synthetic batched decode step (test infrastructure).

The step follows ds4 pull request 604, "2. Single-GPU decode batches don't
scale" and "Commit walkthrough / Graph driver": dense projections run once for
all sequences, the key/value append and the attention run per sequence, the
feed-forward and output head run on the batch, and the logits land one row per
sequence.  The pages define no model; the layer used here is the plain dense
pre-norm block with no biases:

    a  = rmsnorm(x) ; q, k, v = split(W_qkv a) ; q, k = rope(q, k, pos)  (last n_rot dims)
    cache[pos] = fp16(k), fp16(v) ; o = attention(q, cache[lo .. pos])  (lo = 0, or
                                                   pos - window + 1 with a window)
    h  = x + W_o o
    n  = rmsnorm(h) ; g, u = split(W_gate_up n) ; x' = h + W_down (silu(g) * u)

Every projection input is quantized to q8 activation blocks first (the consumer
of a q8_0 matmul is a quantized dot), and the final rmsnorm feeds the q8_0 LM
head, whose greedy argmax (lowest index on ties) is the next token.
"""
import numpy as np

import oracle as O


class Model:
    """Host copy of a synthetic model: fields mirror the library's model struct."""

    def __init__(self, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab, eps, theta,
                 tok_embd_bits, out_norm, w_lm, layers, n_rot=0, window=0):
        self.hidden, self.n_heads, self.n_kv_heads = hidden, n_heads, n_kv_heads
        self.head_dim, self.ffn, self.vocab = head_dim, ffn, vocab
        self.eps, self.theta = eps, theta
        self.n_rot = n_rot or head_dim        # rotated dims: the last n_rot of each head
        self.window = window                  # attention window in positions, 0 = none
        self.tok_embd_bits = tok_embd_bits    # uint16 [vocab][hidden]
        self.out_norm = out_norm              # fp32 [hidden]
        self.w_lm = w_lm                      # q8_0 blob [vocab][hidden]
        self.layers = layers                  # list of dicts (w_qkv, w_o, w_gu, w_down,
        #                                       attn_norm, ffn_norm)


def _quant_like(codes, x):
    """The new rows x in the cache type of `codes`: q4_0 nibble pairs (uint8),
    else q8_0 codes (int8)."""
    if codes.dtype == np.uint8:
        return O.quantize_kv_q4_0(x)
    return O.quantize_kv_q8_0(x)


def decode_step(m: Model, caches, tokens, pos):
    """One step for n = len(tokens) sequences.

    caches[s] = (k_bits, v_bits), each uint16 [n_layers][capacity][H_kv][D],
    or quantized caches (kq, kd_bits, vq, vd_bits) with codes int8 [..][D]
    (q8_0) or nibble pairs uint8 [..][D/2] (q4_0), K and V each either, and
    scale bits uint16 [..][D/32]; updated in place at row pos[s] of every layer.  Returns (logits [n][vocab]
    fp32, next tokens int32 [n]).
    """
    tokens = np.asarray(tokens, np.int64)
    pos = np.asarray(pos, np.int32)
    n = tokens.size
    H, Hq, Hkv, D, F = m.hidden, m.n_heads, m.n_kv_heads, m.head_dim, m.ffn
    scale = np.float32(1.0) / np.sqrt(np.float32(D))
    x = O.f16_decode(m.tok_embd_bits[tokens]).astype(np.float32)
    for li, L in enumerate(m.layers):
        a = O.rmsnorm(x, L["attn_norm"], m.eps)
        aq, ad = O.quantize_q8_act(a)
        qkv = O.qgemv_q8_0(L["w_qkv"], (Hq + 2 * Hkv) * D, H, aq, ad)
        q = qkv[:, :Hq * D].reshape(n, Hq, D)
        k = qkv[:, Hq * D:(Hq + Hkv) * D].reshape(n, Hkv, D)
        v = qkv[:, (Hq + Hkv) * D:].reshape(n, Hkv, D)
        q = O.rope_posvec(q, pos, m.theta, m.n_rot)
        k = O.rope_posvec(k, pos, m.theta, m.n_rot)
        for s in range(n):
            if len(caches[s]) == 4:  # quantized cache: codes and fp16 scales of the new rows
                kq, kd = _quant_like(caches[s][0], k[s])
                vq, vd = _quant_like(caches[s][2], v[s])
                caches[s][0][li, pos[s]], caches[s][1][li, pos[s]] = kq, kd
                caches[s][2][li, pos[s]], caches[s][3][li, pos[s]] = vq, vd
            else:
                caches[s][0][li, pos[s]] = O.f32_to_f16_bits(k[s])
                caches[s][1][li, pos[s]] = O.f32_to_f16_bits(v[s])
        o = O.attn_verify(q, [tuple(a[li] for a in c) for c in caches],
                          [int(p) + 1 for p in pos], [1] * n, scale, window=m.window)
        oq, od = O.quantize_q8_act(o.reshape(n, Hq * D))
        h = O.qgemv_q8_0(L["w_o"], H, Hq * D, oq, od, residual=x)
        nrm = O.rmsnorm(h, L["ffn_norm"], m.eps)
        nq, nd = O.quantize_q8_act(nrm)
        gu = O.qgemv_q8_0(L["w_gu"], 2 * F, H, nq, nd)
        mm = O.swiglu(gu[:, :F], gu[:, F:])
        mq, md = O.quantize_q8_act(mm)
        x = O.qgemv_q8_0(L["w_down"], H, F, mq, md, residual=h)
    xf = O.rmsnorm(x, m.out_norm, m.eps)
    fq, fd = O.quantize_q8_act(xf)
    logits = O.qgemv_q8_0(m.w_lm, m.vocab, H, fq, fd)
    return logits, O.argmax_rows(logits)
