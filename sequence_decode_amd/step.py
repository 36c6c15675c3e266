"""Device-side synthetic model and the sd_decode_step binding.

Holds the model's device tensors and the ctypes structs that point at them
(torch allocates; the library computes).  Weights either come from host arrays
(the seeded generator's output, for tests) or are drawn on the device (large
benchmark models).
"""
import ctypes

import numpy as np

from . import _lib, synth
from . import _check, _stream, kv_type_of


class DecodeModel:
    """A dense decoder in the library's layout (see sd_model in seqdecode.h)."""

    def __init__(self, dims, layers, tok_embd, out_norm, w_lm):
        import torch
        self.dims = dict(dims)
        self.layers = layers          # list of dicts of device tensors
        self.tok_embd = tok_embd      # float16 [vocab][hidden] (fp16 bits)
        self.out_norm = out_norm
        self.w_lm = w_lm
        d = self.dims
        self._lw = (_lib.LayerWeights * d["n_layers"])()
        for i, L in enumerate(layers):
            self._lw[i] = _lib.LayerWeights(L["w_qkv"].data_ptr(), L["w_o"].data_ptr(),
                                            L["w_gu"].data_ptr(), L["w_down"].data_ptr(),
                                            L["attn_norm"].data_ptr(), L["ffn_norm"].data_ptr())
        self.struct = _lib.Model(d["n_layers"], d["hidden"], d["n_heads"], d["n_kv_heads"],
                                 d["head_dim"], d["ffn"], d["vocab"], float(d["eps"]),
                                 float(d["theta"]), tok_embd.data_ptr(), out_norm.data_ptr(),
                                 w_lm.data_ptr(), ctypes.cast(self._lw, ctypes.c_void_p),
                                 int(d.get("n_rot", 0)), int(d.get("window", 0)))
        self.device = tok_embd.device
        del torch

    @property
    def weight_bytes(self) -> int:
        n = sum(t.numel() for L in self.layers for k, t in L.items() if k.startswith("w_"))
        return n + self.w_lm.numel()

    @classmethod
    def from_host(cls, h: dict, device="cuda"):
        import torch

        def dev(a, dtype=None):
            t = torch.from_numpy(np.ascontiguousarray(a))
            return t.to(device) if dtype is None else t.view(dtype).to(device)

        layers = []
        for L in h["layers"]:
            layers.append({k: dev(v) for k, v in L.items()})
        dims = {k: h[k] for k in ("n_layers", "hidden", "n_heads", "n_kv_heads", "head_dim",
                                  "ffn", "vocab", "eps", "theta")}
        dims.update({k: h[k] for k in ("n_rot", "window") if k in h})
        return cls(dims, layers, dev(h["tok_embd_bits"], torch.float16), dev(h["out_norm"]),
                   dev(h["w_lm"]))

    @classmethod
    def random_device(cls, seed: int, dims: dict, device="cuda"):
        """Same distributions as synth.model_host, drawn by torch on the device."""
        import torch
        g = torch.Generator(device=device)
        g.manual_seed(seed)
        H, Hq, Hkv, D, F, V = (dims[k] for k in ("hidden", "n_heads", "n_kv_heads", "head_dim",
                                                  "ffn", "vocab"))
        qkv_rows = (Hq + 2 * Hkv) * D

        def w(N, K):
            lo, hi = synth.unit_gain_scale_range(K)
            return synth.torch_q8_0_weights(g, N, K, device, lo, hi)

        def gamma(n):
            return torch.rand(n, device=device, generator=g) + 0.5

        layers = []
        for _ in range(dims["n_layers"]):
            layers.append({"w_qkv": w(qkv_rows, H), "w_o": w(H, Hq * D), "w_gu": w(2 * F, H),
                           "w_down": w(H, F), "attn_norm": gamma(H), "ffn_norm": gamma(H)})
        tok = synth.torch_normal_f16(g, (V, H), device)
        return cls(dims, layers, tok, gamma(H), w(V, H))


class SeqCache:
    """One sequence's caches, fp16 [n_layers][capacity][H_kv][D]."""

    def __init__(self, k, v):
        self.k, self.v = k, v
        self.capacity = k.shape[1]

    @classmethod
    def from_host(cls, k_bits, v_bits, device="cuda"):
        import torch
        return cls(torch.from_numpy(k_bits).view(torch.float16).to(device),
                   torch.from_numpy(v_bits).view(torch.float16).to(device))

    @classmethod
    def random_device(cls, gen, n_layers, capacity, H_kv, D, device="cuda"):
        return cls(synth.torch_normal_f16(gen, (n_layers, capacity, H_kv, D), device),
                   synth.torch_normal_f16(gen, (n_layers, capacity, H_kv, D), device))


class SeqCacheQ8:
    """One sequence's quantized caches: K and V codes each q8_0 (int8
    [n_layers][capacity][H_kv][D]) or q4_0 (nibble pairs, uint8
    [n_layers][capacity][H_kv][D/2]), the type told by the dtype, and fp16
    block scales kd, vd [n_layers][capacity][H_kv][D/32]."""

    def __init__(self, kq, kd, vq, vd):
        import torch
        self.kq, self.kd, self.vq, self.vd = kq, kd, vq, vd
        self.capacity = kq.shape[1]
        self.k_type = "q4_0" if kq.dtype == torch.uint8 else "q8_0"
        self.v_type = "q4_0" if vq.dtype == torch.uint8 else "q8_0"

    @classmethod
    def from_host(cls, kq, kd_bits, vq, vd_bits, device="cuda"):
        import torch
        t = lambda a: torch.from_numpy(a).to(device)
        f = lambda a: torch.from_numpy(a).view(torch.float16).to(device)
        return cls(t(kq), f(kd_bits), t(vq), f(vd_bits))

    @classmethod
    def random_device(cls, gen, n_layers, capacity, H_kv, D, device="cuda", k_type="q8_0",
                      v_type="q8_0"):
        """q8_0 halves: codes uniform in [-127, 127], scales those of N(0,1) blocks
        (about 2.5/127); q4_0 halves: nibbles uniform in 1..15, scales about 2.5/7."""
        import torch
        def codes(ty):
            if ty == "q4_0":
                n = lambda: torch.randint(1, 16, (n_layers, capacity, H_kv, D // 2), generator=gen,
                                          device=device, dtype=torch.int32)
                return (n() | (n() << 4)).to(torch.uint8)
            return torch.randint(-127, 128, (n_layers, capacity, H_kv, D), generator=gen,
                                 device=device, dtype=torch.int32).to(torch.int8)
        def scales(ty):
            u = torch.rand((n_layers, capacity, H_kv, D // 32), generator=gen, device=device)
            return ((u + 2.0) / (7.0 if ty == "q4_0" else 127.0)).to(torch.float16)
        return cls(codes(k_type), scales(k_type), codes(v_type), scales(v_type))


class StepRunner:
    """Preallocated inputs/outputs/workspace for repeated sd_decode_step calls.

    n_new[s] (default 1) is the number of tokens sequence s brings to each step
    (a verify step when above 1); token rows are packed by sequence.
    block_tables[s] (int32 device tensors, with block_size): the caches are a
    paged pool (the same SeqCache may serve several sequences) and sequence s
    keeps position j in row block_tables[s][j // block_size] * block_size
    + j % block_size of every layer."""

    def __init__(self, model: DecodeModel, caches, max_ctx: int, n_new=None, ring=False,
                 block_tables=None, block_size=0):
        import torch
        self.model = model
        self.caches = list(caches)
        n = len(self.caches)
        self.n_new = [1] * n if n_new is None else [int(t) for t in n_new]
        if len(self.n_new) != n:
            raise ValueError("one n_new entry per sequence")
        rows = sum(self.n_new)
        V = model.dims["vocab"]
        dev = model.device
        need = _lib.load().sd_decode_step_workspace_bytes(ctypes.byref(model.struct), rows, max_ctx)
        if need == 0:
            raise ValueError("model or batch not supported by sd_decode_step")
        self.ws = torch.zeros(need, dtype=torch.uint8, device=dev)
        self.logits = torch.empty((rows, V), dtype=torch.float32, device=dev)
        self.next_tokens = torch.empty(rows, dtype=torch.int32, device=dev)
        self.tokens = torch.zeros(rows, dtype=torch.int32, device=dev)
        self.positions = torch.zeros(rows, dtype=torch.int32, device=dev)
        self.block_tables = None if block_tables is None else list(block_tables)
        if self.block_tables is not None:
            if len(self.block_tables) != n:
                raise ValueError("one block table per sequence")
            for bt in self.block_tables:
                if bt.dtype != torch.int32 or not bt.is_cuda or not bt.is_contiguous():
                    raise TypeError("block tables must be contiguous int32 device tensors")
        self._seqs = (_lib.StepSeq * n)()
        for s, c in enumerate(self.caches):
            bt = 0 if self.block_tables is None else self.block_tables[s].data_ptr()
            if isinstance(c, SeqCacheQ8):
                self._seqs[s] = _lib.StepSeq(0, 0, c.capacity, 0, self.n_new[s], 1 if ring else 0, bt,
                                             int(block_size) if bt else 0,
                                             kv_type_of(c.k_type, c.v_type), c.kq.data_ptr(),
                                             c.vq.data_ptr(), c.kd.data_ptr(), c.vd.data_ptr())
            else:
                self._seqs[s] = _lib.StepSeq(c.k.data_ptr(), c.v.data_ptr(), c.capacity, 0,
                                             self.n_new[s], 1 if ring else 0, bt,
                                             int(block_size) if bt else 0, 0)
        self.io = _lib.StepIO(n, ctypes.cast(self._seqs, ctypes.c_void_p), self.tokens.data_ptr(),
                              self.positions.data_ptr(), self.logits.data_ptr(),
                              self.next_tokens.data_ptr(), self.ws.data_ptr(), need)

    def set_positions(self, pos):
        """Sets every sequence's first position this step (host structs and the
        device position of every token row)."""
        import torch
        rows = []
        for s, p in enumerate(pos):
            self._seqs[s].pos = int(p)
            rows += [int(p) + i for i in range(self.n_new[s])]
        self.positions.copy_(torch.tensor(rows, dtype=torch.int32))

    def advance(self):
        """One-token steps: moves every sequence one position on and feeds the
        greedy tokens back, without a host round trip (both updates are
        enqueued on the stream)."""
        if any(t != 1 for t in self.n_new):
            raise ValueError("advance() is for one-token steps")
        for s in range(len(self.caches)):
            self._seqs[s].pos += 1
        self.positions.add_(1)
        self.tokens.copy_(self.next_tokens)

    def step(self, stream=None):
        """Enqueues one step reading self.tokens / positions (already on device)."""
        _check("sd_decode_step", _lib.load().sd_decode_step(
            ctypes.byref(self.model.struct), ctypes.byref(self.io), _stream(stream)))
