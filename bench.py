#!/usr/bin/env python3
"""Benchmark of the batch-invariant multi-sequence decode step on one MI355X.

Headline (one JSON line on stdout): q8_0 narrow-batch GEMV throughput in GB/s
over the 8B-class decode projections -- 32 layers of QKV 4096->6144, O
4096->4096, gate|up 4096->2x14336 (one fused matrix), down 14336->4096, q8_0
weights with fp16 scales uniform[1e-3, 1e-2], fp32 N(0,1) activations
quantized per token -- at n_tok = 4.  A step is one sweep over one batch of
n_tok synthetic activation rows: quantize them (once for the 4096-wide input
of QKV, O and gate|up, once for the 14336-wide input of down), then the 128
GEMVs of the 32 layers (7.42 GB of weights, far beyond the 256 MB Infinity
Cache).  The timed steps replay a HIP graph of the sweep, so the host's launch
rate does not limit the GPU; the headline is the median of 5 repeats of the
timed steps.  Inputs are resident in HBM before timing starts.

Also reported: the sweep at n_tok = 1..4 (medians of 5); the single 4096x4096
GEMV over 64 rotated weight copies at n_tok 1..4; a plain streaming read of
the same sizes (the achievable-bandwidth reference); the widened verify batch
at n_tok = 8, 12, 16 on the v_dot4 kernels and on the matrix-core kernel (with
a bitwise comparison of the two); the dominant kernel's roofline (per-launch
HIP-event durations of every GEMV in an eager pass of the same sweep, and the
committed rocprofv3 trace's durations of the same launches); attention per
call; the aggregate tokens/s of the full synthetic decode step for 1..4
sequences (8 warmups, 64 timed steps, median of 3 fresh child processes
started before this process touches the GPU), plus verify, paged, q8_0-cache
and serial variants; and the CPU oracle on bounded samples of the same
workloads (GEMV GB/s, one attention call, one decode step per sequence count).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "q8_0 narrow-batch GEMV GB/s (%HBM peak) n_tok 1-4; aggregate decode tok/s"
SHAPES = [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336)]
N_LAYERS = 32


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def profile_fields():
    """Fields of the committed rocprofv3 summary of the GEMV sweep, if it was
    taken on the kernel source that is built now (else {})."""
    import hashlib
    prof = os.path.join(ROOT, "profiles", "qgemv_q8_0_sweep_ntok1-4.md")
    src = os.path.join(ROOT, "sequence_decode_amd", "csrc", "qgemv.hip")
    try:
        fields = dict(line.split(": ", 1) for line in open(prof).read().splitlines()
                      if ": " in line and line.split(": ", 1)[0] in (
                          "traffic_bytes_per_launch", "kernel_source_sha256", "trace_avg_us_per_launch",
                          "trace_launches"))
        sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
        if fields.get("kernel_source_sha256", "").strip() != sha:
            return {}
        return {k: v.strip() for k, v in fields.items()}
    except (OSError, ValueError):
        return {}


def gemv_bytes(N, K, n_tok):
    """Algorithmic bytes of one launch: weights once, q8 activations, fp32 outputs."""
    return N * (K // 32) * 34 + n_tok * (K + 4 * (K // 32)) + 4 * n_tok * N


class Sweep:
    def __init__(self, sd, torch, seed, max_tok):
        from sequence_decode_amd import synth
        self.sd, self.torch = sd, torch
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.w = [{name: synth.torch_q8_0_weights(g, N, K, "cuda") for name, N, K in SHAPES}
                  for _ in range(N_LAYERS)]
        self.x = torch.randn((max_tok, 14336), dtype=torch.float32, device="cuda", generator=g)
        self.xq = {K: torch.empty((max_tok, K), dtype=torch.int8, device="cuda") for K in (4096, 14336)}
        self.xd = {K: torch.empty((max_tok, K // 32), dtype=torch.float32, device="cuda")
                   for K in (4096, 14336)}
        self.y = {name: torch.empty((max_tok, N), dtype=torch.float32, device="cuda")
                  for name, N, K in SHAPES}
        self.weight_bytes = sum(N * (K // 32) * 34 for _, N, K in SHAPES) * N_LAYERS

    def step(self, n_tok, path=None):
        """One sweep; path=None uses sd_qgemv_q8_0_batch, else the kernel that
        sd_qgemv_q8_0_batch_path picks for that path."""
        sd, lib = self.sd, self.sd._lib.load()
        import ctypes
        st = ctypes.c_void_p(self.torch.cuda.current_stream().cuda_stream)
        P = ctypes.c_void_p
        for K in (4096, 14336):
            rc = lib.sd_quantize_q8_act(P(self.x.data_ptr()), 14336, n_tok, K,
                                        P(self.xq[K].data_ptr()), P(self.xd[K].data_ptr()), st)
            if rc:
                raise sd.SdError("sd_quantize_q8_act", rc)
        for L in self.w:
            for name, N, K in SHAPES:
                xq, xd = self.xq[K], self.xd[K]
                y = self.y[name]
                if path is None:
                    rc = lib.sd_qgemv_q8_0_batch(P(L[name].data_ptr()), N, K, P(xq.data_ptr()),
                                                 P(xd.data_ptr()), n_tok, None, P(y.data_ptr()), N, st)
                else:
                    rc = lib.sd_qgemv_q8_0_batch_path(P(L[name].data_ptr()), N, K, P(xq.data_ptr()),
                                                      P(xd.data_ptr()), n_tok, None, P(y.data_ptr()), N,
                                                      path, st)
                if rc:
                    raise sd.SdError("sd_qgemv_q8_0_batch", rc)

    def bytes_per_step(self, n_tok):
        return sum(gemv_bytes(N, K, n_tok) for _, N, K in SHAPES) * N_LAYERS


def time_graph(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g.capture_begin()
        fn()
        g.capture_end()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    del g
    return dt / steps


# launches of each shape's 32 matrices before the timed ones in the roofline
# pass: one eager round, one graph replay
ROOF_WARM_ROUNDS = 2
# timed replays per shape
ROOF_REPS = 4


def roofline_pass(torch, sweep, n_tok, reps):
    """Average duration of the GEMV kernel per shape: the shape's 32 matrices
    launched back to back as one HIP graph (as the sweep runs them), replayed
    `reps` times between HIP events on the graph's stream (nothing else in
    between), so each average is one kernel's duration plus the dispatch gap to
    the next launch of the same kernel."""
    import ctypes
    lib = sweep.sd._lib.load()
    P = ctypes.c_void_p
    per = {}
    tot_bytes, tot_ms, launches = 0, 0.0, 0
    s = torch.cuda.Stream()
    for name, N, K in SHAPES:
        xq, xd, y = sweep.xq[K], sweep.xd[K], sweep.y[name]
        def run():
            st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for L in sweep.w:
                rc = lib.sd_qgemv_q8_0_batch(P(L[name].data_ptr()), N, K, P(xq.data_ptr()), P(xd.data_ptr()),
                                             n_tok, None, P(y.data_ptr()), N, st)
                if rc:
                    raise sweep.sd.SdError("sd_qgemv_q8_0_batch", rc)
        run()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            g.capture_begin()
            run()
            g.capture_end()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):
            g.replay()
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
        torch.cuda.synchronize()
        del g
        ms = e0.elapsed_time(e1)
        n = reps * len(sweep.w)
        b = gemv_bytes(N, K, n_tok) * n
        per[name] = {"GB_s": round(b / (ms / 1e3) / 1e9, 1), "avg_us": round(ms / n * 1e3, 3),
                     "bytes_per_launch": gemv_bytes(N, K, n_tok), "launches": n}
        tot_bytes += b
        tot_ms += ms
        launches += n
    return tot_bytes, tot_ms, launches, per


def verify_widths(torch, sweep, steps):
    """The widened verify batch (n_tok 8, 12, 16) on the same 32-layer sweep:
    GB/s of the v_dot4 kernels and of the matrix-core kernel, and whether the
    two give bitwise the same outputs."""
    from sequence_decode_amd import GEMV_NARROW, GEMV_MFMA
    out = {}
    for n in (8, 12, 16):
        row = {}
        ys = {}
        for label, path in (("narrow", GEMV_NARROW), ("mfma", GEMV_MFMA)):
            dt = time_graph(torch, lambda: sweep.step(n, path), steps, 2)
            gbs = sweep.bytes_per_step(n) / dt / 1e9
            row[label] = {"GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                          "ms_per_step": round(dt * 1e3, 4)}
            sweep.step(n, path)
            torch.cuda.synchronize()
            ys[label] = {name: sweep.y[name][:n].clone() for name, _, _ in SHAPES}
        row["bitwise_equal"] = all(torch.equal(ys["narrow"][k].view(torch.int32), ys["mfma"][k].view(torch.int32))
                                   for k in ys["narrow"])
        row["mfma_speedup"] = round(row["mfma"]["GB_s"] / row["narrow"]["GB_s"], 3)
        out[str(n)] = row
        log(f"verify width n_tok={n}: narrow {row['narrow']['GB_s']} GB/s, mfma {row['mfma']['GB_s']} GB/s, "
            f"bitwise equal {row['bitwise_equal']}")
    return out


def cpu_baseline(torch, sweep, n_tok, budget_s):
    """The oracle's GEMV on host copies of the sweep's matrices: GB/s of
    algorithmic bytes on all the threads OpenMP gives it (budget_s of oracle
    time), and on one thread (a quarter of that budget)."""
    import oracle
    x = sweep.x[:n_tok].cpu().numpy()
    host = []  # host copies of the layers already visited (copies are not timed)

    def run(budget):
        done_bytes, t_used, layers = 0, 0.0, 0
        while t_used < budget:
            for li, L in enumerate(sweep.w):
                if li == len(host):
                    host.append({name: L[name].cpu().numpy() for name, _, _ in SHAPES})
                for name, N, K in SHAPES:
                    q, d = oracle.quantize_q8_act(x[:, :K])
                    t0 = time.perf_counter()
                    oracle.qgemv_q8_0(host[li][name], N, K, q, d)
                    t_used += time.perf_counter() - t0
                    done_bytes += gemv_bytes(N, K, n_tok)
                layers += 1
                if t_used >= budget:
                    break
        return done_bytes, t_used, layers

    cores = oracle.num_threads()
    b_all, t_all, l_all = run(budget_s)
    oracle.set_num_threads(1)
    try:
        b_one, t_one, l_one = run(budget_s / 4)
    finally:
        oracle.set_num_threads(cores)
    return {"value": round(b_all / t_all / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"{l_all} layer passes over the 32 layers (4 projections each) at "
                      f"n_tok={n_tok}, {b_all / 1e9:.2f} GB of weights, {t_all:.1f} s",
            "single_core": {"value": round(b_one / t_one / 1e9, 3), "unit": "GB/s", "cores": 1,
                            "sample": f"{l_one} layer passes, {b_one / 1e9:.2f} GB of weights, "
                                      f"{t_one:.1f} s"}}


def decode_bench(torch, steps, warmup):
    """Verify, paged, q8_0-cache and serial variants of the full step (one
    process; the plain decode tok/s come from decode_children)."""
    from sequence_decode_amd.step import DecodeModel, SeqCache, StepRunner
    dims = DECODE_DIMS
    model = DecodeModel.random_device(11, dims)
    ragged = RAGGED
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    span = warmup + steps + 4
    caches = [SeqCache.random_device(g, 32, ctx + span, 8, 128) for ctx in ragged]
    res = {}
    # verify steps: every sequence brings n_new proposed tokens (causal within the burst);
    # the same positions are re-verified each timed step
    for label, ctxs in (("ragged", ragged), ("ctx2050", [2050] * 4)):
        for T in (2, 4):
            r = StepRunner(model, caches, max_ctx=max(ctxs) + span, n_new=[T] * 4)
            r.tokens.copy_(torch.arange(4 * T, dtype=torch.int32) + 7)
            r.set_positions([c - 1 for c in ctxs])
            for _ in range(warmup):
                r.step()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                r.step()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / steps
            res[f"verify_{label}_n4_t{T}"] = {"tok_s": round(4 * T / dt, 2), "ms_per_step": round(dt * 1e3, 3),
                                              "rows": 4 * T}
            log(f"verify step {label} 4 sequences x {T} tokens: {4 * T / dt:.1f} tok/s ({dt * 1e3:.3f} ms/step)")
    # paged pool: the four ragged sequences in one shared pool of 64-row blocks at
    # shuffled places (block-table lookup in the append and attention kernels)
    bs = 64
    nb = [(c + span + bs - 1) // bs for c in ragged]
    place = torch.randperm(sum(nb), generator=g, device="cuda").to(torch.int32)
    tables = [place[sum(nb[:s]):sum(nb[:s + 1])].contiguous() for s in range(4)]
    pool = SeqCache.random_device(g, 32, sum(nb) * bs, 8, 128)
    r = StepRunner(model, [pool] * 4, max_ctx=max(ragged) + span, block_tables=tables, block_size=bs)
    r.tokens.copy_(torch.arange(4, dtype=torch.int32) + 7)
    r.set_positions([c - 1 for c in ragged])
    for _ in range(warmup):
        r.step()
        r.advance()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
        r.advance()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    res["paged64_ragged_n4"] = {"tok_s": round(4 / dt, 2), "ms_per_step": round(dt * 1e3, 3)}
    log(f"decode paged (64-row blocks) ragged n_seq=4: {4 / dt:.1f} tok/s ({dt * 1e3:.3f} ms/step)")
    del r, pool
    # q8_0 KV caches (int8 codes, fp16 scale per 32 dims) for the ragged contexts
    from sequence_decode_amd.step import SeqCacheQ8
    q8c = [SeqCacheQ8.random_device(g, 32, ctx + span, 8, 128) for ctx in ragged]
    for n in (1, 4):
        r = StepRunner(model, q8c[:n], max_ctx=max(ragged[:n]) + span)
        r.tokens.copy_(torch.arange(n, dtype=torch.int32) + 7)
        r.set_positions([c - 1 for c in ragged[:n]])
        for _ in range(warmup):
            r.step()
            r.advance()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            r.step()
            r.advance()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        res[f"q8kv_ragged_n{n}"] = {"tok_s": round(n / dt, 2), "ms_per_step": round(dt * 1e3, 3)}
        log(f"decode q8_0 KV ragged n_seq={n}: {n / dt:.1f} tok/s ({dt * 1e3:.3f} ms/step)")
    del r, q8c
    # mixed Q4/Q8 KV caches (K q4_0, V q8_0) for the four ragged contexts
    q48 = [SeqCacheQ8.random_device(g, 32, ctx + span, 8, 128, k_type="q4_0") for ctx in ragged]
    r = StepRunner(model, q48, max_ctx=max(ragged) + span)
    r.tokens.copy_(torch.arange(4, dtype=torch.int32) + 7)
    r.set_positions([c - 1 for c in ragged])
    for _ in range(warmup):
        r.step()
        r.advance()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
        r.advance()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    res["q4q8kv_ragged_n4"] = {"tok_s": round(4 / dt, 2), "ms_per_step": round(dt * 1e3, 3)}
    log(f"decode Q4/Q8 KV ragged n_seq=4: {4 / dt:.1f} tok/s ({dt * 1e3:.3f} ms/step)")
    del r, q48
    # serial baseline: the four ragged sequences one at a time (one-token steps back to back)
    runners = [StepRunner(model, [caches[s]], max_ctx=ragged[s] + span) for s in range(4)]
    for s in range(4):
        runners[s].set_positions([ragged[s] - 1])
    for _ in range(2):
        for s in range(4):
            runners[s].step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        for s in range(4):
            runners[s].step()
            runners[s].advance()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    res["serial_ragged_n4"] = {"tok_s": round(4 / dt, 2), "ms_per_round": round(dt * 1e3, 3)}
    log(f"decode serial 4 sequences: {4 / dt:.1f} tok/s")
    return res


def launch_floor_us(torch, n=64):
    """Time per kernel of a graph of n one-element kernels back to back (no host
    work between them): the per-dispatch floor that every launch pays here."""
    x = torch.zeros(1, device="cuda")

    def run():
        for _ in range(n):
            x.add_(1.0)
    return time_graph(torch, run, 20, 2) * 1e6 / n


# cache kinds of the attention pass: fp16, q8_0, the mixed Q4/Q8 and Q8/Q4
# types (K type first), fp16 in a paged pool
ATTN_KINDS = ("f16", "q8_0", "q4_q8", "q8_q4", "f16_paged64")


def attn_key_bytes(kind):
    """Cache bytes per position (8 KV heads of 128 dims, K and V): fp16 2 B per
    value; a q8_0 half 128 + 8 B per head, a q4_0 half 64 + 8 B."""
    half = {"q8": 8 * (128 + 8), "q4": 8 * (64 + 8)}
    if kind in ("q4_q8", "q8_q4"):
        return half[kind[:2]] + half[kind[3:]]
    return 2 * half["q8"] if kind == "q8_0" else 4096


def attn_sets(lens, kind):
    """Cache sets the attention pass cycles through: at least 4, and enough that
    together they exceed 512 MB (at most 64)."""
    per_key = attn_key_bytes(kind)
    set_bytes = sum(lens) * per_key
    return min(64, max(4, -(-512 * 2**20 // set_bytes)))


def attention_bench(torch, reps=20):
    """Graph-timed sd_decode_attn_multiseq (chunk + combine kernels) at the decode
    contexts: fp16, q8_0 and mixed Q4/Q8, Q8/Q4 caches, and fp16 in a paged pool
    (64-row blocks).  GB/s counts the cache bytes the call must read."""
    import sequence_decode_amd as sd
    g = torch.Generator(device="cuda")
    g.manual_seed(21)
    H_q, H_kv, D = 32, 8, 128
    cases = {"n1_2050": [2050], "n4_2050": [2050] * 4, "n4_ragged": [2050, 3072, 16384, 32768],
             "n1_32768": [32768]}
    out = {}
    for cname, lens in cases.items():
        for kind in ATTN_KINDS:
            keep, sets = [], []
            # cache sets, cycled, enough of them to exceed twice the 256 MB
            # Infinity Cache: like a decode step (which reads the rest of the
            # model between two reads of a layer's cache), no call finds its
            # cache in any cache level
            n_sets = attn_sets(lens, kind)
            def half(ty, L):
                """Codes and fp16 scales of one quantized half ("q8" or "q4")."""
                if ty == "q8":
                    c = torch.randint(-127, 128, (L, H_kv, D), generator=g, device="cuda",
                                      dtype=torch.int32).to(torch.int8)
                    d = ((torch.rand((L, H_kv, D // 32), generator=g, device="cuda") + 2) / 127).half()
                else:
                    lo = torch.randint(1, 16, (L, H_kv, D // 2), generator=g, device="cuda", dtype=torch.int32)
                    hi = torch.randint(1, 16, (L, H_kv, D // 2), generator=g, device="cuda", dtype=torch.int32)
                    c = (lo | (hi << 4)).to(torch.uint8)
                    d = ((torch.rand((L, H_kv, D // 32), generator=g, device="cuda") + 2) / 7).half()
                return c, d
            for _ in range(n_sets):
                if kind in ("q4_q8", "q8_q4"):
                    cs = []
                    for L in lens:
                        kq, kd = half(kind[:2], L)
                        vq, vd = half(kind[3:], L)
                        cs.append((kq, kd, vq, vd))
                    types = {"q8": "q8_0", "q4": "q4_0"}
                    views = [sd.seqview_quant(*c, L, types[kind[:2]], types[kind[3:]]) for c, L in zip(cs, lens)]
                elif kind == "q8_0":
                    cs = []
                    for L in lens:
                        kq = torch.randint(-127, 128, (L, H_kv, D), generator=g, device="cuda",
                                           dtype=torch.int32).to(torch.int8)
                        vq = torch.randint(-127, 128, (L, H_kv, D), generator=g, device="cuda",
                                           dtype=torch.int32).to(torch.int8)
                        kd = ((torch.rand((L, H_kv, D // 32), generator=g, device="cuda") + 2) / 127).half()
                        vd = ((torch.rand((L, H_kv, D // 32), generator=g, device="cuda") + 2) / 127).half()
                        cs.append((kq, kd, vq, vd))
                    views = [sd.seqview_q8(*c, L) for c, L in zip(cs, lens)]
                elif kind == "f16":
                    cs = [(torch.randn((L, H_kv, D), generator=g, device="cuda").half(),
                           torch.randn((L, H_kv, D), generator=g, device="cuda").half()) for L in lens]
                    views = [sd.seqview(k, v, L) for (k, v), L in zip(cs, lens)]
                else:
                    bs = 64
                    nb = [(L + bs - 1) // bs for L in lens]
                    pk = torch.randn((sum(nb) * bs, H_kv, D), generator=g, device="cuda").half()
                    pv = torch.randn((sum(nb) * bs, H_kv, D), generator=g, device="cuda").half()
                    place = torch.randperm(sum(nb), generator=g, device="cuda").to(torch.int32)
                    tabs = [place[sum(nb[:i]):sum(nb[:i + 1])].contiguous() for i in range(len(lens))]
                    cs = [pk, pv, tabs]
                    views = [sd.seqview(pk, pv, L, block_table=t, block_size=bs)
                             for t, L in zip(tabs, lens)]
                keep.append(cs)
                sets.append(views)
            q = torch.randn((len(lens), H_q, D), generator=g, device="cuda")
            o = torch.empty_like(q)
            ws = torch.zeros(max(16, sd.decode_attn_workspace_bytes(sets[0], H_q, D)),
                             dtype=torch.uint8, device="cuda")
            def cycle():  # one call per cache set, captured in one graph
                for v in sets:
                    sd.decode_attn_multiseq(q, v, H_kv, 0.08838835, out=o, ws=ws)
            us = time_graph(torch, cycle, reps, 2) * 1e6 / n_sets
            gbs = sum(lens) * attn_key_bytes(kind) / us / 1e3
            out[f"{cname}_{kind}"] = {"us": round(us, 2), "GB_s": round(gbs, 1),
                                      "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                                      "cache_sets": n_sets}
            log(f"attention {cname} {kind}: {us:.2f} us, {gbs:.1f} GB/s of cache bytes")
            del keep, sets
            torch.cuda.empty_cache()
    return out


def step_only(torch, n_seq, steps, warmup):
    """Decode steps of n_seq sequences at the ragged contexts {2050, 3072, 16384,
    32768}[:n_seq] and nothing else: the run a kernel trace of one step's
    kernels is taken on (per-kernel totals / (warmup + steps) = one step)."""
    from sequence_decode_amd.step import DecodeModel, SeqCache, StepRunner
    dims = dict(n_layers=32, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                vocab=151936, eps=1e-6, theta=1e6)
    model = DecodeModel.random_device(11, dims)
    ctxs = [2050, 3072, 16384, 32768][:n_seq]
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    span = warmup + steps + 4
    caches = [SeqCache.random_device(g, 32, ctx + span, 8, 128) for ctx in ctxs]
    r = StepRunner(model, caches, max_ctx=max(ctxs) + span)
    r.tokens.copy_(torch.arange(n_seq, dtype=torch.int32) + 7)
    r.set_positions([c - 1 for c in ctxs])
    for _ in range(warmup):
        r.step()
        r.advance()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        r.step()
        r.advance()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    log(f"decode ragged n_seq={n_seq}: {n_seq / dt:.1f} tok/s ({dt * 1e3:.3f} ms/step), "
        f"{warmup + steps} steps in the run")
    return {"step_only": {"n_seq": n_seq, "contexts": ctxs, "tok_s": round(n_seq / dt, 2),
                          "ms_per_step": round(dt * 1e3, 3), "steps_in_run": warmup + steps}}


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def sweep_median(torch, sweep, n, steps, warmup, repeats=5):
    """Median over `repeats` graph-timed runs of `steps` sweeps (seconds per sweep)."""
    runs = [time_graph(torch, lambda: sweep.step(n), steps, warmup) for _ in range(repeats)]
    return median(runs), runs


def config1_rotated(torch, sd, steps, repeats=5):
    """The single 4096x4096 q8_0 GEMV over 64 distinct weight copies (1.14 GB,
    beyond the 256 MB Infinity Cache) launched round robin, at n_tok 1..4:
    GB/s of algorithmic bytes, median of `repeats` graph-timed runs."""
    import ctypes
    from sequence_decode_amd import synth
    lib = sd._lib.load()
    g = torch.Generator(device="cuda")
    g.manual_seed(2)
    N = K = 4096
    copies = [synth.torch_q8_0_weights(g, N, K, "cuda") for _ in range(64)]
    x = torch.randn((4, K), dtype=torch.float32, device="cuda", generator=g)
    xq = torch.empty((4, K), dtype=torch.int8, device="cuda")
    xd = torch.empty((4, K // 32), dtype=torch.float32, device="cuda")
    y = torch.empty((4, N), dtype=torch.float32, device="cuda")
    P = ctypes.c_void_p
    out = {}
    for n in (1, 2, 3, 4):
        def run():
            st = P(torch.cuda.current_stream().cuda_stream)
            lib.sd_quantize_q8_act(P(x.data_ptr()), K, n, K, P(xq.data_ptr()), P(xd.data_ptr()), st)
            for w in copies:
                rc = lib.sd_qgemv_q8_0_batch(P(w.data_ptr()), N, K, P(xq.data_ptr()), P(xd.data_ptr()), n, None,
                                             P(y.data_ptr()), N, st)
                if rc:
                    raise sd.SdError("sd_qgemv_q8_0_batch", rc)
        runs = [time_graph(torch, run, steps, 2) for _ in range(repeats)]
        dt = median(runs) / len(copies)
        b = gemv_bytes(N, K, n)
        out[str(n)] = {"GB_s": round(b / dt / 1e9, 1), "frac_hbm_peak": round(b / dt / 1e9 / HBM_PEAK_GBS, 4),
                       "us_per_gemv": round(dt * 1e6, 3), "weight_copies": len(copies), "repeats": repeats}
        log(f"4096x4096 GEMV over 64 rotated copies, n_tok={n}: {b / dt / 1e9:.1f} GB/s ({dt * 1e6:.2f} us)")
    del copies
    torch.cuda.empty_cache()
    return out


def stream_read_ceiling(torch, sd, steps=10, repeats=3):
    """A plain streaming read (sd_hbm_stream_read) of the GEMV and attention
    sizes: each timed round reads distinct buffers worth at least 1 GiB (so no
    read is served by the 256 MB Infinity Cache), one launch per buffer, like
    the GEMV sweep.  GB/s, median of `repeats` graph-timed runs."""
    import ctypes
    lib = sd._lib.load()
    P = ctypes.c_void_p
    sink = torch.zeros(64, dtype=torch.int32, device="cuda")
    sizes = [("O 4096x4096", 17825792), ("QKV 6144x4096", 26738688), ("down/gate|up 62.4 MB", 62390272),
             ("gate|up 28672x4096", 124780544), ("LM head 151936x4096", 661225472), ("4 GiB", 4 << 30)]
    out = {}
    for label, nbytes in sizes:
        nbytes = nbytes // 16 * 16
        n_buf = max(1, -(-(1 << 30) // nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(n_buf)]

        def run():
            st = P(torch.cuda.current_stream().cuda_stream)
            for b in bufs:
                rc = lib.sd_hbm_stream_read(P(b.data_ptr()), nbytes, P(sink.data_ptr()), st)
                if rc:
                    raise sd.SdError("sd_hbm_stream_read", rc)
        runs = [time_graph(torch, run, steps, 2) for _ in range(repeats)]
        dt = median(runs) / n_buf
        gbs = nbytes / dt / 1e9
        out[label] = {"bytes": nbytes, "GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                      "us": round(dt * 1e6, 3), "buffers": n_buf}
        log(f"stream read {label}: {gbs:.1f} GB/s ({dt * 1e6:.2f} us per buffer)")
        del bufs
        torch.cuda.empty_cache()
    return out


DECODE_DIMS = dict(n_layers=32, hidden=4096, n_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                   vocab=151936, eps=1e-6, theta=1e6)
RAGGED = [2050, 3072, 16384, 32768]


def decode_child(steps, warmup):
    """One fresh process's decode timings: aggregate tok/s of sd_decode_step
    for 1..4 sequences at the ragged contexts and at all-2050 (the scaling
    control), `warmup` untimed steps then `steps` timed ones each."""
    import torch
    import sequence_decode_amd as sd
    from sequence_decode_amd.step import DecodeModel, SeqCache, StepRunner
    sd.load()
    torch.cuda.set_device(0)
    model = DecodeModel.random_device(11, DECODE_DIMS)
    g = torch.Generator(device="cuda")
    g.manual_seed(12)
    span = warmup + steps + 4
    caches = [SeqCache.random_device(g, 32, ctx + span, 8, 128) for ctx in RAGGED]
    res = {}
    for label, ctxs in (("ragged", RAGGED), ("ctx2050", [2050] * 4)):
        for n in (1, 2, 3, 4):
            r = StepRunner(model, caches[:n], max_ctx=max(ctxs[:n]) + span)
            r.tokens.copy_(torch.arange(n, dtype=torch.int32) + 7)
            r.set_positions([c - 1 for c in ctxs[:n]])
            for _ in range(warmup):
                r.step()
                r.advance()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            host = 0.0
            for _ in range(steps):
                h0 = time.perf_counter()
                r.step()
                host += time.perf_counter() - h0
                r.advance()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / steps
            res[f"{label}_n{n}"] = {"ms_per_step": dt * 1e3, "host_enqueue_ms": host / steps * 1e3}
    return {"decode_child": res, "weight_bytes": model.weight_bytes}


def decode_children(n_proc, steps, warmup):
    """Runs decode_child in n_proc fresh processes one after another (started
    before this process touches the GPU) and returns the per-configuration
    median, with every process's figure."""
    import subprocess
    runs = []
    for i in range(n_proc):
        cmd = [sys.executable, os.path.abspath(__file__), "--decode-child", "--steps", str(steps),
               "--warmup", str(warmup)]
        log(f"decode step, fresh process {i + 1}/{n_proc}")
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=900)
        if r.returncode != 0:
            raise RuntimeError(f"decode child failed ({r.returncode}):\n{r.stderr[-2000:]}")
        line = [ln for ln in r.stdout.splitlines() if ln.startswith("{")][-1]
        runs.append(json.loads(line))
    wb = runs[0]["weight_bytes"]
    out = {"model": "random-init dense 32-layer, hidden 4096, 32/8 heads, ffn 14336, vocab 151936, "
                    "q8_0 weights, fp16 KV", "weight_bytes": wb,
           "protocol": f"{warmup} warmup + {steps} timed steps per configuration, median of {n_proc} fresh "
                       f"processes"}
    res = {}
    for key in runs[0]["decode_child"]:
        ms = [r["decode_child"][key]["ms_per_step"] for r in runs]
        host = [r["decode_child"][key]["host_enqueue_ms"] for r in runs]
        label, n = key.rsplit("_n", 1)
        n = int(n)
        ctxs = (RAGGED if label == "ragged" else [2050] * 4)[:n]
        dt = median(ms) / 1e3
        step_bytes = wb + sum(ctxs) * 4096 * DECODE_DIMS["n_layers"]
        res[key] = {"tok_s": round(n / dt, 2), "ms_per_step": round(dt * 1e3, 3),
                    "ms_per_step_runs": [round(v, 3) for v in ms], "host_enqueue_ms": round(median(host), 3),
                    "step_bytes": step_bytes, "frac_hbm_peak": round(step_bytes / dt / 1e9 / HBM_PEAK_GBS, 4)}
        log(f"decode {label} n_seq={n}: {n / dt:.1f} tok/s (median {dt * 1e3:.3f} ms/step over {n_proc} "
            f"processes: {', '.join(f'{v:.3f}' for v in ms)})")
    out["results"] = res
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_attention_and_step(torch, budget_steps=4):
    """The oracle on the attention and decode-step workloads, one bounded sample
    each: one multi-sequence attention call over the four ragged contexts
    (one layer, 32 query heads, 8 KV heads, head_dim 128, fp64 softmax), and
    one decode step of the full 32-layer model for 1..4 sequences at the
    ragged contexts (host copies of the device model's weights and caches)."""
    import numpy as np
    import oracle
    from oracle import step as ostep
    from sequence_decode_amd import synth
    from sequence_decode_amd.step import DecodeModel, SeqCache
    out = {}
    g = synth.rng(31)
    H_q, H_kv, Dh = 32, 8, 128
    caches = [(synth.kv_cache(g, L, H_kv, Dh), synth.kv_cache(g, L, H_kv, Dh)) for L in RAGGED]
    q = synth.queries(g, 4, H_q, Dh)
    scale = np.float32(1.0) / np.sqrt(np.float32(Dh))
    t0 = time.perf_counter()
    oracle.attn_decode_multiseq(q, caches, RAGGED, scale)
    dt = time.perf_counter() - t0
    kv_bytes = sum(RAGGED) * 4096
    out["attention"] = {"ms": round(dt * 1e3, 2), "GB_s": round(kv_bytes / dt / 1e9, 3),
                        "sample": "one call: 4 sequences at contexts 2050/3072/16384/32768, one layer"}
    log(f"oracle attention (ragged contexts, one layer): {dt * 1e3:.1f} ms")
    del caches
    # the full model: device draw (the benchmark's seed), host copies
    model = DecodeModel.random_device(11, DECODE_DIMS)
    gd = torch.Generator(device="cuda")
    gd.manual_seed(12)

    def hc(t):
        return t.cpu().numpy()
    layers = [{k: hc(L[k]) for k in ("w_qkv", "w_o", "w_gu", "w_down", "attn_norm", "ffn_norm")}
              for L in model.layers]
    om = ostep.Model(4096, 32, 8, 128, 14336, 151936, 1e-6, 1e6,
                     model.tok_embd.cpu().view(torch.int16).numpy().view(np.uint16),
                     hc(model.out_norm), hc(model.w_lm), layers)
    del model
    torch.cuda.empty_cache()
    hcaches = []
    for ctx in RAGGED:
        c = SeqCache.random_device(gd, 32, ctx + 1, 8, 128)
        hcaches.append((c.k.cpu().view(torch.int16).numpy().view(np.uint16),
                        c.v.cpu().view(torch.int16).numpy().view(np.uint16)))
        del c
    torch.cuda.empty_cache()
    steps = {}
    for n in range(1, budget_steps + 1):
        t0 = time.perf_counter()
        ostep.decode_step(om, hcaches[:n], list(range(7, 7 + n)), [c - 1 for c in RAGGED[:n]])
        dt = time.perf_counter() - t0
        steps[str(n)] = {"tok_s": round(n / dt, 3), "s_per_step": round(dt, 2)}
        log(f"oracle decode step, {n} sequence(s): {dt:.2f} s ({n / dt:.3f} tok/s)")
    out["decode_step"] = {"per_n_seq": steps,
                          "sample": "one step per sequence count of the 32-layer model, contexts "
                                    "2050/3072/16384/32768[:n], host copies of the benchmark's weights"}
    return out


def trace_summary(trace_db, fetch_db=None, write_db=None, n_tok=4):
    """Summary (markdown) of rocprofv3 results databases of `bench.py
    --sweep-only --calibrate-copy`: per-kernel statistics of the trace, and
    for the launches the roofline pass times (per shape, the 128 timed ones of
    its 160, in launch order: QKV, O, gate|up on the staged one-chunk kernel,
    down on the four-chunk one) their average trace duration and, from the
    counter runs, their HBM bytes: FETCH_SIZE and WRITE_SIZE (KiB) scaled by
    what the same counters read for the 1 GiB calibration copy."""
    import hashlib
    import sqlite3
    import statistics

    def dispatches(db, pmc=None):
        con = sqlite3.connect(db)
        if pmc is None:
            q = ("select k.display_name, d.start, d.end from rocpd_kernel_dispatch d join "
                 "rocpd_info_kernel_symbol k on d.kernel_id = k.id order by d.start")
            return [(n, (e - s_) / 1e3) for n, s_, e in con.execute(q)]
        q = "select name, counter_value from pmc_events where counter_name = ? order by dispatch_id"
        return list(con.execute(q, (pmc,)))

    def short(name):
        name = name.replace("void ", "", 1)
        name = name.replace("sd::(anonymous namespace)::", "")
        i = name.find("(")
        return name[:i] if i > 0 else name

    staged = f"k_qgemv_q8_0_dma<{n_tok}, 1, 1, 8, true, false, false, false>"
    four = f"k_qgemv_q8_0_dma<{n_tok}, 4, 1, 4, false, false, false, false>"

    per_shape_n = (ROOF_WARM_ROUNDS + ROOF_REPS) * N_LAYERS  # dispatches per shape in the pass
    skip = ROOF_WARM_ROUNDS * N_LAYERS

    def roofline_launches(rows):
        a = [v for n, v in rows if short(n) == staged][-3 * per_shape_n:]
        b = [v for n, v in rows if short(n) == four][-per_shape_n:]
        if len(a) < 3 * per_shape_n or len(b) < per_shape_n:
            raise RuntimeError("the database does not hold the roofline pass")
        return {"qkv": a[skip:per_shape_n], "o": a[per_shape_n + skip:2 * per_shape_n],
                "gate_up": a[2 * per_shape_n + skip:], "down": b[skip:]}

    tr = dispatches(trace_db)
    per = {}
    for n, us in tr:
        per.setdefault(short(n), []).append(us)
    lines = ["| kernel | calls | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1]))[:24]:
        lines.append(f"| {k[:110]} | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{sum(v) / 1e3:.2f} |")
    roof = roofline_launches(tr)
    shapes = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}
    out = {"kernel_stats": "\n".join(lines), "per_shape": {}}
    tot_us, tot_b = 0.0, 0
    for k, v in roof.items():
        N, K = shapes[k]
        b = gemv_bytes(N, K, n_tok)
        out["per_shape"][k] = {"trace_avg_us": round(statistics.mean(v), 3), "GB_s": round(b / statistics.mean(v) / 1e3, 1)}
        tot_us += sum(v)
        tot_b += b * len(v)
    n_roof = 4 * ROOF_REPS * N_LAYERS
    out["trace_avg_us_per_launch"] = round(tot_us / n_roof, 3)
    out["trace_launches"] = n_roof
    out["achieved_GB_s"] = round(tot_b / tot_us / 1e3, 1)
    out["gemv_us_per_sweep"] = round(sum(statistics.mean(v) for v in roof.values()) * N_LAYERS, 1)
    # the same kernels in the graph-replayed n_tok sweeps of the run (every
    # launch before the roofline pass, in layer order QKV, O, gate|up, down):
    # what a sweep's wall time holds
    sw = [(short(n), v) for n, v in tr if short(n) in (staged, four)][:-4 * per_shape_n]
    if sw and len(sw) % (4 * N_LAYERS) == 0 and all(
            nm == (four if i % 4 == 3 else staged) for i, (nm, _) in enumerate(sw)):
        by = {k: [v for i, (_, v) in enumerate(sw) if i % 4 == j] for j, k in enumerate(shapes)}
        out["graph_sweeps"] = {
            "sweeps": len(sw) // (4 * N_LAYERS),
            "per_shape_avg_us": {k: round(statistics.mean(v), 3) for k, v in by.items()},
            "gemv_us_per_sweep": round(sum(statistics.mean(v) for v in by.values()) * N_LAYERS, 1),
            "GB_s": round(sum(gemv_bytes(*shapes[k], n_tok) for k in shapes) * N_LAYERS /
                          (sum(statistics.mean(v) for v in by.values()) * N_LAYERS) / 1e3, 1)}
    if fetch_db and write_db:
        f = dispatches(fetch_db, "FETCH_SIZE")
        w = dispatches(write_db, "WRITE_SIZE")
        fcal = [v for n, v in f if "copyBuffer" in n]
        wcal = [v for n, v in w if "copyBuffer" in n]
        ff = (1 << 30) / (fcal[-1] * 1024)
        wf = (1 << 30) / (wcal[-1] * 1024)
        rf, rw = roofline_launches(f), roofline_launches(w)
        fetched = sum(sum(v) for v in rf.values()) * 1024 * ff / n_roof
        written = sum(sum(v) for v in rw.values()) * 1024 * wf / n_roof
        out["fetch_factor"], out["write_factor"] = round(ff, 4), round(wf, 4)
        out["traffic_bytes_per_launch"] = int(round(fetched + written))
        out["algorithmic_bytes_per_launch"] = int(round(tot_b / n_roof))
        out["traffic_over_algorithmic"] = round((fetched + written) / (tot_b / n_roof), 4)
    src = os.path.join(ROOT, "sequence_decode_amd", "csrc", "qgemv.hip")
    out["kernel_source_sha256"] = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return out


def _rocpd_dispatches(db, pmc=None):
    """(kernel display name, duration us) of every dispatch of a rocprofv3
    results database in start order, or (name, counter value) per dispatch of
    a counter run."""
    import sqlite3
    con = sqlite3.connect(db)
    if pmc is None:
        q = ("select k.display_name, d.start, d.end from rocpd_kernel_dispatch d join "
             "rocpd_info_kernel_symbol k on d.kernel_id = k.id order by d.start")
        return [(n, (e - s_) / 1e3) for n, s_, e in con.execute(q)]
    q = "select name, counter_value from pmc_events where counter_name = ? order by dispatch_id"
    return list(con.execute(q, (pmc,)))


def _short_kernel(name):
    name = name.replace("void ", "", 1).replace("sd::(anonymous namespace)::", "")
    i = name.find("(")
    return name[:i] if i > 0 else name


def _kernel_stats(rows, top=24):
    import statistics
    per = {}
    for n, us in rows:
        per.setdefault(_short_kernel(n), []).append(us)
    lines = ["| kernel | calls | avg us | min us | max us | total ms |", "|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(kv[1]))[:top]:
        lines.append(f"| {k[:110]} | {len(v)} | {statistics.mean(v):.2f} | {min(v):.2f} | {max(v):.2f} | "
                     f"{sum(v) / 1e3:.2f} |")
    return "\n".join(lines)


def wide_trace_summary(trace_db, fetch_db=None, write_db=None, n_tok=16):
    """Summary of rocprofv3 results databases of `bench.py --wide-only` (and,
    for the counter runs, `--wide-only --calibrate-copy`): the matrix-core
    GEMV's launches of the roofline pass at n_tok 16 (per shape, in launch order
    QKV, O, gate|up, down, the 128 timed ones of its 192), their average trace
    duration, and from the counter runs their HBM bytes per launch (FETCH_SIZE
    and WRITE_SIZE scaled by what the counters read for the 1 GiB calibration
    copy)."""
    import hashlib
    import statistics
    kern = "k_qgemv_q8_0_mfma"
    per_shape_n = (ROOF_WARM_ROUNDS + ROOF_REPS) * N_LAYERS
    skip = ROOF_WARM_ROUNDS * N_LAYERS
    shapes = {"qkv": (6144, 4096), "o": (4096, 4096), "gate_up": (28672, 4096), "down": (4096, 14336)}

    def launches(rows):
        a = [v for n, v in rows if _short_kernel(n) == kern][-4 * per_shape_n:]
        if len(a) < 4 * per_shape_n:
            raise RuntimeError("the database does not hold the matrix-core roofline pass")
        return {k: a[i * per_shape_n + skip:(i + 1) * per_shape_n] for i, k in enumerate(shapes)}

    tr = _rocpd_dispatches(trace_db)
    roof = launches(tr)
    out = {"kernel_stats": _kernel_stats(tr), "n_tok": n_tok, "per_shape": {}}
    tot_us, tot_b, n_all = 0.0, 0, 0
    for k, v in roof.items():
        b = gemv_bytes(*shapes[k], n_tok)
        out["per_shape"][k] = {"trace_avg_us": round(statistics.mean(v), 3),
                               "GB_s": round(b / statistics.mean(v) / 1e3, 1)}
        tot_us += sum(v)
        tot_b += b * len(v)
        n_all += len(v)
    out["trace_avg_us_per_launch"] = round(tot_us / n_all, 3)
    out["achieved_GB_s"] = round(tot_b / tot_us / 1e3, 1)
    out["gemv_us_per_sweep"] = round(sum(statistics.mean(v) for v in roof.values()) * N_LAYERS, 1)
    if fetch_db and write_db:
        f = _rocpd_dispatches(fetch_db, "FETCH_SIZE")
        w = _rocpd_dispatches(write_db, "WRITE_SIZE")
        ff = (1 << 30) / ([v for n, v in f if "copyBuffer" in n][-1] * 1024)
        wf = (1 << 30) / ([v for n, v in w if "copyBuffer" in n][-1] * 1024)
        rf, rw = launches(f), launches(w)
        out["fetch_factor"], out["write_factor"] = round(ff, 4), round(wf, 4)
        out["traffic_per_shape"] = {}
        for k in shapes:
            fb = statistics.mean(rf[k]) * 1024 * ff
            wb = statistics.mean(rw[k]) * 1024 * wf
            alg = gemv_bytes(*shapes[k], n_tok)
            out["traffic_per_shape"][k] = {"fetched": int(round(fb)), "written": int(round(wb)),
                                           "algorithmic": alg, "ratio": round((fb + wb) / alg, 4)}
        fetched = sum(sum(v) for v in rf.values()) * 1024 * ff / n_all
        written = sum(sum(v) for v in rw.values()) * 1024 * wf / n_all
        out["traffic_bytes_per_launch"] = int(round(fetched + written))
        out["algorithmic_bytes_per_launch"] = int(round(tot_b / n_all))
        out["traffic_over_algorithmic"] = round((fetched + written) / (tot_b / n_all), 4)
    src = os.path.join(ROOT, "sequence_decode_amd", "csrc", "qgemv.hip")
    out["kernel_source_sha256"] = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return out


ATTN_CASES = {"n1_2050": [2050], "n4_2050": [2050] * 4, "n4_ragged": [2050, 3072, 16384, 32768],
              "n1_32768": [32768]}


def attn_trace_summary(trace_db, fetch_db=None, write_db=None, reps=20):
    """Summary (markdown) of rocprofv3 results databases of `bench.py
    --attention-only` (and, for the counter runs, `--attention-only
    --calibrate-copy`): per case of the attention pass (its order: each context
    set with fp16, q8_0 and paged fp16 caches), the average trace duration of
    the chunk kernel and of the merge kernel over the timed calls (the last
    `reps` graph replays of every cache set; each case makes 2 warm-up rounds,
    one untimed replay and `reps` timed ones), and from the counter runs the
    HBM bytes per chunk-kernel dispatch: FETCH_SIZE and WRITE_SIZE (KiB) scaled
    by what the same counters read for the 1 GiB calibration copy."""
    import hashlib
    import statistics

    def split(rows):
        chunk = [v for n, v in rows if _short_kernel(n).startswith("k_attn_chunk")]
        comb = [v for n, v in rows if _short_kernel(n).startswith("k_attn_combine")]
        out, i = {}, 0
        for cname, lens in ATTN_CASES.items():
            for kind in ATTN_KINDS:
                sets = attn_sets(lens, kind)
                n = (3 + reps) * sets
                out[f"{cname}_{kind}"] = (chunk[i + 3 * sets:i + n], comb[i + 3 * sets:i + n])
                i += n
        if i != len(chunk) or i != len(comb):
            raise RuntimeError(f"the database does not hold exactly one attention pass ({len(chunk)} "
                               f"chunk and {len(comb)} merge dispatches, expected {i})")
        return out

    tr = _rocpd_dispatches(trace_db)
    cases = split(tr)
    have_pmc = fetch_db and write_db
    if have_pmc:
        f = _rocpd_dispatches(fetch_db, "FETCH_SIZE")
        w = _rocpd_dispatches(write_db, "WRITE_SIZE")
        ff = (1 << 30) / ([v for n, v in f if "copyBuffer" in n][-1] * 1024)
        wf = (1 << 30) / ([v for n, v in w if "copyBuffer" in n][-1] * 1024)
        fc, wc = split(f), split(w)
    lines = ["| case | chunk kernel avg us | merge avg us | cache bytes | fetched B (calibrated) | ratio | written B |",
             "|---|---|---|---|---|---|---|"]
    for key, (ch, cb) in cases.items():
        cname, kind = key.split("_", 2)[0] + "_" + key.split("_", 2)[1], key.split("_", 2)[2]
        lens = ATTN_CASES[cname]
        cache = sum(lens) * attn_key_bytes(kind)
        row = f"| {key} | {statistics.mean(ch):.2f} | {statistics.mean(cb):.2f} | {cache:,} |"
        if have_pmc:
            fb = statistics.mean(fc[key][0]) * 1024 * ff
            wb = statistics.mean(wc[key][0]) * 1024 * wf
            row += f" {fb:,.0f} | {fb / cache:.3f} | {wb:,.0f} |"
        else:
            row += " | | |"
        lines.append(row)
    src = os.path.join(ROOT, "sequence_decode_amd", "csrc", "attn.hip")
    out = {"per_case": "\n".join(lines), "kernel_stats": _kernel_stats(tr, 8),
           "kernel_source_sha256": hashlib.sha256(open(src, "rb").read()).hexdigest()}
    if have_pmc:
        out["fetch_factor"], out["write_factor"] = round(ff, 4), round(wf, 4)
    return out


def step_trace_summary(trace_db, n_steps=10):
    """Summary (markdown) of a rocprofv3 results database of `bench.py
    --step-only N`: the library's kernels of the last `n_steps` steps (a step
    ends with its argmax), per kernel and per step, with the step's span and
    its kernel-busy time."""
    import statistics
    rows = []
    import sqlite3
    con = sqlite3.connect(trace_db)
    q = ("select k.display_name, d.start, d.end, d.grid_size_x, d.grid_size_y from rocpd_kernel_dispatch d "
         "join rocpd_info_kernel_symbol k on d.kernel_id = k.id order by d.start")
    for n, s_, e, gx, gy in con.execute(q):
        if "sd::" in n:
            rows.append((_short_kernel(n), s_, e, f"{gx}" if gy == 1 else f"{gx}x{gy}"))
    ends, prev = [], None
    for i, r in enumerate(rows):
        if r[0].startswith("k_argmax"):
            if prev is not None and i == prev + 1:
                ends[-1] = i
            else:
                ends.append(i)
            prev = i
    ends = ends[-(n_steps + 1):]
    acc, spans, busy = {}, [], []
    for a, b in zip(ends[:-1], ends[1:]):
        seg = rows[a + 1:b + 1]
        spans.append((seg[-1][2] - rows[a][2]) / 1e3)
        busy.append(sum(e - s_ for _, s_, e, _ in seg) / 1e3)
        for n, s_, e, g in seg:
            acc.setdefault((n, g), []).append((e - s_) / 1e3)
    k = len(spans)
    lines = [f"{k} steps: span {statistics.mean(spans):.1f} us per step, kernel-busy {statistics.mean(busy):.1f} us",
             "", "| kernel | grid (threads, x or x by y) | per step | avg us | us per step |", "|---|---|---|---|---|"]
    for (n, g), v in sorted(acc.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"| {n[:100]} | {g} | {len(v) / k:.1f} | {statistics.mean(v):.2f} | {sum(v) / k:.1f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--n-tok", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--decode-procs", type=int, default=3,
                    help="fresh processes the decode tok/s are the median of")
    ap.add_argument("--decode-only", action="store_true", help="only the decode-step tok/s and its variants")
    ap.add_argument("--decode-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--step-only", type=int, default=0, metavar="N_SEQ",
                    help="only decode steps of N_SEQ ragged sequences (for a kernel trace of the step)")
    ap.add_argument("--attention-only", action="store_true",
                    help="only the attention timings (fp16, q8_0 and paged caches)")
    ap.add_argument("--sweep-only", action="store_true",
                    help="only the projection sweeps and the per-shape event pass (for a kernel trace)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for byte counters)")
    ap.add_argument("--attn-trace-summary", nargs="+", metavar="DB",
                    help="print the per-case summary of rocprofv3 databases of --attention-only: "
                         "trace [FETCH_SIZE WRITE_SIZE]")
    ap.add_argument("--step-trace-summary", metavar="DB",
                    help="print the per-step kernel breakdown of a rocprofv3 database of --step-only N")
    ap.add_argument("--wide-only", action="store_true",
                    help="only the matrix-core GEMV's per-shape roofline pass at 16 tokens (for profiling)")
    ap.add_argument("--wide-trace-summary", nargs="+", metavar="DB",
                    help="summarize rocprofv3 databases of --wide-only: trace [fetch write]")
    ap.add_argument("--trace-summary", nargs="+", metavar="DB",
                    help="summarize rocprofv3 results databases of a --sweep-only run: the kernel-trace "
                         "database, then optionally the FETCH_SIZE and WRITE_SIZE ones (no GPU used)")
    args = ap.parse_args()
    if args.attn_trace_summary:
        r = attn_trace_summary(*args.attn_trace_summary[:3])
        print(r["per_case"] + "\n\n" + r["kernel_stats"] + "\n\nkernel_source_sha256: " + r["kernel_source_sha256"])
        return
    if args.step_trace_summary:
        print(step_trace_summary(args.step_trace_summary))
        return
    if args.trace_summary:
        print(json.dumps(trace_summary(*args.trace_summary[:3], n_tok=args.n_tok), indent=1))
        return
    if args.wide_trace_summary:
        print(json.dumps(wide_trace_summary(*args.wide_trace_summary[:3]), indent=1))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode step here is built and measured on a "
              "single MI355X; run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.decode_child:
        print(json.dumps(decode_child(args.steps, args.warmup)), flush=True)
        return

    # the decode tok/s come from fresh processes started before this one
    # touches the GPU: 8 warmups, 64 timed steps, median of the processes
    decode = None
    if (not args.no_decode and not args.step_only and not args.attention_only and not args.sweep_only
            and not args.wide_only):
        decode = decode_children(args.decode_procs, 64, 8)

    import torch
    import sequence_decode_amd as sd
    sd.load()
    torch.cuda.set_device(0)
    if args.step_only:
        print(json.dumps(step_only(torch, args.step_only, args.steps, args.warmup)), flush=True)
        return
    if args.decode_only:
        decode["variants"] = decode_bench(torch, steps=max(8, args.steps), warmup=args.warmup)
        print(json.dumps(decode), flush=True)
        return
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        log("calibration copy: 1073741824 bytes read, 1073741824 bytes written")
        del a, b
    if args.attention_only:
        print(json.dumps(attention_bench(torch)), flush=True)
        return
    log("generating 7.42 GB of q8_0 projection weights on the device")
    sweep = Sweep(sd, torch, seed=1, max_tok=16)
    torch.cuda.synchronize()
    if args.wide_only:
        # the 16-token sweep (graph-timed) and its per-shape roofline pass, on
        # the matrix-core kernel that sd_qgemv_q8_0_batch picks at 16 tokens
        dt, runs = sweep_median(torch, sweep, 16, max(3, args.steps // 2), 2)
        _, _, _, roof_shapes = roofline_pass(torch, sweep, 16, ROOF_REPS)
        print(json.dumps({"n_tok": 16, "GB_s": round(sweep.bytes_per_step(16) / dt / 1e9, 1),
                          "ms_per_step": round(dt * 1e3, 4), "per_shape": roof_shapes}), flush=True)
        return

    per_n = {}
    for n in (1, 2, 3, 4):
        dt, runs = sweep_median(torch, sweep, n, max(3, args.steps // 2), 2)
        gbs = sweep.bytes_per_step(n) / dt / 1e9
        per_n[str(n)] = {"GB_s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                         "ms_per_step": round(dt * 1e3, 4),
                         "GB_s_runs": [round(sweep.bytes_per_step(n) / r / 1e9, 1) for r in runs]}
        log(f"sweep n_tok={n}: {gbs:.1f} GB/s ({gbs / HBM_PEAK_GBS:.1%} of 8 TB/s), "
            f"{dt * 1e3:.3f} ms (median of {len(runs)})")

    n = args.n_tok
    dt, runs = sweep_median(torch, sweep, n, args.steps, args.warmup)
    value = sweep.bytes_per_step(n) / dt / 1e9

    tb, tms, launches, per_shape = roofline_pass(torch, sweep, n, reps=ROOF_REPS)
    achieved = tb / (tms / 1e3) / 1e9
    log(f"GEMV kernel (event-timed, {launches} launches): {achieved:.1f} GB/s; {per_shape}")
    floor = launch_floor_us(torch)
    for v in per_shape.values():
        body = v["avg_us"] - floor
        v["GB_s_after_launch_floor"] = round(v["bytes_per_launch"] / body / 1e3, 1) if body > 0 else None
    log(f"launch floor (graph of one-element kernels): {floor:.2f} us per launch")
    prof = profile_fields()
    traffic = int(prof["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in prof else None
    roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
            "algorithmic_bytes_per_launch": round(tb / launches),
            "kernel": f"k_qgemv_q8_0_dma<{n}, SP, 1, NW, STAGE, false, false, false> (QKV, O, gate|up: SP=1, "
                      f"8 waves, staged; down: SP=4, 4 waves)", "launches": launches,
            "launch_floor_us": round(floor, 3),
            "avg_launch_us": round(tms / launches * 1e3, 3), "per_shape": per_shape}
    if "trace_avg_us_per_launch" in prof:
        # the same launches' average duration in the committed kernel trace
        t_us = float(prof["trace_avg_us_per_launch"])
        roof["trace_avg_launch_us"] = t_us
        roof["frac_trace"] = round(tb / launches / (t_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    if args.sweep_only:
        print(json.dumps({"per_n_tok": per_n, "value": round(value, 1), "roofline": roof}), flush=True)
        return

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(dt * 1e3, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": "8B-class q8_0 decode projections, 32 layers x (QKV 6144x4096, "
                               "O 4096x4096, gate|up 28672x4096, down 4096x14336)",
                   "n_tok": n, "layers": N_LAYERS, "weight_bytes": sweep.weight_bytes,
                   "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4), "repeats": len(runs),
                   "GB_s_runs": [round(sweep.bytes_per_step(n) / r / 1e9, 1) for r in runs]},
        "per_n_tok": per_n,
        "roofline": roof,
    }
    line["config1_rotated"] = config1_rotated(torch, sd, max(3, args.steps // 2))
    line["stream_read_ceiling"] = stream_read_ceiling(torch, sd)
    line["verify_widths"] = verify_widths(torch, sweep, max(3, args.steps // 2))
    line["attention"] = attention_bench(torch)
    line["decode_step"] = decode
    if decode is not None:
        line["decode_step"]["variants"] = decode_bench(torch, steps=max(8, args.steps), warmup=args.warmup)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(torch, sweep, n, args.cpu_seconds)
        del sweep
        torch.cuda.empty_cache()
        line["cpu_baseline"]["oracle_workloads"] = oracle_attention_and_step(torch)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
