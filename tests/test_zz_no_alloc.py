"""The allocation-free attention entry point (sd_decode_attn_multiseq_noalloc)
against the workspace entry point (sd_decode_attn_multiseq) it varies.

Both run the same kernels, the first with its chunk partials in the library's
static scratch array, so the outputs must be bitwise equal.  Two calls in a
row, the second with a smaller input (fewer sequences, shorter contexts), show
that the scratch array's leftovers from a call never reach the next one.  A
call whose partials would not fit the array is refused before any launch.
"""
import numpy as np
import pytest

import oracle
from helpers import bits, dev, host, say
from sequence_decode_amd import synth

pytestmark = pytest.mark.gpu

H_Q, H_KV, D = 32, 8, 128
SCALE = np.float32(1.0) / np.sqrt(np.float32(D))


def _views(sd, lens, seed):
    import torch
    g = synth.rng(seed)
    kv = [(synth.kv_cache(g, L + 3, H_KV, D), synth.kv_cache(g, L + 3, H_KV, D)) for L in lens]
    devkv = [(dev(k, torch.float16), dev(v, torch.float16)) for k, v in kv]
    return kv, devkv, [sd.seqview(k, v, L) for (k, v), L in zip(devkv, lens)]


def test_noalloc_equals_workspace_entry_point_two_calls(sd):
    big = [2050, 3072, 16384, 32768]
    small = [300, 17]
    outs = []
    for i, lens in enumerate((big, small)):
        say(f"noalloc attention call {i}: contexts {lens}")
        kv, devkv, views = _views(sd, lens, 9100 + i)
        q = dev(synth.queries(synth.rng(9200 + i), len(lens), H_Q, D))
        o_ws = host(sd.decode_attn_multiseq(q, views, H_KV, SCALE))
        o_na = host(sd.decode_attn_multiseq_noalloc(q, views, H_KV, SCALE))
        assert np.array_equal(bits(o_na), bits(o_ws)), lens
        outs.append((kv, host(q), o_na, lens))
    # the smaller second call against the oracle too (its partials overwrite
    # only the front of what the first call left in the scratch array)
    kv, q, o, lens = outs[1]
    ref = oracle.attn_decode_multiseq(q, kv, lens, SCALE)
    assert np.max(np.abs(o - ref)) <= 2e-3


def test_noalloc_refuses_partials_beyond_the_scratch_array(sd):
    """Four sequences of 65536 keys need 4 * 280 chunks * 32 heads * 528 B =
    18.9 MB of partials, beyond the 16 MiB array: SD_EWORKSPACE, no launch."""
    import torch
    # real 65536-row caches, so that every access would stay in bounds even if
    # the call were (wrongly) launched
    k = torch.zeros((65536, H_KV, D), dtype=torch.float16, device="cuda")
    views = [sd.seqview(k, k, 65536) for _ in range(4)]
    assert sd.decode_attn_workspace_bytes(views, H_Q, D) > sd.ATTN_SCRATCH_BYTES
    q = torch.zeros((4, H_Q, D), dtype=torch.float32, device="cuda")
    with pytest.raises(sd.SdError) as e:
        sd.decode_attn_multiseq_noalloc(q, views, H_KV, SCALE)
    assert e.value.status == -4
