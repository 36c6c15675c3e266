"""Host <-> device helpers for the GPU tests (numpy in, numpy out)."""
import numpy as np


def dev(a, dtype=None):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.view(dtype)
    return t.cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    if t.dtype == torch.float16:
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().numpy()


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def gemv_tolerance(absterm):
    """|y_gpu - y_oracle| <= 1e-5 * sum_b |s_b| per element (the 1e-5 relative
    bar, measured against the magnitude the rounding error scales with)."""
    return 1e-5 * absterm


def say(msg):
    print(msg, flush=True)
