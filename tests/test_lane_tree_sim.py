"""Host simulation of the GEMV's one-pass lane tree for 2-8 tokens.

The streaming GEMV sums each token's 64 lane cells with a fixed tree (lane
partners l^1, l^2, 7-l within 8, 15-l within 16, l^16, l^32).  For 2-4 tokens
it runs that tree once over all tokens: at the first two (2-4 tokens) or
three (5-8 tokens) levels a lane keeps some tokens and hands the others to
its partner.  This test replays both forms
in float32 with the same partner patterns and checks, lane by lane, that every
token's total has the bits of the per-token tree, and that the writing lanes
(2, 4 or 8) name each token once.  The GPU width-invariance tests check the
kernel itself."""
import numpy as np

F32 = np.float32
L = np.arange(64)
PARTNER = {"x1": L ^ 1, "x2": L ^ 2, "hmir": (L & ~7) | (7 - (L & 7)), "mir": (L & ~15) | (15 - (L & 15))}


def _add(a, b):
    return (a + b).astype(F32)


def _cross(v):
    v = _add(v, v[L ^ 16])
    return _add(v, v[L ^ 32])


def _tree(v):
    for k in ("x1", "x2", "hmir", "mir"):
        v = _add(v, v[PARTNER[k]])
    return _cross(v)


def _tree_tr8(vs):
    vs = vs + [np.zeros(64, F32)] * (8 - len(vs))
    c1 = ((L ^ (L >> 2)) & 1) == 1         # keeps tokens 4..7
    k = [_add(np.where(c1, vs[4 + i], vs[i]), np.where(c1, vs[i], vs[4 + i])[PARTNER["x1"]]) for i in range(4)]
    c2 = (((L >> 1) ^ (L >> 2)) & 1) == 1  # keeps the second two of its four
    m = [_add(np.where(c2, k[2 + i], k[i]), np.where(c2, k[i], k[2 + i])[PARTNER["x2"]]) for i in range(2)]
    c3 = ((L ^ (L >> 3)) & 1) == 1         # keeps the second of its two
    e = _add(np.where(c3, m[1], m[0]), np.where(c3, m[0], m[1])[PARTNER["hmir"]])
    e = _add(e, e[PARTNER["mir"]])
    return _cross(e)


def _tree_tr(vs, nt):
    if nt > 4:
        return _tree_tr8(vs)
    lo1 = ((L ^ (L >> 2)) & 1) == 0
    if nt == 2:
        e = _add(np.where(lo1, vs[0], vs[1]), np.where(lo1, vs[1], vs[0])[PARTNER["x1"]])
        e = _add(e, e[PARTNER["x2"]])
    else:
        v3 = vs[3] if nt == 4 else np.zeros(64, F32)
        a = _add(np.where(lo1, vs[0], vs[2]), np.where(lo1, vs[2], vs[0])[PARTNER["x1"]])
        b = _add(np.where(lo1, vs[1], v3), np.where(lo1, v3, vs[1])[PARTNER["x1"]])
        lo2 = (((L >> 1) ^ (L >> 2)) & 1) == 0
        e = _add(np.where(lo2, a, b), np.where(lo2, b, a)[PARTNER["x2"]])
    e = _add(e, e[PARTNER["hmir"]])
    e = _add(e, e[PARTNER["mir"]])
    return _cross(e)


def _token(lane, nt):
    b0, b1, b2, b3 = lane & 1, (lane >> 1) & 1, (lane >> 2) & 1, (lane >> 3) & 1
    if nt == 2:
        return b0 ^ b2
    if nt <= 4:
        return 2 * (b0 ^ b2) + (b1 ^ b2)
    return 4 * (b0 ^ b2) + 2 * (b1 ^ b2) + (b0 ^ b3)


def test_one_pass_tree_matches_per_token_tree_bitwise():
    rng = np.random.default_rng(11)
    for _ in range(400):
        for nt in (2, 3, 4, 5, 6, 7, 8):
            vs = [(rng.standard_normal(64) * np.exp(rng.uniform(-8, 8, 64))).astype(F32) for _ in range(nt)]
            ref = [_tree(v) for v in vs]
            out = _tree_tr(vs, nt)
            for lane in range(64):
                t = _token(lane, nt)
                if t < nt:
                    assert out[lane].view(np.uint32) == ref[t][lane].view(np.uint32)
            writers = 2 if nt == 2 else (4 if nt <= 4 else 8)
            assert sorted(_token(lane, nt) for lane in range(writers)) == list(range(writers))
