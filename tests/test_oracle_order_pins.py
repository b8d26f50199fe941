"""Order-revealing pins of the oracle's composed reductions and of the
attention gradients' fixed-point format.

The reduction order is the method's definition of every result (onedev.kr
summary of Open-1B, "How": one fixed reduction order on every backend); the
order read here is CanonSum: 32-wide blocks summed left to right from their
first term, then a level-by-level pairwise tree over the block sums.  The
functions pinned below each walk their own 32-block loop (the squared norm,
the weight step's mean of |w|, dX over n, dW over m and its microbatch
running sum), so each gets an input whose exact binary32 result depends on
that order, with the expected bits derived by hand in the comments.  Every
pin comes with a sensitivity check: the same terms summed in a plausible
wrong order (one sequential chain, a midpoint split of the blocks, 16- or
64-wide blocks, a block boundary shifted by one term, blocks summed right to
left) give other bits.

The attention gradients' format (onedev.kr, "Use", attention paragraph:
64-bit fixed-point accumulation of the query gradient; the same format for
the key and value gradients is this library's reading) is pinned bit for
bit: tile sums at odd multiples of 2^-41 (exact ties at the 2^-40 grid),
terms in the two 32-halves of one 64-position tile, and terms on both sides
of position 64.  A 32-position tile, a 2^32 scale, rounding half away from
zero or truncation each change at least one pinned value.
"""
import numpy as np

import oracle

f32 = np.float32


def _bits(x):
    return np.asarray(x, np.float32).view(np.uint32)


# ---- the order-revealing term sequence ---------------------------------------
# Six 32-term blocks.  Blocks 0-3 are a one then 31 zeros (sum 1), block 4 a
# two then zeros (sum 2), block 5 is 2^24 followed by 31 ones: every
# 2^24 + 1 is a tie that rounds back to the even 2^24, so the block sum is
# 2^24.  The tree over [1, 1, 1, 1, 2, 2^24] is
#   ((1 + 1) + (1 + 1)) + (2 + 2^24) = 4 + 16777218 = 16777222 (exact).
_Z31 = [0.0] * 31
TERMS = np.array([1.0] + _Z31 + [1.0] + _Z31 + [1.0] + _Z31 + [1.0] + _Z31 + [2.0] + _Z31
                 + [2.0 ** 24] + [1.0] * 31, np.float32)
CANON = f32(16777222.0)


def _seq(p):
    s = p[0]
    for x in p[1:]:
        s = f32(s + x)
    return s


def _blocks(p, width=32, first=None):
    starts = list(range(0, len(p), width)) if first is None else [0] + list(range(first, len(p), width))
    return [_seq(p[a:(starts[i + 1] if i + 1 < len(starts) else len(p))]) for i, a in enumerate(starts)]


def _level(b):
    b = list(b)
    while len(b) > 1:
        nxt = [f32(b[i] + b[i + 1]) for i in range(0, len(b) - 1, 2)]
        if len(b) % 2:
            nxt.append(b[-1])
        b = nxt
    return b[0]


def _mid(b):
    if len(b) == 1:
        return b[0]
    m = (len(b) + 1) // 2
    return f32(_mid(b[:m]) + _mid(b[m:]))


def wrong_orders(p):
    """The same terms summed in plausible wrong orders (host binary32)."""
    return {
        "sequential": _seq(p),
        "midpoint split": _mid(_blocks(p)),
        "16-wide blocks": _level(_blocks(p, 16)),
        "64-wide blocks": _level(_blocks(p, 64)),
        "boundary shifted by one": _level(_blocks(p, 32, first=31)),
        "blocks right to left": _level([_seq(p[j:j + 32][::-1]) for j in range(0, len(p), 32)]),
    }


def test_terms_separate_every_wrong_order():
    """Sensitivity of every pin below: each wrong order gives other bits."""
    for name, v in wrong_orders(TERMS).items():
        assert _bits(v) != _bits(CANON), name
    # the hand-derived value is what the oracle's own CanonSum gives
    assert _bits(oracle.canon_sum(TERMS)) == _bits(CANON)


# ---- global L2 norm ------------------------------------------------------------
def test_l2norm_order_pin():
    """T's squares are the terms above (block 4 holds two ones, 4096^2 =
    2^24), so Q = 16777222.  sqrt(2^24 + 6) = 4096 (1 + 3*2^-24 - ...) lies
    just below 4096 + 1.5 ulp (ulp = 2^-11), so nu = 4096 + 2^-11.  Any of
    the wrong orders gives Q = 16777224 or more, and sqrt(16777224) rounds
    to 4096 + 2^-10."""
    T = np.array([1.0] + _Z31 + [1.0] + _Z31 + [1.0] + _Z31 + [1.0] + _Z31 + [1.0, 1.0] + [0.0] * 30
                 + [4096.0] + [1.0] * 31, np.float32)
    nu = oracle.l2norm(T)
    assert _bits(nu) == _bits(f32(4096.0 + 2.0 ** -11))
    sq = (T * T).astype(np.float32)
    assert np.array_equal(sq, TERMS + np.where(np.arange(192) == 129, f32(1), f32(0)) -
                          np.where(np.arange(192) == 128, f32(1), f32(0)))
    for name, Q in wrong_orders(sq).items():
        assert Q >= f32(16777224.0), name
    assert _bits(f32(np.sqrt(np.float64(16777224.0)))) == _bits(f32(4096.0 + 2.0 ** -10))
    # the same vector at an offset: two leading zero blocks make J = 8 (a
    # complete tree): ((0+0)+(1+1)) + ((1+1)+(2+2^24)) = 16777222 again
    T2 = np.concatenate([np.zeros(64, np.float32), T])
    assert _bits(oracle.l2norm(T2)) == _bits(f32(4096.0 + 2.0 ** -11))


# ---- weight step ---------------------------------------------------------------
def test_weight_scale_order_pin():
    """|W| = the terms above with alternating signs, W [4, 48] so that the
    32-wide blocks of the row-major walk cross rows.  S = 16777222;
    mu = S / 192 = 87381.3646 rounds to 87381.3671875 (ulp 2^-7);
    s_w = (2 mu) / fl(sqrt(127)) = 174762.734375 / 11.269427490234375
    = 15507.6855... -> 0x46724ebe.  With S = 16777224 (every wrong order but
    two gives it; the others give more) mu = 87381.375 exactly and s_w =
    0x46724ebf."""
    signs = np.where(np.arange(192) % 3 == 0, f32(-1), f32(1))
    W = (TERMS * signs).reshape(4, 48)
    s_w = oracle.weight_scale(W)
    assert hex(int(_bits(s_w))) == "0x46724ebe"
    assert _bits(f32(np.sqrt(np.float64(127.0)))) == 0x41344F93
    mu_alt = f32(f32(16777224.0) / f32(192.0))
    assert mu_alt == f32(87381.375)
    sw_alt = f32(f32(2.0) * mu_alt) / f32(np.sqrt(np.float64(127.0)))
    assert hex(int(_bits(sw_alt))) == "0x46724ebf"
    for name, S in wrong_orders(TERMS).items():
        assert S >= f32(16777224.0), name


# ---- dX and dW -----------------------------------------------------------------
S_W = f32(2.0 ** -6)     # weight step passed in: q_w = W / 2^-6 exactly


def test_dx_order_pin():
    """dX[m, k] = CanonSum_n(dY[m, n] * What[n, k]) with What = q_w * 2^-6
    exact.  Column 0 of W has q_w = 1, column 1 q_w = 2, and dY row 0 is the
    terms times 2^6, so the products of column 0 are the terms (16777222)
    and those of column 1 twice the terms (every partial sum doubles
    exactly: 33554444).  Row 1 is the negated row (-16777222).  X[1, 2] is
    out of the quantiser's range, so dX[1, 2] = +0."""
    N, K = 192, 3
    W = np.zeros((N, K), np.float32)
    W[:, 0] = S_W
    W[:, 1] = 2 * S_W
    W[:, 2] = S_W
    dY = np.stack([TERMS * f32(64.0), -TERMS * f32(64.0)]).astype(np.float32)
    X = np.zeros((2, K), np.float32)
    X[1, 2] = f32(100.0)                 # 100 / 0.05 = 2000 > 127
    dX = oracle.dx_rows(dY, X, W, 0.05, [0, 1], s_w=S_W)
    want = np.array([[16777222.0, 33554444.0, 16777222.0], [-16777222.0, -33554444.0, 0.0]], np.float32)
    assert np.array_equal(_bits(dX), _bits(want)), dX
    # sensitivity: the products are the terms and their double, which every
    # wrong order sums to other bits
    for name, v in wrong_orders(TERMS * f32(2.0)).items():
        assert _bits(v) != _bits(f32(33554444.0)), name


def test_dw_order_pin_and_microbatches():
    """dW[n, k] = CanonSum_m(dY[m, n] * Xhat[m, k]), Xhat = q_x * s_x with
    s_x = 2^-6: X column 0 is 2^-6 (q_x = 1), column 1 is 2^-5 (q_x = 2),
    and dY column n is the terms times 2^6, so dW = [16777222, 33554444].
    With microbatches of 96 rows the running sum is D = dW_0 + dW_1 with
    dW_0 = CanonSum of the first three blocks = (1 + 1) + 1 = 3 and dW_1 =
    (1 + 2) + 2^24 = 16777219, a tie that rounds to 16777220; then
    3 + 16777220 = 16777223 ties to 16777224."""
    M, K = 192, 2
    X = np.zeros((M, K), np.float32)
    X[:, 0] = f32(2.0 ** -6)
    X[:, 1] = f32(2.0 ** -5)
    W = np.full((2, K), S_W, np.float32)
    dYc = np.stack([TERMS * f32(64.0)] * 2).astype(np.float32)
    dW = oracle.dw_rows(dYc, X, W, 2.0 ** -6, [0, 1], s_w=S_W)
    assert np.array_equal(_bits(dW), _bits(np.array([[16777222.0, 33554444.0]] * 2, np.float32))), dW
    dWmb = oracle.dw_rows(dYc, X, W, 2.0 ** -6, [0, 1], mb=96, s_w=S_W)
    assert _bits(dWmb[0, 0]) == _bits(f32(16777224.0)), dWmb
    # sensitivity: the microbatch split changes the bits, and a running sum
    # started from the second microbatch would too
    assert _bits(dWmb[0, 0]) != _bits(dW[0, 0])
    assert _level(_blocks(TERMS[96:])) == f32(16777220.0)


# ---- attention: the fixed-point format of dQ, dK and dV -----------------------
# One batch entry, one head, S = 160, window 64.  With Q = 0 (case A) or
# K = 0 (case B) every logit is 0, p = E(0) = 1 on the row's keys, and rows
# i >= 63 have l = 64, so P = 1/64 = 2^-6 exactly.  O = 0 makes Delta = +0,
# and s_v = 1 with V in {0, 1} makes V^ = V.  Then
#   dS_ij = 2^-6 * (dP_ij - 0),   dP_ij = sum_d dO_id V_jd,
# and every pinned tile sum is a small multiple of 2^-41 (with K or Q
# entries 2^-35 times small integers).  In units of 2^-41 a tile sum u
# contributes rne(u / 2) to the integer total T, and the output is
# T * 2^-40 (times c = fl(1/fl(sqrt(128))) for dQ and dK).
S_A, D_A, WIN = 160, 128, 64
U = f32(2.0 ** -35)


def _c():
    return f32(f32(1.0) / np.sqrt(f32(128.0)))


def _case_a():
    """Case A (Q = 0): dQ of row 64 and dV of keys 40 and 64."""
    Q = np.zeros((1, S_A, 1, D_A), np.float32)
    K = np.zeros((1, S_A, 1, D_A), np.float32)
    V = np.zeros((1, S_A, 1, D_A), np.float32)
    O = np.zeros((1, S_A, 1, D_A), np.float32)
    dO = np.zeros((1, S_A, 1, D_A), np.float32)
    # row 64 attends keys 1..64; dO_64 = e_0 gives dS_64,j = 2^-6 V_j0
    dO[0, 64, 0, 0] = 1.0
    for j in (10, 31, 32, 63, 64):
        V[0, j, 0, 0] = 1.0
    # dQ_64,d = sum over key tiles g of rne(u_gd / 2) 2^-40 c, with
    # u_gd = sum_{j in tile g} K_jd (in units of 2^-41):
    k = {  # d: {key: multiple of 2^-35}
        0: {10: 1},            # u0 = 1: rne(0.5) = 0 (half away: 1)             T = 0
        1: {10: 3},            # u0 = 3: rne(1.5) = 2 (truncation: 1)             T = 2
        2: {10: 5},            # u0 = 5: rne(2.5) = 2 (half away: 3)              T = 2
        3: {31: 1, 32: 1},     # one 64-tile: u0 = 2 -> 1 (32-tiles: 0 + 0)       T = 1
        4: {63: 1, 64: 1},     # two tiles: 0 + 0 (a tile across 64: 1)           T = 0
        5: {63: 3, 64: 3},     # two tiles: 2 + 2 (one sum: rne(3) = 3)           T = 4
        6: {10: -1},           # rne(-0.5) = -0 -> integer 0                      T = 0
        7: {10: -3},           # rne(-1.5) = -2                                   T = -2
        8: {10: 2},            # u0 = 2 -> 1 (scale 2^32: rne(2^-8) = 0)         T = 1
        9: {10: 2 ** 17, 64: 1},  # u0 = 2^17 -> 2^16; u1 = 1 -> 0               T = 65536
    }
    for d, terms in k.items():
        for j, mult in terms.items():
            K[0, j, 0, d] = f32(mult) * U
    dq_T = {0: 0, 1: 2, 2: 2, 3: 1, 4: 0, 5: 4, 6: 0, 7: -2, 8: 1, 9: 65536}
    # dV_jd = sum over query tiles of rne(w / 2) 2^-40, w = sum over the
    # tile's rows i attending j of 2^-6 dO_id (rows 63: tile 0; 64..127:
    # tile 1; rows 80 and 100 lie in different 32-halves of tile 1)
    dO[0, 63, 0, 1] = U; dO[0, 64, 0, 1] = U            # key 40, d 1: 0 + 0 (one sum: 1)
    dO[0, 80, 0, 2] = U; dO[0, 100, 0, 2] = U           # key 64, d 2: tile 1 u = 2 -> 1 (32-tiles: 0)
    dO[0, 64, 0, 3] = 3 * U                             # key 40, d 3: rne(1.5) = 2
    dO[0, 64, 0, 4] = 5 * U                             # key 40, d 4: rne(2.5) = 2 (half away: 3)
    dO[0, 64, 0, 5] = 2 * U                             # key 40, d 5: 1 (scale 2^32: 0)
    # key 40 is attended by rows 40..103 (rows 63, 64, 80, 100 all of them),
    # key 64 by rows 64..127 (rows 64, 80, 100)
    dv_T = {(40, 1): 0, (40, 2): 1, (40, 3): 2, (40, 4): 2, (40, 5): 1,
            (64, 1): 0, (64, 2): 1, (64, 3): 2, (64, 4): 2, (64, 5): 1}
    return Q, K, V, O, dO, dq_T, dv_T


def test_attention_dq_fixed_point_pin():
    Q, K, V, O, dO, dq_T, _ = _case_a()
    dq = oracle.attn_bwd_dq(Q, K, V, O, dO, WIN, 1.0, rows=[64])[0]
    c = _c()
    for d in range(D_A):
        T = dq_T.get(d, 0)
        want = f32(f32(f32(T) * f32(2.0 ** -40)) * c)
        assert _bits(dq[d]) == _bits(want), (d, dq[d], want)


def test_attention_dv_fixed_point_pin():
    Q, K, V, O, dO, _, dv_T = _case_a()
    _, dv = oracle.attn_bwd_dkdv(Q, K, V, O, dO, WIN, 1.0, rows=[40, 64])
    for (j, d), T in dv_T.items():
        r = 0 if j == 40 else 1
        assert _bits(dv[r, d]) == _bits(f32(T * 2.0 ** -40)), (j, d, dv[r, d])


def test_attention_dk_fixed_point_pin():
    """Case B (K = 0): dK_jd = (sum over query tiles of rne(z / 2)) 2^-40 c
    with z = sum of dS_ij Q_id over the tile's rows.  dO_63 = dO_64 =
    dO_80 = dO_100 = e_0 and V_40,0 = V_64,0 = 1 give dS = 2^-6 at keys 40
    and 64 for each of those rows that attends them."""
    Q = np.zeros((1, S_A, 1, D_A), np.float32)
    K = np.zeros((1, S_A, 1, D_A), np.float32)
    V = np.zeros((1, S_A, 1, D_A), np.float32)
    O = np.zeros((1, S_A, 1, D_A), np.float32)
    dO = np.zeros((1, S_A, 1, D_A), np.float32)
    for i in (63, 64, 80, 100):
        dO[0, i, 0, 0] = 1.0
    V[0, 40, 0, 0] = 1.0
    V[0, 64, 0, 0] = 1.0
    Q[0, 63, 0, 1] = U; Q[0, 64, 0, 1] = U        # key 40: 0 + 0; key 64: row 64 alone, 0
    Q[0, 80, 0, 2] = U; Q[0, 100, 0, 2] = U       # keys 40 and 64: tile 1 u = 2 -> 1 (32-tiles: 0)
    Q[0, 64, 0, 3] = 3 * U                        # keys 40 and 64: rne(1.5) = 2
    Q[0, 64, 0, 4] = 5 * U                        # rne(2.5) = 2
    dk, _ = oracle.attn_bwd_dkdv(Q, K, V, O, dO, WIN, 1.0, rows=[40, 64])
    c = _c()
    want_T = {1: (0, 0), 2: (1, 1), 3: (2, 2), 4: (2, 2)}
    for d in range(D_A):
        for r in (0, 1):
            T = want_T.get(d, (0, 0))[r]
            want = f32(f32(f32(T) * f32(2.0 ** -40)) * c)
            assert _bits(dk[r, d]) == _bits(want), (r, d, dk[r, d], want)


def _format_variants(tiles_units):
    """Integer totals under other fixed-point formats, for lists of tile
    sums in units of 2^-41 (the terms of each 32-half kept apart)."""
    import math

    def rne_half(x):                     # rne(x / 2) for an integer x
        q, r = divmod(x, 2)
        return q + (1 if r and (q % 2) else 0) if r else q

    out = {}
    out["format as read"] = sum(rne_half(sum(h for h in t)) for t in tiles_units)
    out["32-position tiles"] = sum(rne_half(h) for t in tiles_units for h in t)
    out["one sum over all tiles"] = rne_half(sum(h for t in tiles_units for h in t))
    out["scale 2^32"] = sum(round(sum(t) / 2 ** 9) for t in tiles_units)
    out["round half away"] = sum(int(math.copysign(math.floor(abs(sum(t)) / 2 + 0.5), sum(t)))
                                 for t in tiles_units)
    out["truncation"] = sum(int(sum(t) / 2) for t in tiles_units)
    return out


def test_fixed_point_pins_separate_other_formats():
    """Sensitivity of the three pins above: the tile sums they use (in units
    of 2^-41, each tile given as its two 32-halves) under other formats.
    Every alternative format misses at least one pinned total."""
    cases = [  # (tile halves, total as read)
        ([[1, 0]], 0), ([[3, 0]], 2), ([[5, 0]], 2), ([[1, 1]], 1), ([[0, 1], [1, 0]], 0),
        ([[0, 3], [3, 0]], 4), ([[-1, 0]], 0), ([[-3, 0]], -2), ([[2, 0]], 1),
    ]
    missed = {}
    for tiles, total in cases:
        got = _format_variants(tiles)
        assert got["format as read"] == total, (tiles, got)
        for name, v in got.items():
            if name != "format as read" and v != total:
                missed[name] = True
    assert set(missed) == {"32-position tiles", "one sum over all tiles", "scale 2^32", "round half away",
                           "truncation"}, missed
