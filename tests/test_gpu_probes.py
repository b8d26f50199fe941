"""The device probes behind two facts the library relies on.

1. The K = 1 fp32 matrix-core instruction, given a non-zero accumulator
   input, rounds product and sum once (a fused multiply-add).  The method
   rounds every binary32 operation on its own (Open-1B summary on onedev.kr,
   "How": no fused multiply-add), so the backward gives that instruction an
   accumulator of -0 and adds its products on the vector ALU.  The expected
   values here are exact rationals rounded once to binary32 by a helper of
   this file, not by the oracle (the method has no fused operation).

2. The sustained-rate probe that the benchmark times runs the operations it
   claims: with few steps its chains end at values known in closed form.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def round_f32(x: Fraction) -> np.float32:
    """x rounded once to the nearest binary32, ties to even (normal range)."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    x = abs(x)
    e = x.numerator.bit_length() - x.denominator.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    assert -126 <= e <= 127
    scaled = x / Fraction(2) ** (e - 23)            # in [2^23, 2^24)
    q, r = divmod(scaled.numerator, scaled.denominator)
    twice = 2 * r
    if twice > scaled.denominator or (twice == scaled.denominator and q % 2 == 1):
        q += 1
    return np.float32(sign * float(Fraction(q) * Fraction(2) ** (e - 23)))


def _f32(v):
    return np.float32(v)


def test_k1_mfma_with_an_accumulator_rounds_once():
    # crafted: a*a = 1 + 2^-11 + 2^-24; rounding the product first loses the
    # 2^-24 (a tie to even), so the two-rounding result is 0, the fused one 2^-24
    a = [_f32(1 + 2.0 ** -12)]
    b = [_f32(-(1 + 2.0 ** -11))]
    g = np.random.default_rng(11)
    # random pairs with b close to -a*a, where one and two roundings differ most
    x = (g.uniform(1, 2, 4000)).astype(np.float32)
    y = (-(x.astype(np.float64) ** 2) * (1 + g.uniform(-1e-6, 1e-6, 4000))).astype(np.float32)
    a += list(x)
    b += list(y)
    a = np.array(a, np.float32)
    b = np.array(b, np.float32)
    got = brl.probe_f32("mfma_fma", torch.from_numpy(a).to(DEV), torch.from_numpy(b).to(DEV)).cpu().numpy()
    fused = np.array([round_f32(Fraction(float(p)) ** 2 + Fraction(float(q))) for p, q in zip(a, b)], np.float32)
    two = np.array([np.float32(np.float32(p * p) + q) for p, q in zip(a, b)], np.float32)
    assert got[0] == np.float32(2.0 ** -24) and two[0] == 0.0
    assert np.array_equal(got.view(np.uint32), fused.view(np.uint32))
    assert np.count_nonzero(fused != two) > 100      # the set tells the two apart


def _rate_expected(unit: str, iters: int, n: int) -> np.ndarray:
    t = np.arange(n) % 256                            # threadIdx.x
    lane = t % 64
    if unit in ("v_add_f32", "v_mul_f32", "v_add_f32_sgpr"):
        out = np.zeros(n, np.float32)
        for i in range(8):
            x = (t + i) * 0.25 + 1.0 + (0.0 if unit == "v_mul_f32" else 0.5 * iters)
            out = (out + x.astype(np.float32)).astype(np.float32)
        return out
    if unit == "valu_u32":
        gid = np.arange(n, dtype=np.uint32)
        t = np.zeros(n, np.uint32)
        for i in range(8):
            x = gid * np.uint32(8) + np.uint32(i + 1)
            for _ in range(iters):
                x ^= x >> np.uint32(3)
            t ^= x
        return (t & np.uint32(0xFFFFFF)).astype(np.float32)
    if unit in ("mfma_k1_f32", "k1_engine"):
        # c = 0.5: lane l feeds A = 0.5 (l % 8) as row l % 16 of block l / 16 and
        # B = 0.5; it holds rows 4 (l / 16) + e of each block's column l % 16
        rows = 4 * (lane // 16)
        s = sum(((rows + e) % 8) for e in range(4))
        # k1_engine: 4 chains, chain i feeding A = 0.5 (l % 8) (i + 1)
        weight = 8 if unit == "mfma_k1_f32" else 1 + 2 + 3 + 4
        return (weight * 4 * iters * 0.25 * s).astype(np.float32)
    # i8, c = 1: lane l holds bytes (v, v+1, v+2, v+3) of A at bytes 0, 4, 8, 12
    # and (v+4, v, v+1, v+2) of B, v = 1 + l % 4; row i of A comes from lanes i
    # and i + 32, column j of B likewise, so D[i][j] depends on i % 4, j % 4
    def d(vi, vj):
        return 2 * (vi * (vj + 4) + (vi + 1) * vj + (vi + 2) * (vj + 1) + (vi + 3) * (vj + 2))
    vj = 1 + (lane % 32) % 4
    col = sum(d(1 + a, vj) for a in range(4)) * 4     # each row residue 4 times among 16 rows
    return (8 * iters * col).astype(np.float32)


def _i8_data_wave_sums(iters: int, n: int) -> np.ndarray:
    """Per-wave sums of the data-toggling i8 probe's outputs, mod 2^24.

    Fragment f of lane l holds 16 bytes (byte 4k + m = byte m of its register
    k); A fragments are f < 16, B fragments f >= 16, and each step runs, for
    p = 0..3, the grid A_{4p+i} x B_{16+2p+j}.  Rows of A come from lanes i
    and i + 32 (columns of B likewise) with the same byte-to-k assignment for
    A and B, so the sum of all 32 x 32 outputs of one MFMA is, whatever that
    assignment, the sum over the lane half h and byte b of (sum of A's bytes
    over the 32 lanes of h) x (the same for B)."""
    gid = np.arange(n, dtype=np.uint32)
    fr = []
    with np.errstate(over="ignore"):            # uint32 arithmetic wraps, as on the device
        for f in range(24):
            regs = []
            for k in range(4):
                x = (gid + np.uint32(1)) * np.uint32(0x9E3779B1) + np.uint32(4 * f + k + 1) * np.uint32(0x85EBCA77)
                x = x ^ (x << np.uint32(13))
                x = x ^ (x >> np.uint32(17))
                x = x ^ (x << np.uint32(5))
                regs.append(x)
            # [waves, half, 32 lanes, 16 bytes] -> byte sums over the lanes of a half
            fr.append(np.stack(regs, axis=1).view(np.int8).reshape(n // 64, 2, 32, 16).astype(np.int64).sum(axis=2))
    total = np.zeros(n // 64, np.int64)
    for p in range(4):
        for q in range(8):
            total += (fr[4 * p + q // 2] * fr[16 + 2 * p + q % 2]).sum(axis=(1, 2))
    return (iters * total) % (1 << 24)


def test_i8_probe_with_changing_operands_computes_its_products():
    iters = 40
    out = brl.probe_rate("mfma_i8_data", iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.int64).reshape(-1, 64).sum(axis=1) % (1 << 24)
    want = _i8_data_wave_sums(iters, out.numel())
    assert np.array_equal(got, want), (got[:4], want[:4])


def _k1_data_threads(iters: int, gids: np.ndarray) -> np.ndarray:
    """Outputs of the data-toggling product-engine probe for whole waves.

    Operand f of side ab (0: A, 1: B) of thread g is the binary32 with the
    sign and significand of xorshift(hash(g, 2f + ab)) and exponent 0.  In
    the 4-block 16x16x1 MFMA, lane l, register 4b + e receives block b's
    row 4(l / 16) + e, column l % 16: the product of A from lane
    16b + 4(l / 16) + e and B from lane 16b + l % 16.  Chain i adds, per
    step and round u, the products of operand pair 4u + i; the output is
    the sum of the 64 chain values, chain by chain, register by register.
    Every product and sum is rounded to binary32 by numpy."""
    g = gids.astype(np.uint32)
    vals = {}
    with np.errstate(over="ignore"):
        for f in range(16):
            for ab in range(2):
                x = (g + np.uint32(1)) * np.uint32(0x9E3779B1) + np.uint32(2 * f + ab + 1) * np.uint32(0x85EBCA77)
                x = x ^ (x << np.uint32(13))
                x = x ^ (x >> np.uint32(17))
                x = x ^ (x << np.uint32(5))
                vals[f, ab] = ((x & np.uint32(0x807FFFFF)) | np.uint32(0x3F800000)).view(np.float32).reshape(-1, 64)
    lane = np.arange(64)
    # [lane, register] -> source lanes of A and B
    src_a = np.array([[16 * (r // 4) + 4 * (l // 16) + r % 4 for r in range(16)] for l in lane])
    src_b = np.array([[16 * (r // 4) + l % 16 for r in range(16)] for l in lane])
    acc = np.zeros((4, len(gids) // 64, 64, 16), np.float32)
    prods = [(vals[f, 0][:, src_a] * vals[f, 1][:, src_b]).astype(np.float32) for f in range(16)]
    for _ in range(iters):
        for u in range(4):
            for i in range(4):
                acc[i] = (acc[i] + prods[4 * u + i]).astype(np.float32)
    out = np.zeros((len(gids) // 64, 64), np.float32)
    for i in range(4):
        for r in range(16):
            out = (out + acc[i][:, :, r]).astype(np.float32)
    return out.reshape(-1)


def test_product_engine_probe_with_changing_operands_computes_its_sums():
    iters = 40
    out = brl.probe_rate("k1_engine_data", iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # whole waves from the first, a middle and the last workgroup
    gids = np.concatenate([np.arange(0, 256), np.arange(2048 * 256, 2048 * 256 + 256),
                           np.arange(got.size - 256, got.size)])
    want = _k1_data_threads(iters, gids)
    assert np.array_equal(got[gids].view(np.uint32), want.view(np.uint32)), (got[gids][:4], want[:4])


@pytest.mark.parametrize("unit", [u for u in brl.RATE_UNITS if u not in ("mfma_i8_data", "k1_engine_data")])
def test_rate_probe_chains_end_where_they_should(unit):
    iters = 40
    out = brl.probe_rate(unit, iters)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    want = _rate_expected(unit, iters, got.size)
    assert got.size == 4096 * 256
    assert np.array_equal(got, want), (unit, got[:4], want[:4])
