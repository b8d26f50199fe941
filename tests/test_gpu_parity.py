"""GPU parity of the HIP path against the CPU oracle, element by element, at
0 ULP (bitwise equality of every output).  Small and ragged sizes that span
several tiles; every call goes through the C ABI.

Tolerance: none.  The method defines each output by its exact sequence of
binary32 operations (Open-1B summary on onedev.kr, "How"), so the only
correct result is the oracle's bit pattern.
"""
import numpy as np
import pytest
import torch

import bitwise_reproducible_lsq_amd as brl
import oracle
import synth

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _bits(x):
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, np.float32).view(np.uint32)


def assert_bitwise(got, want, what):
    g, w = _bits(got), _bits(want)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.flatnonzero(g.ravel() != w.ravel())
    if bad.size:
        i = bad[0]
        raise AssertionError(f"{what}: {bad.size} of {g.size} differ; first at flat {i}: "
                             f"got {g.ravel()[i]:#010x} want {w.ravel()[i]:#010x}")


def _cuda(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _case_inputs(M, K, N, seed, sub=0.0, swiglu=False, x_kind="normal"):
    case = synth.small_case(f"s{seed}", seed, M, K, N, subnormal_frac=sub, swiglu=swiglu, x_kind=x_kind)
    return synth.linear_inputs(case)


# ---- binary32 conformance of the device operations --------------------------------
def _probe_inputs(n, seed):
    g = np.random.default_rng(seed)
    a = (g.standard_normal(n) * np.exp(g.uniform(-40, 40, n))).astype(np.float32)
    b = (g.standard_normal(n) * np.exp(g.uniform(-40, 40, n))).astype(np.float32)
    tiny = np.float32(np.finfo(np.float32).tiny)
    directed = [
        (np.float32(1 - 2.0 ** -24), tiny),          # tiny at 24 bits: flushed
        (np.float32(1 - 2.0 ** -23), tiny),          # exact subnormal product (flushed)
        (np.float32(0.96875), np.float32(1082401 * 2.0 ** -146)),   # 2^-126(1-2^-25): rounds up, kept
        (np.float32(-0.96875), np.float32(1082401 * 2.0 ** -146)),
        (np.float32(1e-20), np.float32(-1e-20)),     # -0 after flush
        (np.float32(1.5) * tiny, -tiny),             # exact subnormal sum
        (np.float32(1e-40), np.float32(1.0)),        # subnormal operand
        (np.float32(-1e-40), np.float32(-0.0)),
        (tiny, np.float32(1.0 + 2.0 ** -23)),        # quotient just below 2^-126 (div)
        (np.float32(3.0), np.float32(7.0)),
        (np.float32(1.0 + 2.0 ** -12), np.float32(1.0 + 2.0 ** -12)),
    ]
    for i, (x, y) in enumerate(directed):
        a[i], b[i] = x, y
    return a, b


@pytest.mark.parametrize("op", ["add", "sub", "mul", "div", "sqrt", "rne", "exp", "mfma_mul"])
def test_device_binary32_ops_match_oracle(op):
    a, b = _probe_inputs(20000, 3)
    if op == "sqrt":
        a = np.abs(a)
    if op == "rne":
        a = (np.random.default_rng(5).standard_normal(20000) * 300).astype(np.float32)
        a[:521] = (np.arange(-260, 261) / 2).astype(np.float32)
    if op == "exp":
        a = np.random.default_rng(6).uniform(-110, 95, 20000).astype(np.float32)
        # the range ends, the special values and the signed zeros
        edge = [89.0, np.nextafter(np.float32(89), np.float32(90)), np.nextafter(np.float32(89), np.float32(0)),
                -104.0, np.nextafter(np.float32(-104), np.float32(-105)),
                np.nextafter(np.float32(-104), np.float32(0)), 0.0, -0.0, np.inf, -np.inf, np.nan, 1e-30, -1e-30]
        a[:len(edge)] = np.array(edge, np.float32)
    got = brl.probe_f32(op, _cuda(a), _cuda(b)).cpu().numpy()
    fn = {"add": oracle.add, "sub": oracle.sub, "mul": oracle.mul, "mfma_mul": oracle.mul, "div": oracle.div,
          "sqrt": lambda x, y: oracle.sqrt(x), "rne": lambda x, y: oracle.rne(x),
          "exp": lambda x, y: oracle.exp(x)}[op]
    want = np.array([fn(x, y) for x, y in zip(a, b)], np.float32)
    nan = np.isnan(got) & np.isnan(want)
    bad = np.flatnonzero((_bits(got) != _bits(want)) & ~nan)
    assert bad.size == 0, [(a[i], b[i], got[i], want[i]) for i in bad[:5]]


def test_matrix_core_products_on_crafted_classes():
    """The matrix-core product equals the oracle's binary32 product on classes
    aimed at its corners: random bit patterns, products around 2^-126 (the FTZ
    band where tininess after rounding keeps a normal result), subnormal
    operands, signed zeros, overflow, and products that are exact ties."""
    g = np.random.default_rng(8)
    n = 1 << 16
    sign = lambda: g.integers(0, 2, n, dtype=np.uint32) << 31
    man = lambda: g.integers(0, 1 << 23, n, dtype=np.uint32)
    classes = []
    ea = g.integers(1, 255, n, dtype=np.uint32); eb = g.integers(1, 255, n, dtype=np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (eb << 23) | man()))
    ea = g.integers(1, 127, n, dtype=np.uint32); eb = 127 - ea + g.integers(0, 3, n, dtype=np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (eb << 23) | man()))
    ea = np.where(g.integers(0, 2, n) == 1, 0, 100).astype(np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (np.uint32(127) << 23) | man()))
    z = np.where(g.integers(0, 3, n) == 0, 0, np.uint32(127) << 23).astype(np.uint32)
    classes.append((sign() | z | np.where(z == 0, 0, man()).astype(np.uint32), sign() | (np.uint32(127) << 23) | man()))
    ea = g.integers(190, 255, n, dtype=np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (ea << 23) | man()))
    ea = g.integers(120, 135, n, dtype=np.uint32)
    classes.append((sign() | (ea << 23) | (man() & 0x7FF000), sign() | (ea << 23) | (man() & 0x7FF800)))
    for i, (ua, ub) in enumerate(classes):
        a, b = ua.view(np.float32), ub.view(np.float32)
        got = brl.probe_f32("mfma_mul", _cuda(a), _cuda(b)).cpu().numpy()
        want = np.array([oracle.mul(x, y) for x, y in zip(a, b)], np.float32)
        nan = np.isnan(got) & np.isnan(want)
        bad = np.flatnonzero((_bits(got) != _bits(want)) & ~nan)
        assert bad.size == 0, (i, [(hex(ua[k]), hex(ub[k]), got[k], want[k]) for k in bad[:5]])


def test_device_int_to_float_rne():
    ints = np.array([0, 1, -1, 2**24 + 1, 2**24 + 3, 2**31 - 1, -2**31, 90_832_001, -16_777_217], np.int32)
    got = brl.probe_f32("i2f", _cuda(ints.view(np.float32))).cpu().numpy()
    want = np.array([oracle.i2f(int(v)) for v in ints], np.float32)
    assert_bitwise(got, want, "i2f")


# ---- linear layer: forward ------------------------------------------------------------
SHAPES = [
    (256, 512, 512),     # the tiny workload's shape
    (300, 200, 130),     # ragged in every dimension
    (1, 7, 3),
    (257, 64, 256),
    (64, 1000, 96),
    (513, 96, 300),
]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_fwd_parity(M, K, N):
    inp = _case_inputs(M, K, N, seed=M + K + N)
    X, W = _cuda(inp.X), _cuda(inp.W)
    Y, _, s_w = brl.qat_linear_fwd(X, W, synth.S_X)
    torch.cuda.synchronize()
    assert_bitwise(s_w, np.array([oracle.weight_scale(inp.W)]), "s_w")
    assert_bitwise(Y, oracle.linear_fwd(inp.X, inp.W, synth.S_X), "Y")


def test_fwd_tiny_workload():
    inp = synth.linear_inputs(synth.CASES["tiny"])
    Y, _, s_w = brl.qat_linear_fwd(_cuda(inp.X), _cuda(inp.W), synth.S_X)
    assert_bitwise(Y, oracle.linear_fwd(inp.X, inp.W, synth.S_X), "Y")


def test_fwd_addend():
    inp = _case_inputs(130, 70, 90, seed=9)
    add = np.random.default_rng(1).standard_normal((130, 90)).astype(np.float32)
    Y, _, _ = brl.qat_linear_fwd(_cuda(inp.X), _cuda(inp.W), synth.S_X, addend=_cuda(add))
    assert_bitwise(Y, oracle.linear_fwd(inp.X, inp.W, synth.S_X, addend=add), "Y+C")


# (256, 512, 512) and (512, 128, 1024) are whole 256 x 256 tiles (the
# epilogue's branch-free path); (300, 64, 640) mixes whole tiles with tiles
# cut by M and by the gate columns in one launch
@pytest.mark.parametrize("want_ypre", [True, False])
@pytest.mark.parametrize("M,K,N", [(200, 96, 256), (70, 64, 198), (256, 512, 512), (512, 128, 1024), (300, 64, 640)])
def test_fwd_swiglu_parity(M, K, N, want_ypre):
    inp = _case_inputs(M, K, N, seed=11, swiglu=True)
    Y, Ypre, _ = brl.qat_linear_fwd(_cuda(inp.X), _cuda(inp.W), synth.S_X, epilogue=brl.EPILOGUE_SWIGLU,
                                    want_ypre=want_ypre)
    wantY, wantPre = oracle.linear_fwd(inp.X, inp.W, synth.S_X, epilogue=1)
    if want_ypre:
        assert_bitwise(Ypre, wantPre, "Ypre")
    else:
        assert Ypre is None
    assert_bitwise(Y, wantY, "SwiGLU(Y)")


def test_fwd_zero_weights_and_empty_rows():
    X = np.random.default_rng(0).standard_normal((40, 32)).astype(np.float32)
    W = np.zeros((24, 32), np.float32)
    Y, _, s_w = brl.qat_linear_fwd(_cuda(X), _cuda(W), synth.S_X)
    assert float(s_w.item()) == 0.0
    assert_bitwise(Y, oracle.linear_fwd(X, W, synth.S_X), "Y (zero W)")
    W = np.random.default_rng(1).standard_normal((24, 32)).astype(np.float32)
    Y, _, s_w = brl.qat_linear_fwd(_cuda(np.zeros((0, 32), np.float32)), _cuda(W), synth.S_X)
    assert Y.shape == (0, 24)
    assert_bitwise(s_w, np.array([oracle.weight_scale(W)]), "s_w (M=0)")


# The forward's preparation (weight step, W codes, X codes) runs as one launch
# by default and as separate launches with fwd_prep=2.  The in-launch tail
# reduces the |W| run roots with 1, 2, 4, 8 or 16 roots per thread depending
# on their count P (P <= 256, 512, 1024, 2048, 4096): the shapes below reach
# every one, with a short last run where N*K is not a multiple of 8192.
PREP_SHAPES = [
    (70, 1000, 1500),     # P = 184, short last run
    (64, 2048, 1100),     # P = 275
    (96, 2048, 3000),     # P = 750
    (64, 2048, 6000),     # P = 1500
    (64, 4096, 4500),     # P = 2250
    (300, 64, 9),         # P = 1 (the single run is also the last)
]


@pytest.mark.parametrize("M,K,N", PREP_SHAPES)
def test_fwd_prep_one_launch(M, K, N):
    g = np.random.default_rng(M * 7 + N)
    W = (g.standard_normal((N, K)) * np.exp(g.uniform(-3, 3, (N, 1)))).astype(np.float32)
    X = g.standard_normal((M, K)).astype(np.float32)
    Xd, Wd = _cuda(X), _cuda(W)
    Y1, _, s1 = brl.qat_linear_fwd(Xd, Wd, synth.S_X)
    Y2, _, s2 = brl.qat_linear_fwd(Xd, Wd, synth.S_X, tune=brl.Tuning(fwd_prep=2))
    torch.cuda.synchronize()
    assert_bitwise(s1, np.array([oracle.weight_scale(W)]), "s_w (one launch)")
    assert_bitwise(s2, np.array([oracle.weight_scale(W)]), "s_w (separate launches)")
    assert_bitwise(Y1, Y2, "Y one launch vs separate launches")
    rows = np.unique(np.r_[0, M // 2, M - 1])
    assert_bitwise(Y1[rows], oracle.fwd_rows(X[rows], W, synth.S_X), "Y rows")


def test_fwd_accumulator_at_the_int32_limit():
    """K = 133144, the largest K the forward accepts: rows of X whose codes
    are all +127 or all -127 against a weight row whose codes are all 127
    (the other rows zero, so the weight step is small) give |acc| =
    127 * 127 * K = 2147479576, within 6071 of 2^31 - 1; the remaining rows
    and columns are mixed.  Every element against the oracle."""
    M, K, N = 5, 133144, 25
    g = np.random.default_rng(21)
    X = g.standard_normal((M, K)).astype(np.float32)
    X[0] = 10.0                      # t = 200: code +127
    X[1] = -10.0                     # code -127
    X[2, ::2] = 10.0                 # alternating +127 / normal
    W = np.zeros((N, K), np.float32)
    W[0] = 1.0                       # mean |w| = 1/25: t = 140.8, code 127
    W[3] = (g.standard_normal(K) * 0.02).astype(np.float32)
    Y, _, s_w = brl.qat_linear_fwd(_cuda(X), _cuda(W), synth.S_X)
    torch.cuda.synchronize()
    assert_bitwise(s_w, np.array([oracle.weight_scale(W)]), "s_w")
    want = oracle.linear_fwd(X, W, synth.S_X)
    assert_bitwise(Y, want, "Y")
    # the extreme sums really are there: acc = +-127^2 K before the scale
    s_y = np.float32(np.float32(synth.S_X) * np.float32(oracle.weight_scale(W)))
    assert want[0, 0] == np.float32(np.float32(127 * 127 * K) * s_y)
    assert want[1, 0] == -want[0, 0]


@pytest.mark.parametrize("N", [8192, 8200])
def test_fwd_prep_largest_one_launch_and_beyond(N):
    """N*K = 2^25 is the largest weight count one launch prepares (4096 run
    roots, 16 per thread of its tail); one more row takes the separate
    launches.  s_w and sampled rows of Y against the oracle."""
    M, K = 64, 4096
    g = np.random.default_rng(N)
    W = (g.standard_normal((N, K)) * 0.02).astype(np.float32)
    X = g.standard_normal((M, K)).astype(np.float32)
    Y, _, s_w = brl.qat_linear_fwd(_cuda(X), _cuda(W), synth.S_X)
    torch.cuda.synchronize()
    assert_bitwise(s_w, np.array([oracle.weight_scale(W)]), "s_w")
    rows = np.array([0, 37, M - 1])
    assert_bitwise(Y[rows], oracle.fwd_rows(X[rows], W, synth.S_X), "Y rows")


def test_fwd_prep_unaligned_weights_and_reused_workspace():
    """W 4 bytes off a 16-byte boundary takes the per-thread block path in
    every run; one workspace serves calls with different weights in a row
    (the launch clears the counter and flag it leaves behind)."""
    M, K, N = 130, 96, 700
    g = np.random.default_rng(5)
    X = g.standard_normal((M, K)).astype(np.float32)
    Xd = _cuda(X)
    ws = brl.workspace(brl.OP_FWD, M, K, N, DEV)
    for rep, scale in enumerate((1.0, 0.003, 40.0)):
        W = (g.standard_normal((N, K)) * scale).astype(np.float32)
        buf = torch.empty(N * K + 1, dtype=torch.float32, device=DEV)
        Wd = buf[1:].view(N, K)
        Wd.copy_(_cuda(W))
        assert Wd.data_ptr() % 16 == 4
        Y, _, s_w = brl.qat_linear_fwd(Xd, Wd, synth.S_X, ws=ws)
        torch.cuda.synchronize()
        assert_bitwise(s_w, np.array([oracle.weight_scale(W)]), f"s_w call {rep}")
        assert_bitwise(Y, oracle.linear_fwd(X, W, synth.S_X), f"Y call {rep}")


def test_fwd_prep_swiglu_separate_launches():
    inp = _case_inputs(200, 96, 256, seed=12, swiglu=True)
    Y, Ypre, _ = brl.qat_linear_fwd(_cuda(inp.X), _cuda(inp.W), synth.S_X, epilogue=brl.EPILOGUE_SWIGLU,
                                    tune=brl.Tuning(fwd_prep=2))
    wantY, wantPre = oracle.linear_fwd(inp.X, inp.W, synth.S_X, epilogue=1)
    assert_bitwise(Ypre, wantPre, "Ypre")
    assert_bitwise(Y, wantY, "SwiGLU(Y)")


def _boundary_inputs(s, seed, rows=48, cols=96):
    """X whose quotients by the step s sit within a few ulp of the points
    where the quantiser's result changes: the rounding midpoints k + 1/2 and
    the range ends +-127, +-127.5; the rest of X is N(0, 1)."""
    s = np.float32(s)
    vals = []
    for t in [k + 0.5 for k in range(-128, 128)] + [-127.0, 127.0]:
        v = np.float32(np.float64(t) * np.float64(s)).view(np.int32)
        vals += [np.int32(v + d).view(np.float32) for d in range(-3, 4)]
    vals = np.array(vals, np.float32)
    X = np.random.default_rng(seed).standard_normal(rows * cols).astype(np.float32)
    X[:vals.size] = vals
    return X.reshape(rows, cols), vals


@pytest.mark.parametrize("s", [0.05, 0.0371, 1.0 / 3.0, 2.5e-3])
def test_quantizer_at_rounding_boundaries(s):
    """Forward (q_x) and backward (the STE mask of X) on inputs whose
    quotients v/s lie next to rounding midpoints.  The CPU check first shows
    the set is sensitive: a quotient formed as v * fl32(1/s) changes some
    codes, so a kernel taking that shortcut would fail here."""
    from fractions import Fraction
    X, vals = _boundary_inputs(s, seed=int(s * 1e4))
    sf = np.float32(s)
    exact = [Fraction(float(v)) / Fraction(float(sf)) for v in vals]
    naive = [np.float32(v * np.float32(np.float32(1.0) / sf)) for v in vals]
    correct = [np.float32(float(q)) for q in exact]      # round-to-nearest of the exact quotient
    assert any(np.rint(a) != np.rint(b) for a, b in zip(naive, correct)), \
        "boundary set does not separate the shortcut"
    assert all(np.float32(oracle.div(v, sf)) == c for v, c in zip(vals, correct))
    W = np.random.default_rng(3).standard_normal((80, X.shape[1])).astype(np.float32) * np.float32(0.02)
    Y, _, _ = brl.qat_linear_fwd(_cuda(X), _cuda(W), float(sf))
    assert_bitwise(Y, oracle.linear_fwd(X, W, sf), "Y")
    dY = np.random.default_rng(4).standard_normal((X.shape[0], 80)).astype(np.float32) * np.float32(1e-3)
    wX, wW = oracle.linear_bwd(dY, X, W, sf)
    for engine in ENGINES:
        dX, dW = brl.qat_linear_bwd(_cuda(dY), _cuda(X), _cuda(W), float(sf), tune=brl.Tuning(bwd_engine=engine))
        assert_bitwise(dX, wX, f"dX (engine {engine})")
        assert_bitwise(dW, wW, f"dW (engine {engine})")


# ---- linear layer: backward -----------------------------------------------------------
ENGINES = [1, 2]   # products on the VALU / on the matrix cores


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_bwd_parity(M, K, N, engine):
    inp = _case_inputs(M, K, N, seed=M * 3 + K + N, sub=0.01)
    dX, dW = brl.qat_linear_bwd(_cuda(inp.dY), _cuda(inp.X), _cuda(inp.W), synth.S_X,
                                tune=brl.Tuning(bwd_engine=engine))
    wX, wW = oracle.linear_bwd(inp.dY, inp.X, inp.W, synth.S_X)
    assert_bitwise(dX, wX, f"dX (engine {engine})")
    assert_bitwise(dW, wW, f"dW (engine {engine})")


@pytest.mark.parametrize("M,K,N", [(300, 200, 132), (97, 64, 36), (40, 256, 4)])
def test_bwd_matrix_core_ragged_reductions(M, K, N):
    """Reductions that end inside a 32-block (M and N not multiples of 32)
    on the matrix-core engine (N % 4 == 0), and the same call with dY at a
    4-byte but not 16-byte aligned address, which runs the VALU engine."""
    inp = _case_inputs(M, K, N, seed=M + 7 * N, sub=0.01)
    wX, wW = oracle.linear_bwd(inp.dY, inp.X, inp.W, synth.S_X)
    X, W = _cuda(inp.X), _cuda(inp.W)
    mc = brl.Tuning(bwd_engine=2)
    dX, dW = brl.qat_linear_bwd(_cuda(inp.dY), X, W, synth.S_X, tune=mc)
    assert_bitwise(dX, wX, "dX")
    assert_bitwise(dW, wW, "dW")
    flat = torch.empty(M * N + 1, dtype=torch.float32, device="cuda")
    dY_odd = flat[1:].view(M, N)
    dY_odd.copy_(_cuda(inp.dY))
    assert dY_odd.data_ptr() % 16 != 0
    dX, dW = brl.qat_linear_bwd(dY_odd, X, W, synth.S_X, tune=mc)
    assert_bitwise(dX, wX, "dX (unaligned dY)")
    assert_bitwise(dW, wW, "dW (unaligned dY)")


def test_bwd_finish_alignment_paths():
    """The chunk-root finish reads the mask source and writes the output as
    16-byte vectors only when both are 16-byte aligned; tensors at 4-byte but
    not 16-byte aligned addresses take its per-element path.  Both give the
    oracle's bits, also when dW accumulates (dW + dW = 2 dW exactly, the
    oracle's outputs being normal numbers or zeros)."""
    M, K, N = 300, 72, 200
    inp = _case_inputs(M, K, N, seed=77, sub=0.01)
    wX, wW = oracle.linear_bwd(inp.dY, inp.X, inp.W, synth.S_X)

    def odd(a):
        flat = torch.empty(a.size + 1, dtype=torch.float32, device="cuda")
        t = flat[1:].view(*a.shape)
        t.copy_(_cuda(a))
        assert t.data_ptr() % 16 != 0
        return t

    dY = _cuda(inp.dY)
    cases = [("aligned", _cuda(inp.X), _cuda(inp.W), False),
             ("mask sources unaligned", odd(inp.X), odd(inp.W), False),
             ("outputs unaligned", _cuda(inp.X), _cuda(inp.W), True)]
    tune = brl.Tuning(bwd_chunk_log2=1)      # several chunk roots per output at this size
    for what, X, W, odd_out in cases:
        if odd_out:
            dX, dW = odd(np.zeros((M, K), np.float32)), odd(np.zeros((N, K), np.float32))
        else:
            dX = torch.empty((M, K), dtype=torch.float32, device="cuda")
            dW = torch.empty((N, K), dtype=torch.float32, device="cuda")
        brl.qat_linear_bwd(dY, X, W, synth.S_X, dX=dX, dW=dW, tune=tune)
        assert_bitwise(dX, wX, f"dX ({what})")
        assert_bitwise(dW, wW, f"dW ({what})")
        brl.qat_linear_bwd(dY, X, W, synth.S_X, need_dX=False, dW=dW, dW_accumulate=True, tune=tune)
        assert_bitwise(dW, np.float32(2) * wW, f"dW accumulated ({what})")


def test_bwd_tiny_workload():
    inp = synth.linear_inputs(synth.CASES["tiny"])
    dX, dW = brl.qat_linear_bwd(_cuda(inp.dY), _cuda(inp.X), _cuda(inp.W), synth.S_X)
    wX, wW = oracle.linear_bwd(inp.dY, inp.X, inp.W, synth.S_X)
    assert_bitwise(dX, wX, "dX")
    assert_bitwise(dW, wW, "dW")


@pytest.mark.parametrize("engine", ENGINES)
def test_bwd_long_reductions_and_masks(engine):
    """Reductions of many blocks (several chunks and a ragged tail) and
    activations that clip (mask false)."""
    M, K, N = 2100, 40, 1100
    inp = _case_inputs(M, K, N, seed=21, x_kind="silu_x_normal")
    X = inp.X * np.float32(2.0)
    assert (np.abs(X / synth.S_X) > 127).any()
    dX, dW = brl.qat_linear_bwd(_cuda(inp.dY), _cuda(X), _cuda(inp.W), synth.S_X, tune=brl.Tuning(bwd_engine=engine))
    wX, wW = oracle.linear_bwd(inp.dY, X, inp.W, synth.S_X)
    assert_bitwise(dX, wX, "dX")
    assert_bitwise(dW, wW, "dW")


@pytest.mark.parametrize("engine", ENGINES)
def test_bwd_swiglu_parity(engine):
    M, K, N = 160, 96, 192
    inp = _case_inputs(M, K, N, seed=31, swiglu=True)
    X, W = _cuda(inp.X), _cuda(inp.W)
    _, Ypre, _ = brl.qat_linear_fwd(X, W, synth.S_X, epilogue=brl.EPILOGUE_SWIGLU)
    dX, dW = brl.qat_linear_bwd(_cuda(inp.dY), X, W, synth.S_X, Ypre=Ypre, epilogue=brl.EPILOGUE_SWIGLU,
                                tune=brl.Tuning(bwd_engine=engine))
    _, wPre = oracle.linear_fwd(inp.X, inp.W, synth.S_X, epilogue=1)
    G = oracle.swiglu_bwd(wPre, inp.dY)
    wX, wW = oracle.linear_bwd(G, inp.X, inp.W, synth.S_X)
    assert_bitwise(dX, wX, "dX")
    assert_bitwise(dW, wW, "dW")


@pytest.mark.parametrize("engine", ENGINES)
def test_bwd_microbatch_running_sum(engine):
    M, K, N, B = 4 * 96, 72, 80, 4
    inp = _case_inputs(M, K, N, seed=41)
    X, W, dY = _cuda(inp.X), _cuda(inp.W), _cuda(inp.dY)
    mb = M // B
    dW = None
    for b in range(B):
        _, dW = brl.qat_linear_bwd(dY[b * mb:(b + 1) * mb], X[b * mb:(b + 1) * mb], W, synth.S_X,
                                   need_dX=False, dW=dW, dW_accumulate=b > 0, tune=brl.Tuning(bwd_engine=engine))
    want = oracle.dw_rows(np.ascontiguousarray(inp.dY.T), inp.X, inp.W, synth.S_X, np.arange(N), mb=mb)
    assert_bitwise(dW, want, "dW (4 microbatches)")


def test_bwd_empty_rows():
    W = np.random.default_rng(2).standard_normal((24, 32)).astype(np.float32) * np.float32(0.02)
    z = np.zeros((0, 32), np.float32)
    dX, dW = brl.qat_linear_bwd(_cuda(np.zeros((0, 24), np.float32)), _cuda(z), _cuda(W), synth.S_X)
    assert dX.shape == (0, 32)
    assert_bitwise(dW, np.zeros((24, 32), np.float32), "dW (M=0)")


def test_bwd_launch_shape_invariance():
    """The chunking of the reduction and the CanonSum workgroup size change
    only the launch shape: every setting gives the oracle's bits."""
    M, K, N = 1500, 64, 700
    inp = _case_inputs(M, K, N, seed=51)
    wX, wW = oracle.linear_bwd(inp.dY, inp.X, inp.W, synth.S_X)
    X, W, dY = _cuda(inp.X), _cuda(inp.W), _cuda(inp.dY)
    for e in ENGINES:
        for c, r in [(1, 64), (2, 128), (3, 256), (4, 64), (5, 128), (6, 256), (7, 64)]:
            tune = brl.Tuning(bwd_chunk_log2=c, reduce_wg_blocks=r, bwd_engine=e)
            dX, dW = brl.qat_linear_bwd(dY, X, W, synth.S_X, tune=tune)
            assert_bitwise(dX, wX, f"dX chunk=2^{c} wg={r} engine={e}")
            assert_bitwise(dW, wW, f"dW chunk=2^{c} wg={r} engine={e}")


def test_repeat_runs_identical():
    inp = _case_inputs(700, 128, 300, seed=61)
    X, W, dY = _cuda(inp.X), _cuda(inp.W), _cuda(inp.dY)
    ref = None
    for _ in range(5):
        Y, _, _ = brl.qat_linear_fwd(X, W, synth.S_X)
        dX, dW = brl.qat_linear_bwd(dY, X, W, synth.S_X)
        cur = [_bits(t).copy() for t in (Y, dX, dW)]
        if ref is None:
            ref = cur
        for a, b in zip(ref, cur):
            assert (a == b).all()


# ---- replay -----------------------------------------------------------------------------
def _replay_gpu(partials_np, R, S, max_norm=1.0, persist=False, tune=None, resident=False):
    L = partials_np[0].size
    st = brl.ReduceState(R, S, L, device=DEV, partials_persist=persist, tune=tune, replica_resident=resident)
    out = None
    keep = []      # with persist the shard-0 partials must outlive the shard-1 call
    for v in range(R * S):
        g = _cuda(partials_np[v])
        keep.append(g)
        out = brl.ordered_reduce(st, g)
    nu = brl.grad_l2norm_clip(out, max_norm, tune=tune)
    torch.cuda.synchronize()
    return out, nu, st


@pytest.mark.parametrize("mode", ["plain", "persist", "resident"])
@pytest.mark.parametrize("R,S,L", [(6, 8, 65536 + 5), (1, 1, 1000), (2, 3, 4097), (3, 2, 333),
                                   (5, 1, 1024), (7, 2, 100), (16, 2, 2048), (6, 8, 3), (6, 11, 4099),
                                   (3, 64, 257), (2, 65, 130), (1, 4, 1001), (64, 2, 33)])
def test_replay_parity(R, S, L, mode):
    """Every running sum A_r (but the last, which the fold consumes) and the
    clipped TreeFold, with the partials streamed one call at a time, with each
    replica's shard-0 partial kept until its shard-1 call, and with every
    partial of a replica kept until its last shard's call (one pass per
    replica; 65 shards exceed the pointer table and take the persist path)."""
    parts = [synth.replay_partial_host(4, v, L, std=1e-2) for v in range(R * S)]
    out, nu, st = _replay_gpu(parts, R, S, persist=mode == "persist", resident=mode == "resident")
    T, wnu, A = oracle.replay(parts, R, S)
    assert_bitwise(nu, np.array([wnu]), "nu")
    assert_bitwise(out, T, "clipped TreeFold")
    for r in range(R - 1):      # the last replica's running sum is fused into the fold
        if S > 1 or r < R - 1:
            assert_bitwise(st.acc[r], A[r], f"A_{r}")
    with pytest.raises(brl.BrlError) as e:
        brl.ordered_reduce(st, _cuda(parts[0]))
    assert e.value.status == brl.BRL_EORDER


def test_replay_no_clip_and_empty():
    parts = [synth.replay_partial_host(5, v, 5000, std=1e-5) for v in range(4)]
    out, nu, _ = _replay_gpu(parts, 2, 2)
    T, wnu, _ = oracle.replay(parts, 2, 2)
    assert float(wnu) <= 1.0
    assert_bitwise(out, T, "TreeFold (no clip)")
    assert_bitwise(nu, np.array([wnu]), "nu")
    g = torch.zeros(0, dtype=torch.float32, device=DEV)
    nu0 = brl.grad_l2norm_clip(g)
    assert float(nu0.item()) == 0.0


@pytest.mark.parametrize("n", [1, 31, 32, 33, 8191, 8192 * 256 + 77, 3 * 2**20])
def test_norm_clip_parity(n):
    g = np.random.default_rng(n).standard_normal(n).astype(np.float32) * np.float32(0.01)
    g[: min(n, 10)] = np.float32(1e-40)       # subnormals read as zero
    t = _cuda(g)
    nu = brl.grad_l2norm_clip(t, 1.0)
    wnu = oracle.l2norm(g)
    w = g.copy()
    oracle.clip(w, wnu, 1.0, 0.0)
    assert_bitwise(nu, np.array([wnu]), "nu")
    assert_bitwise(t, w, "clipped g")


def test_norm_reduce_wg_invariance():
    n = 5_000_003
    g = np.random.default_rng(7).standard_normal(n).astype(np.float32)
    wnu = oracle.l2norm(g)
    for wg in (64, 128, 256):
        nu = brl.grad_l2norm_clip(_cuda(g), 1e30, tune=brl.Tuning(reduce_wg_blocks=wg))
        assert_bitwise(nu, np.array([wnu]), f"nu wg={wg}")


@pytest.mark.parametrize("n, wg", [
    (64 * 32 * 2401 + 35, 64),       # 2402 roots: one tail pass, runs of 4, last run of 2
    (64 * 32 * 10001 + 3, 64),       # 10002 roots: a 64-wide pass (157 roots), then the tail
    (2**26 + 5, 64),                 # 32769 roots: a 64-wide pass (513 roots), then the tail
    (2**27 + 12345, 64),             # 65543 roots: a 64-wide pass, then 1025 roots in runs of 2
])
def test_norm_tail_runs(n, wg):
    """The last CanonSum pass reduces aligned runs of roots per thread before
    the workgroup tree, after as many coalesced passes as the root count
    needs; run lengths, ragged last runs and the number of passes leave the
    bits alone."""
    g = np.random.default_rng(n).standard_normal(n, dtype=np.float32)
    wnu = oracle.l2norm(g)
    nu = brl.grad_l2norm_clip(_cuda(g), 1e30, tune=brl.Tuning(reduce_wg_blocks=wg))
    assert_bitwise(nu, np.array([wnu]), f"nu n={n} wg={wg}")


def test_replay_resident_unaligned_partials():
    """Partials 4 bytes off a 16-byte boundary take the per-element running
    sum and fold in the one-pass mode."""
    R, S, L = 6, 4, 1003
    parts = [synth.replay_partial_host(6, v, L, std=1e-2) for v in range(R * S)]
    T, wnu, A = oracle.replay(parts, R, S)
    st = brl.ReduceState(R, S, L, device=DEV, replica_resident=True)
    keep = []
    out = None
    for v in range(R * S):
        buf = torch.empty(L + 1, dtype=torch.float32, device=DEV)
        g = buf[1:]
        g.copy_(_cuda(parts[v]))
        assert g.data_ptr() % 16 == 4
        keep.append(buf)
        out = brl.ordered_reduce(st, g)
    nu = brl.grad_l2norm_clip(out, 1.0)
    torch.cuda.synchronize()
    assert_bitwise(out, T, "clipped TreeFold")
    assert_bitwise(nu, np.array([wnu]), "nu")
    for r in range(R - 1):
        assert_bitwise(st.acc[r], A[r], f"A_{r}")


def test_replay_stream_shape_invariance():
    """The number of 16-byte vectors per thread in the streaming kernels
    changes only the launch shape."""
    R, S, L = 6, 3, 100_003
    parts = [synth.replay_partial_host(9, v, L, std=1e-2) for v in range(R * S)]
    T, wnu, _ = oracle.replay(parts, R, S)
    for vec in (1, 2, 4):
        out, nu, _ = _replay_gpu(parts, R, S, tune=brl.Tuning(stream_vec=vec))
        assert_bitwise(out, T, f"TreeFold vec={vec}")
        assert_bitwise(nu, np.array([wnu]), f"nu vec={vec}")


def test_division_on_crafted_classes():
    """The device's binary32 division (the compiler's correctly rounded
    sequence) equals the oracle's binary64-then-rounded quotient on classes
    aimed at its corners: random bit patterns over the whole exponent range,
    quotients around 2^-126 (the flush threshold), subnormal operands and
    zeros of both signs, quotients near overflow, and exact quotients."""
    g = np.random.default_rng(11)
    n = 1 << 15
    sign = lambda: g.integers(0, 2, n, dtype=np.uint32) << 31
    man = lambda: g.integers(0, 1 << 23, n, dtype=np.uint32)
    classes = []
    ea = g.integers(1, 255, n, dtype=np.uint32); eb = g.integers(1, 255, n, dtype=np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (eb << 23) | man()))
    ea = g.integers(1, 100, n, dtype=np.uint32); eb = ea + 126 + g.integers(-2, 2, n).astype(np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (np.minimum(eb, 254) << 23) | man()))
    sub = g.integers(0, 3, n)
    a_bits = np.where(sub == 0, sign() | man(), sign() | (np.uint32(127) << 23) | man()).astype(np.uint32)
    b_bits = np.where(sub == 1, sign() | man(), np.where(sub == 2, sign(), sign() | (np.uint32(127) << 23) | man()))
    classes.append((a_bits, b_bits.astype(np.uint32)))
    ea = g.integers(200, 255, n, dtype=np.uint32); eb = g.integers(1, 60, n, dtype=np.uint32)
    classes.append((sign() | (ea << 23) | man(), sign() | (eb << 23) | man()))
    q = (g.integers(1, 1 << 12, n) * 2).astype(np.float32)
    d = g.integers(1, 1 << 11, n).astype(np.float32)
    classes.append(((q * d).astype(np.float32).view(np.uint32), d.view(np.uint32)))
    for ci, (ab, bb) in enumerate(classes):
        a, b = ab.view(np.float32), bb.view(np.float32)
        got = brl.probe_f32("div", _cuda(a), _cuda(b)).cpu().numpy()
        want = np.array([oracle.div(x, y) for x, y in zip(a, b)], np.float32)
        nan = np.isnan(got) & np.isnan(want)
        bad = np.flatnonzero((_bits(got) != _bits(want)) & ~nan)
        assert bad.size == 0, (ci, [(a[i], b[i], got[i], want[i]) for i in bad[:5]])
