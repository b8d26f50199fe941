"""CPU oracle for the bitwise-reproducible int8 LSQ linear layer and the ordered
gradient reduction (Open-1B "fully auditable training", onedev.kr summary,
sections "How", "Use" and "Limits").

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
The arithmetic lives in ``oracle.c`` (plain C, one binary32 operation at a
time, emulated in double and rounded once, explicit flush-to-zero); this
module only builds it and marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-shared", "-fPIC", "-Wall", "-Wextra"]


def build() -> str:
    """Compile oracle.c into liboracle.so next to it (always recompiles)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None

f32, i64, i32 = C.c_float, C.c_int64, C.c_int
P = C.c_void_p


def lib():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    L = C.CDLL(_LIB)
    sig = {
        "or_add": (f32, [f32, f32]), "or_sub": (f32, [f32, f32]),
        "or_mul": (f32, [f32, f32]), "or_div": (f32, [f32, f32]),
        "or_sqrt": (f32, [f32]), "or_i2f": (f32, [C.c_int32]), "or_rne": (f32, [f32]),
        "or_exp": (f32, [f32]), "or_exp_constants": (None, [P]),
        "or_pair_tree": (f32, [P, i64]), "or_canon_sum": (f32, [P, i64]),
        "or_weight_scale": (f32, [P, i64]),
        "or_adamw": (None, [P, P, P, P, i64, f32, f32, f32, f32, f32, f32, f32, f32, f32, i32]),
        "or_quantize": (None, [P, i64, f32, P, P]),
        "or_gemm_i8": (i64, [P, P, i64, i64, i64, P]),
        "or_swiglu_fwd": (None, [P, i64, i64, P]),
        "or_swiglu_bwd": (None, [P, P, i64, i64, P]),
        "or_fwd_rows": (i32, [P, P, i64, i64, i64, f32, f32, P, i32, P, i64, P, P]),
        "or_fwd_cols": (i32, [P, P, i64, i64, i64, f32, f32, P, i64, P]),
        "or_dx_rows": (None, [P, P, P, i64, i64, f32, f32, P, i64, P]),
        "or_dw_rows": (None, [P, P, P, i64, i64, f32, f32, P, i64, i64, P]),
        "or_replay_accumulate": (None, [P, P, i64, i32]),
        "or_treefold": (i32, [P, i32, i64, P]),
        "or_l2norm": (f32, [P, i64]),
        "or_clip": (f32, [P, i64, f32, f32, f32]),
        "or_attn_fwd": (i32, [P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P, i64]),
        "or_attn_fwd_rows": (i32, [P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P, i64, P, i64]),
        "or_attn_bwd_dq_rows": (i32, [P, P, P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P,
                                      i64, P, i64]),
        "or_attn_bwd_dkdv_rows": (i32, [P, P, P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32,
                                        P, i64, P, P, i64]),
        "or_num_threads": (i32, []),
        "or_set_threads": (None, [i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


# ---- binary32 primitives -------------------------------------------------
def add(a, b): return np.float32(lib().or_add(a, b))
def sub(a, b): return np.float32(lib().or_sub(a, b))
def mul(a, b): return np.float32(lib().or_mul(a, b))
def div(a, b): return np.float32(lib().or_div(a, b))
def sqrt(a): return np.float32(lib().or_sqrt(a))
def i2f(x): return np.float32(lib().or_i2f(int(x)))
def rne(t): return np.float32(lib().or_rne(t))
def exp(x): return np.float32(lib().or_exp(x))


def exp_constants() -> np.ndarray:
    out = np.zeros(11, np.float32)
    lib().or_exp_constants(_p(out))
    return out


# ---- CanonSum ------------------------------------------------------------
def canon_sum(p) -> np.float32:
    p = _f32(p).ravel()
    return np.float32(lib().or_canon_sum(_p(p), p.size))


def pair_tree(b) -> np.float32:
    b = _f32(b).ravel().copy()
    return np.float32(lib().or_pair_tree(_p(b), b.size))


# ---- LSQ -----------------------------------------------------------------
def weight_scale(W) -> np.float32:
    W = _f32(W)
    return np.float32(lib().or_weight_scale(_p(W), W.size))


def quantize(v, s):
    v = _f32(v)
    q = np.empty(v.shape, np.int8)
    inr = np.empty(v.shape, np.uint8)
    lib().or_quantize(_p(v), v.size, float(s), _p(q), _p(inr))
    return q, inr.astype(bool)


def gemm_i8(qx, qw):
    qx = np.ascontiguousarray(qx, np.int8)
    qw = np.ascontiguousarray(qw, np.int8)
    M, K = qx.shape
    N = qw.shape[0]
    acc = np.empty((M, N), np.int64)
    amax = lib().or_gemm_i8(_p(qx), _p(qw), M, K, N, _p(acc))
    return acc, int(amax)


# ---- QAT linear ------------------------------------------------------------
def fwd_rows(X, W, s_x, rows=None, addend=None, epilogue=0, s_w=None):
    """Y (and the pre-SwiGLU Y when epilogue == 1) for the given rows."""
    X, W = _f32(X), _f32(W)
    M, K = X.shape
    N = W.shape[0]
    if s_w is None:
        s_w = weight_scale(W)
    rows = np.arange(M, dtype=np.int64) if rows is None else np.ascontiguousarray(rows, np.int64)
    n_out = N // 2 if epilogue == 1 else N
    Y = np.empty((rows.size, n_out), np.float32)
    ypre = np.empty((rows.size, N), np.float32) if epilogue == 1 else np.empty(1, np.float32)
    add_p = None
    if addend is not None:
        addend = _f32(addend)
        add_p = _p(addend)
    rc = lib().or_fwd_rows(_p(X), _p(W), M, K, N, float(s_x), float(s_w), add_p, epilogue,
                           _p(rows), rows.size, _p(Y), _p(ypre))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow in the oracle GEMM")
    return (Y, ypre) if epilogue == 1 else Y


def fwd_cols(X, W, s_x, cols, s_w=None):
    """Y[:, cols] (pre-activation) as a [len(cols), M] array."""
    X, W = _f32(X), _f32(W)
    M, K = X.shape
    N = W.shape[0]
    if s_w is None:
        s_w = weight_scale(W)
    cols = np.ascontiguousarray(cols, np.int64)
    out = np.empty((cols.size, M), np.float32)
    rc = lib().or_fwd_cols(_p(X), _p(W), M, K, N, float(s_x), float(s_w), _p(cols), cols.size, _p(out))
    if rc != 0:
        raise OverflowError("int32 accumulator overflow in the oracle GEMM")
    return out


def swiglu_fwd(ypre):
    ypre = _f32(ypre)
    R, N = ypre.shape
    act = np.empty((R, N // 2), np.float32)
    lib().or_swiglu_fwd(_p(ypre), R, N, _p(act))
    return act


def swiglu_bwd(ypre, dact):
    ypre, dact = _f32(ypre), _f32(dact)
    R, N = ypre.shape
    d = np.empty((R, N), np.float32)
    lib().or_swiglu_bwd(_p(ypre), _p(dact), R, N, _p(d))
    return d


def dx_rows(dY_rows, X, W, s_x, rows, s_w=None):
    """dX rows; dY_rows[i] is the output gradient of row rows[i]."""
    X, W, dY_rows = _f32(X), _f32(W), _f32(dY_rows)
    K = X.shape[1]
    N = W.shape[0]
    if s_w is None:
        s_w = weight_scale(W)
    rows = np.ascontiguousarray(rows, np.int64)
    dX = np.empty((rows.size, K), np.float32)
    lib().or_dx_rows(_p(dY_rows), _p(X), _p(W), K, N, float(s_x), float(s_w), _p(rows),
                     rows.size, _p(dX))
    return dX


def dw_rows(dY_cols, X, W, s_x, wrows, mb=0, s_w=None):
    """dW rows; dY_cols[i] is the column dY[:, wrows[i]] (length M)."""
    X, W = _f32(X), _f32(W)
    dY_cols = _f32(dY_cols)
    M, K = X.shape
    if s_w is None:
        s_w = weight_scale(W)
    wrows = np.ascontiguousarray(wrows, np.int64)
    dW = np.empty((wrows.size, K), np.float32)
    lib().or_dw_rows(_p(dY_cols), _p(X), _p(W), M, K, float(s_x), float(s_w), _p(wrows),
                     wrows.size, int(mb), _p(dW))
    return dW


def linear_fwd(X, W, s_x, addend=None, epilogue=0):
    return fwd_rows(X, W, s_x, addend=addend, epilogue=epilogue)


def linear_bwd(dY, X, W, s_x, mb=0):
    """Full dX and dW for small problems (dY is the pre-activation gradient)."""
    dY = _f32(dY)
    M = X.shape[0]
    N = W.shape[0]
    dX = dx_rows(dY, X, W, s_x, np.arange(M))
    dW = dw_rows(np.ascontiguousarray(dY.T), X, W, s_x, np.arange(N), mb=mb)
    return dX, dW


# ---- replay ----------------------------------------------------------------
def replay_accumulate(A: np.ndarray, G, first: bool):
    G = _f32(G)
    assert A.dtype == np.float32 and A.flags["C_CONTIGUOUS"] and A.size == G.size
    lib().or_replay_accumulate(_p(A), _p(G), A.size, 1 if first else 0)


def treefold(As):
    As = [_f32(a) for a in As]
    R = len(As)
    ptrs = (C.c_void_p * R)(*[a.ctypes.data for a in As])
    T = np.empty_like(As[0])
    rc = lib().or_treefold(ptrs, R, T.size, _p(T))
    if rc != 0:
        raise AssertionError("recursive-doubling ranks disagree" if rc == -1 else "bad replica count")
    return T


def l2norm(T) -> np.float32:
    T = _f32(T)
    return np.float32(lib().or_l2norm(_p(T), T.size))


def clip(T: np.ndarray, nu, max_norm=1.0, eps=0.0) -> np.float32:
    assert T.dtype == np.float32 and T.flags["C_CONTIGUOUS"]
    return np.float32(lib().or_clip(_p(T), T.size, float(nu), float(max_norm), float(eps)))


def replay(partials, R, S, max_norm=1.0, eps=0.0):
    """Whole replay on host arrays: running sums in mesh order, TreeFold,
    global norm, clip.  Returns (T_clipped, nu, A_list)."""
    L = partials[0].size
    A = [np.empty(L, np.float32) for _ in range(R)]
    for v in range(R * S):
        r, s = divmod(v, S)
        replay_accumulate(A[r], partials[v], first=(s == 0))
    T = treefold(A)
    nu = l2norm(T)
    clip(T, nu, max_norm, eps)
    return T, nu, A


# ---- AdamW ----------------------------------------------------------------------
# Recipe (onedev.kr summary, "Limits", recipe paragraph): AdamW(0.9, 0.95, 1e-8),
# decoupled weight decay 0.1 except input embedding, norm weights and RoPE table;
# linear warm-up to 4.5e-4 over about 2.1B tokens, then one cosine decay to 10% of
# the peak at 400B tokens, keyed to consumed tokens.  The reading taken (see or_adamw in
# oracle.c): the step's scalars in binary64, each rounded once to binary32.
ADAMW = dict(beta1=0.9, beta2=0.95, eps=1e-8, wd=0.1, peak_lr=4.5e-4, min_lr=4.5e-5,
             warmup_tokens=2.1e9, total_tokens=400e9)


def lr_at(tokens: float, cfg=ADAMW) -> float:
    """Learning rate (binary64) after `tokens` consumed tokens."""
    import math
    W, T = cfg["warmup_tokens"], cfg["total_tokens"]
    if tokens < W:
        return cfg["peak_lr"] * tokens / W
    frac = min(1.0, (tokens - W) / (T - W))
    return cfg["min_lr"] + (cfg["peak_lr"] - cfg["min_lr"]) * 0.5 * (1.0 + math.cos(math.pi * frac))


def adamw_scalars(step: int, tokens: float, cfg=ADAMW) -> dict:
    """The binary32 scalars of one step (each a binary64 value rounded once)."""
    b1, b2 = cfg["beta1"], cfg["beta2"]
    lr = lr_at(tokens, cfg)
    f = lambda x: float(np.float32(x))
    return dict(beta1=f(b1), beta2=f(b2), c1=f(1.0 - b1), c2=f(1.0 - b2), bc1=f(1.0 - b1 ** step),
                bc2=f(1.0 - b2 ** step), eps=f(cfg["eps"]), lr=f(lr), d=f(lr * cfg["wd"]))


def adamw(p, g, m, v, sc: dict, decay: bool = True):
    """One AdamW update of (p, m, v) in place (float32 arrays) with scalars sc."""
    for a in (p, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous
    g = _f32(g)
    lib().or_adamw(_p(p), _p(g), _p(m), _p(v), p.size, sc["beta1"], sc["beta2"], sc["c1"], sc["c2"],
                   sc["bc1"], sc["bc2"], sc["eps"], sc["lr"], sc["d"], 1 if decay else 0)


def attn_fwd(Q, K, V, window: int, s_v: float) -> np.ndarray:
    """Attention with int8 P.V on [B, S, H, D] arrays (Q: Hq heads, K and V:
    Hkv heads); returns O [B, S, Hq, D].  See or_attn_fwd for the readings."""
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    assert K.shape == (B, S, Hkv, D) and V.shape == K.shape
    O = np.empty_like(Q)
    rc = lib().or_attn_fwd(_p(Q), _p(K), _p(V), B, S, Hq, Hkv, D, Hq * D, Hkv * D, Hkv * D, int(window),
                           np.float32(s_v), _p(O), Hq * D)
    assert rc == 0, f"or_attn_fwd failed ({rc})"
    return O


def attn_fwd_rows(Q, K, V, window: int, s_v: float, rows) -> np.ndarray:
    """Rows of attn_fwd's output picked by flat id (b*S + i)*Hq + h:
    returns [len(rows), D]."""
    Q, K, V = _f32(Q), _f32(K), _f32(V)
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    rows = np.ascontiguousarray(rows, np.int64)
    out = np.empty((rows.size, D), np.float32)
    rc = lib().or_attn_fwd_rows(_p(Q), _p(K), _p(V), B, S, Hq, Hkv, D, Hq * D, Hkv * D, Hkv * D, int(window),
                                np.float32(s_v), _p(rows), rows.size, _p(out), D)
    assert rc == 0, f"or_attn_fwd_rows failed ({rc})"
    return out


def attn_bwd_dq(Q, K, V, O, dO, window: int, s_v: float, rows=None) -> np.ndarray:
    """Fixed-point-accumulated dQ of the attention (see or_attn_bwd_dq_rows):
    rows by flat id (b*S + i)*Hq + h, all rows by default; returns
    [len(rows), D] (or [B, S, Hq, D] for all rows)."""
    Q, K, V, O, dO = _f32(Q), _f32(K), _f32(V), _f32(O), _f32(dO)
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    assert O.shape == Q.shape and dO.shape == Q.shape
    if rows is None:
        out = np.empty((B * S * Hq, D), np.float32)
        rp, n = None, B * S * Hq
    else:
        rows = np.ascontiguousarray(rows, np.int64)
        out = np.empty((rows.size, D), np.float32)
        rp, n = _p(rows), rows.size
    rc = lib().or_attn_bwd_dq_rows(_p(Q), _p(K), _p(V), _p(O), _p(dO), B, S, Hq, Hkv, D, Hq * D, Hkv * D,
                                   Hkv * D, Hq * D, int(window), np.float32(s_v), rp, n, _p(out), D)
    assert rc == 0, f"or_attn_bwd_dq_rows failed ({rc})"
    return out.reshape(B, S, Hq, D) if rows is None else out


def attn_bwd_dkdv(Q, K, V, O, dO, window: int, s_v: float, rows=None):
    """Fixed-point-accumulated dK and dV of the attention (see
    or_attn_bwd_dkdv_rows): key rows by flat id (b*S + j)*Hkv + hk, all rows
    by default; returns (dK, dV), each [len(rows), D] (or [B, S, Hkv, D])."""
    Q, K, V, O, dO = _f32(Q), _f32(K), _f32(V), _f32(O), _f32(dO)
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    assert K.shape == (B, S, Hkv, D) and V.shape == K.shape
    assert O.shape == Q.shape and dO.shape == Q.shape
    if rows is None:
        n, rp = B * S * Hkv, None
    else:
        rows = np.ascontiguousarray(rows, np.int64)
        n, rp = rows.size, _p(rows)
    dk = np.empty((n, D), np.float32)
    dv = np.empty((n, D), np.float32)
    rc = lib().or_attn_bwd_dkdv_rows(_p(Q), _p(K), _p(V), _p(O), _p(dO), B, S, Hq, Hkv, D, Hq * D, Hkv * D,
                                     Hkv * D, Hq * D, int(window), np.float32(s_v), rp, n, _p(dk), _p(dv), D)
    assert rc == 0, f"or_attn_bwd_dkdv_rows failed ({rc})"
    if rows is None:
        return dk.reshape(B, S, Hkv, D), dv.reshape(B, S, Hkv, D)
    return dk, dv


def num_threads() -> int:
    return int(lib().or_num_threads())


def set_threads(n: int) -> None:
    lib().or_set_threads(int(n))
