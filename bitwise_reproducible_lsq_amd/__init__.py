"""Python binding of libbrlsq, the bit-exact int8 LSQ linear layer and ordered
gradient reduction for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI in include/brlsq.h.  PyTorch provides device memory
(outputs and workspaces are torch tensors) and streams (the current torch
stream is passed to every call).  There is no fallback: if the library is not
built or cannot load, every call raises.

Names follow the C ABI: qat_linear_fwd, qat_linear_bwd, ordered_reduce,
grad_l2norm_clip, state_hash (brl_state_hash).
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbrlsq.so")

BRL_OK, BRL_EINVAL, BRL_ESHAPE, BRL_EORDER, BRL_EDEVICE, BRL_EWORKSPACE = 0, -1, -2, -3, -4, -5
EPILOGUE_NONE, EPILOGUE_SWIGLU = 0, 1
OP_FWD, OP_BWD, OP_NORM, OP_HASH = 0, 1, 2, 3
MAX_REPLICAS = 64
MAX_SHARDS = 64

PROBE_OPS = {"add": 0, "sub": 1, "mul": 2, "div": 3, "sqrt": 4, "i2f": 5, "rne": 6, "exp": 7, "mfma_mul": 8,
             "mfma_fma": 9}


class BrlError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"brlsq status {status}: {msg}")
        self.status = status


class Tuning(C.Structure):
    """Launch shapes of one call (brl_tuning): they never change results.
    Zero fields select the defaults."""
    _fields_ = [("bwd_chunk_log2", C.c_int32), ("reduce_wg_blocks", C.c_int32), ("stream_vec", C.c_int32),
                ("bwd_engine", C.c_int32), ("fwd_prep", C.c_int32)]


class ReduceStateC(C.Structure):
    _fields_ = [("replicas", C.c_int32), ("shards", C.c_int32), ("len", C.c_int64),
                ("next", C.c_int32), ("flags", C.c_uint32), ("pending", C.c_void_p),
                ("acc", C.c_void_p * MAX_REPLICAS), ("tune", Tuning), ("shard_part", C.c_void_p * MAX_SHARDS)]


REDUCE_PARTIALS_PERSIST = 1
REDUCE_REPLICA_RESIDENT = 2


_lib = None
P, i64, i32, f32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_float, C.c_size_t

_SIGS = {
    "brl_workspace_bytes": (sz, [i32, i64, i64, i64, P]),
    "qat_linear_fwd": (i32, [P, P, i64, i64, i64, f32, P, i32, P, P, P, P, sz, P, P]),
    "qat_linear_bwd": (i32, [P, P, P, P, i64, i64, i64, f32, i32, P, P, i32, P, sz, P, P]),
    "brl_reduce_init": (i32, [C.POINTER(ReduceStateC), i32, i32, i64, P]),
    "ordered_reduce": (i32, [C.POINTER(ReduceStateC), P, P, P]),
    "grad_l2norm_clip": (i32, [P, i64, f32, f32, P, P, sz, P, P]),
    "grad_l2norm_clip_noalloc": (i32, [P, i64, f32, f32, P, P, P]),
    "brl_probe_f32": (i32, [i32, P, P, P, i64, P]),
    "brl_state_hash": (i32, [P, P, i32, P, P, sz, P]),
    "brl_adamw_scalars_for_step": (i32, [i64, C.c_double, P, P]),
    "adamw_step": (i32, [P, P, P, P, i64, P, i32, P]),
    "attn_fwd": (i32, [P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P, i64, P, P, sz, P]),
    "attn_fwd_workspace_bytes": (sz, [i64, i64, i64, i64, i64]),
    "attn_fwd_keep_logits": (i32, [P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P, i64, P, P, sz, P,
                                   sz, P]),
    "attn_logits_bytes": (sz, [i64, i64, i64, i64]),
    "attn_bwd_dq_logits": (i32, [P, P, P, P, P, P, P, sz, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P,
                                 P]),
    "attn_bwd_dkdv_logits": (i32, [P, P, P, P, P, P, P, sz, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P,
                                   P, i64, P]),
    "attn_bwd_dq": (i32, [P, P, P, P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P, P]),
    "attn_bwd_dkdv": (i32, [P, P, P, P, P, P, i64, i64, i64, i64, i64, i64, i64, i64, i64, i64, f32, P, P, i64,
                            P]),
    "brl_stream_create": (i32, [C.c_uint64, i32, P, i32, C.POINTER(C.c_void_p)]),
    "brl_stream_destroy": (None, [P]),
    "brl_stream_next": (i32, [P, i64, P, C.POINTER(C.c_int64)]),
    "brl_stream_step": (i32, [P, i64, i32, i32, P]),
    "brl_stream_record_bytes": (i64, [P]),
    "brl_stream_save": (i32, [P, P, i64]),
    "brl_stream_load": (i32, [P, P, i64]),
    "brl_philox_u32": (i32, [C.c_uint64, C.c_uint32, C.c_uint64, i64, P, P]),
    "brl_probe_rate": (i32, [i32, i64, P, i64, P]),
    "brl_probe_rate_threads": (i64, []),
    "brl_status_string": (C.c_char_p, [i32]),
    "brl_last_error": (C.c_char_p, []),
}


def lib() -> C.CDLL:
    """Load libbrlsq.so (built in-tree by build.py); raise if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                               "or python bitwise_reproducible_lsq_amd/build.py")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int):
    if status != BRL_OK:
        L = lib()
        raise BrlError(status, f"{L.brl_status_string(status).decode()}: {L.brl_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("brlsq tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("brlsq tensors must be contiguous")
    return C.c_void_p(t.data_ptr())


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32")
    return t


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _tune(tune: Optional[Tuning]):
    return C.byref(tune) if tune is not None else None


def workspace(op: int, M: int, K: int, N: int, device, tune: Optional[Tuning] = None, stream=None) -> torch.Tensor:
    """A fresh workspace for one call from torch's caching allocator.  Memory
    is reused only in the order of the stream it is used on: a workspace for
    a stream other than the current one is recorded on that stream."""
    n = int(lib().brl_workspace_bytes(op, M, K, N, _tune(tune)))
    if n == 0:
        raise BrlError(BRL_ESHAPE, f"no workspace size for op={op} M={M} K={K} N={N}")
    w = torch.empty(n, dtype=torch.uint8, device=torch.device(device))
    if stream is not None and stream != torch.cuda.current_stream(w.device):
        w.record_stream(stream)
    return w


def workspace_bytes(op: int, M: int, K: int, N: int, tune: Optional[Tuning] = None) -> int:
    return int(lib().brl_workspace_bytes(op, M, K, N, _tune(tune)))


def qat_linear_fwd(X: torch.Tensor, W: torch.Tensor, s_x: float, addend: Optional[torch.Tensor] = None,
                   epilogue: int = EPILOGUE_NONE, want_ypre: bool = True, Y: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None, tune: Optional[Tuning] = None,
                   Ypre: Optional[torch.Tensor] = None):
    """Y = dequant(int8 GEMM) (+ addend), or the SwiGLU activation.  With
    SwiGLU the pre-activation goes to Ypre (given, or allocated when
    want_ypre).  Returns (Y, Ypre or None, s_w as a 1-element device tensor)."""
    _f32(X, "X"), _f32(W, "W")
    M, K = X.shape
    N, K2 = W.shape
    if K2 != K:
        raise ValueError("X and W disagree on K")
    n_out = N // 2 if epilogue == EPILOGUE_SWIGLU else N
    if Y is None:
        Y = torch.empty((M, n_out), dtype=torch.float32, device=X.device)
    if epilogue != EPILOGUE_SWIGLU:
        Ypre = None
    elif Ypre is None and want_ypre:
        Ypre = torch.empty((M, N), dtype=torch.float32, device=X.device)
    for t, shape, name in ((Y, (M, n_out), "Y"), (Ypre, (M, N), "Ypre")):
        if t is not None and (tuple(t.shape) != shape or t.dtype != torch.float32):
            raise ValueError(f"{name} must be float32 {shape}")
    s_w = torch.empty(1, dtype=torch.float32, device=X.device)
    if ws is None:
        ws = workspace(OP_FWD, M, K, N, X.device, tune, stream)
    st = lib().qat_linear_fwd(_ptr(X), _ptr(W), M, K, N, float(s_x), _ptr(addend), epilogue, _ptr(Y),
                              _ptr(Ypre), _ptr(s_w), _ptr(ws), ws.numel(), _tune(tune), _stream(stream))
    _check(st)
    return Y, Ypre, s_w


def qat_linear_bwd(dOut: torch.Tensor, X: torch.Tensor, W: torch.Tensor, s_x: float,
                   Ypre: Optional[torch.Tensor] = None, epilogue: int = EPILOGUE_NONE,
                   need_dX: bool = True, need_dW: bool = True, dW: Optional[torch.Tensor] = None,
                   dW_accumulate: bool = False, dX: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None, tune: Optional[Tuning] = None):
    """Straight-through backward; returns (dX or None, dW or None)."""
    M, K = X.shape
    N = W.shape[0]
    if need_dX and dX is None:
        dX = torch.empty((M, K), dtype=torch.float32, device=X.device)
    if not need_dX:
        dX = None
    if need_dW and dW is None:
        if dW_accumulate:
            raise ValueError("dW_accumulate needs the running dW")
        dW = torch.empty((N, K), dtype=torch.float32, device=X.device)
    if not need_dW:
        dW = None
    if ws is None:
        ws = workspace(OP_BWD, M, K, N, X.device, tune, stream)
    st = lib().qat_linear_bwd(_ptr(dOut), _ptr(X), _ptr(W), _ptr(Ypre), M, K, N, float(s_x), epilogue,
                              _ptr(dX), _ptr(dW), 1 if dW_accumulate else 0, _ptr(ws), ws.numel(),
                              _tune(tune), _stream(stream))
    _check(st)
    return dX, dW


class ReduceState:
    """Host-side replay state: R replica accumulators A_r of `length` floats
    (device tensors owned here) and the next virtual rank in mesh order."""

    def __init__(self, replicas: int, shards: int, length: int, device="cuda",
                 acc: Optional[Sequence[torch.Tensor]] = None, partials_persist: bool = False,
                 tune: Optional[Tuning] = None, replica_resident: bool = False):
        if acc is None:
            acc = [torch.empty(length, dtype=torch.float32, device=device) for _ in range(replicas)]
        self.acc = list(acc)
        self.c = ReduceStateC()
        ptrs = (C.c_void_p * replicas)(*[a.data_ptr() for a in self.acc])
        _check(lib().brl_reduce_init(C.byref(self.c), replicas, shards, length,
                                     C.cast(ptrs, C.c_void_p)))
        # persist: the caller keeps each replica's shard-0 partial valid and
        # unchanged until its shard-1 call has run; replica_resident: every
        # partial of a replica until the replica's last-shard call has run
        # (see the C header)
        self.c.flags = (REDUCE_PARTIALS_PERSIST if partials_persist else 0) | \
            (REDUCE_REPLICA_RESIDENT if replica_resident else 0)
        if tune is not None:
            self.c.tune = tune

    @property
    def next(self) -> int:
        return int(self.c.next)

    @property
    def total(self) -> int:
        return int(self.c.replicas) * int(self.c.shards)

    def reset(self):
        self.c.next = 0
        self.c.pending = None


def ordered_reduce(state: ReduceState, partial: torch.Tensor, out: Optional[torch.Tensor] = None,
                   stream=None) -> Optional[torch.Tensor]:
    """Feed G_v for v = state.next; after the last rank returns the TreeFold."""
    last = state.next == state.total - 1
    if last and out is None:
        out = torch.empty(int(state.c.len), dtype=torch.float32, device=partial.device)
    _check(lib().ordered_reduce(C.byref(state.c), _ptr(partial), _ptr(out), _stream(stream)))
    return out if last else None


def grad_l2norm_clip(g: torch.Tensor, max_norm: float = 1.0, eps: float = 0.0,
                     ws: Optional[torch.Tensor] = None, stream=None, tune: Optional[Tuning] = None) -> torch.Tensor:
    """In-place clip of g; returns the pre-clip norm as a 1-element device tensor."""
    n = g.numel()
    nu = torch.empty(1, dtype=torch.float32, device=g.device)
    if ws is None:
        ws = workspace(OP_NORM, n, 0, 0, g.device, tune, stream)
    _check(lib().grad_l2norm_clip(_ptr(g), n, float(max_norm), float(eps), _ptr(nu), _ptr(ws), ws.numel(),
                                  _tune(tune), _stream(stream)))
    return nu


NOALLOC_NORM_MAX_LEN = 1056565248


def grad_l2norm_clip_noalloc(g: torch.Tensor, max_norm: float = 1.0, eps: float = 0.0, nu: Optional[torch.Tensor] = None,
                             stream=None, tune: Optional[Tuning] = None) -> torch.Tensor:
    """grad_l2norm_clip without a workspace (the library's per-device scratch
    array; at most NOALLOC_NORM_MAX_LEN elements; calls overlapping on one
    device race).  Returns the pre-clip norm in nu (allocated here if None)."""
    n = g.numel()
    if nu is None:
        nu = torch.empty(1, dtype=torch.float32, device=g.device)
    _check(lib().grad_l2norm_clip_noalloc(_ptr(g), n, float(max_norm), float(eps), _ptr(nu), _tune(tune),
                                          _stream(stream)))
    return nu


def state_hash(tensors: Sequence[torch.Tensor], ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """SHA-256 tree hash of the tensors' raw bytes, in order (brl_state_hash);
    returns the 32-byte digest as a uint8 device tensor."""
    if len(tensors) == 0:
        raise ValueError("the state has at least one tensor")
    dev = tensors[0].device
    n = len(tensors)
    ptrs = (C.c_void_p * n)(*[(_ptr(t).value if t.numel() > 0 else None) for t in tensors])
    nbytes = (C.c_int64 * n)(*[t.numel() * t.element_size() for t in tensors])
    total = sum(nbytes)
    if ws is None:
        ws = workspace(OP_HASH, total, n, 0, dev, None, stream)
    out = torch.empty(32, dtype=torch.uint8, device=dev)
    _check(lib().brl_state_hash(C.cast(ptrs, C.c_void_p), C.cast(nbytes, C.c_void_p), n, _ptr(out), _ptr(ws),
                                ws.numel(), _stream(stream)))
    return out


class AdamWConfig(C.Structure):
    _fields_ = [(n, C.c_double) for n in ("beta1", "beta2", "eps", "wd", "peak_lr", "min_lr",
                                          "warmup_tokens", "total_tokens")]


class AdamWScalars(C.Structure):
    _fields_ = [(n, C.c_float) for n in ("beta1", "beta2", "c1", "c2", "bc1", "bc2", "eps", "lr", "d")]

    def as_dict(self) -> dict:
        return {n: float(getattr(self, n)) for n, _ in self._fields_}


def adamw_scalars_for_step(step: int, tokens: float, cfg: Optional[AdamWConfig] = None) -> AdamWScalars:
    """The step's binary32 scalars (brl_adamw_scalars_for_step); cfg None = the recipe."""
    out = AdamWScalars()
    _check(lib().brl_adamw_scalars_for_step(step, float(tokens), C.byref(cfg) if cfg is not None else None,
                                            C.byref(out)))
    return out


def adamw_step(p: torch.Tensor, g: torch.Tensor, m: torch.Tensor, v: torch.Tensor, sc: AdamWScalars,
               decay: bool = True, stream=None) -> None:
    """In-place AdamW update of p, m, v from g (adamw_step)."""
    for t, name in ((p, "p"), (g, "g"), (m, "m"), (v, "v")):
        _f32(t, name)
        if t.numel() != p.numel():
            raise ValueError("p, g, m, v must have the same size")
    _check(lib().adamw_step(_ptr(p), _ptr(g), _ptr(m), _ptr(v), p.numel(), C.byref(sc), 1 if decay else 0,
                            _stream(stream)))


def _heads_view(t: torch.Tensor, name: str):
    """[B, S, H, D] float32 view on the GPU whose (H, D) part is dense and
    whose rows are evenly spaced; returns (pointer, row stride)."""
    _f32(t, name)
    if not t.is_cuda or t.dim() != 4:
        raise ValueError(f"{name} must be a [B, S, H, D] GPU tensor")
    B, S, H, D = t.shape
    if t.stride(3) != 1 or (H > 1 and t.stride(2) != D) or (B > 1 and t.stride(0) != S * t.stride(1)):
        raise ValueError(f"{name}: heads and head dimension must be dense, rows evenly spaced")
    return C.c_void_p(t.data_ptr()), t.stride(1) if S > 1 else H * D


def attn_logits_bytes(B: int, S: int, Hq: int, window: int) -> int:
    """Bytes of the logits attn_fwd keeps when given a logits buffer."""
    return int(lib().attn_logits_bytes(B, S, Hq, int(window)))


def attn_logits_buffer(B: int, S: int, Hq: int, window: int, device="cuda") -> torch.Tensor:
    """A float32 buffer for the logits attn_fwd keeps (attn_fwd_keep_logits)
    and attn_bwd_dq / attn_bwd_dkdv read."""
    n = attn_logits_bytes(B, S, Hq, window)
    if n == 0 and B * S > 0:
        raise BrlError(BRL_ESHAPE, f"attn_logits_bytes: no size for B={B} S={S} Hq={Hq}")
    return torch.empty(max(n // 4, 1), dtype=torch.float32, device=device)


def _logits_arg(logits: torch.Tensor, B: int, S: int, Hq: int, window: int):
    if logits.dtype != torch.float32 or not logits.is_contiguous() or not logits.is_cuda:
        raise ValueError("logits must be a dense float32 device tensor (attn_logits_buffer)")
    return _ptr(logits), logits.numel() * 4


def attn_fwd(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, window: int, s_v: float,
             O: Optional[torch.Tensor] = None, stats: Optional[torch.Tensor] = None, stream=None,
             logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Attention with int8 P.V (attn_fwd).  Q [B, S, Hq, D], K and V
    [B, S, Hkv, D], views with evenly spaced rows (column slices of the QKV
    projection output work); returns O [B, S, Hq, D].  stats, if given, is a
    float32 [B, S, Hq, 2] tensor receiving (m_i, l_i) for attn_bwd_dq.
    logits, if given (attn_logits_buffer), receives the exact logits for the
    backward (attn_fwd_keep_logits)."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    if K.shape != (B, S, Hkv, D) or V.shape != K.shape:
        raise ValueError("Q, K, V shapes disagree")
    if O is None:
        O = torch.empty((B, S, Hq, D), dtype=torch.float32, device=Q.device)
    if stats is not None and (stats.shape != (B, S, Hq, 2) or stats.dtype != torch.float32):
        raise ValueError("stats must be float32 [B, S, Hq, 2]")
    q, ldq = _heads_view(Q, "Q")
    k, ldk = _heads_view(K, "K")
    v, ldv = _heads_view(V, "V")
    o, ldo = _heads_view(O, "O")
    nws = int(lib().attn_fwd_workspace_bytes(B, S, Hq, Hkv, int(window)))
    if nws == 0:
        raise BrlError(BRL_ESHAPE, f"attn_fwd: no workspace size for B={B} S={S} Hq={Hq} Hkv={Hkv}")
    ws = torch.empty(nws, dtype=torch.uint8, device=Q.device)
    if stream is not None and stream != torch.cuda.current_stream(Q.device):
        ws.record_stream(stream)
    if logits is None:
        _check(lib().attn_fwd(q, k, v, B, S, Hq, Hkv, D, ldq, ldk, ldv, int(window), float(s_v), o, ldo,
                              _ptr(stats), _ptr(ws), ws.numel(), _stream(stream)))
    else:
        lp, lb = _logits_arg(logits, B, S, Hq, window)
        _check(lib().attn_fwd_keep_logits(q, k, v, B, S, Hq, Hkv, D, ldq, ldk, ldv, int(window), float(s_v), o, ldo,
                                          _ptr(stats), lp, lb, _ptr(ws), ws.numel(), _stream(stream)))
    return O


def attn_bwd_dq(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor, dO: torch.Tensor,
                stats: torch.Tensor, window: int, s_v: float, dQ: Optional[torch.Tensor] = None,
                stream=None, logits: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dQ of attn_fwd with 64-bit fixed-point accumulation (attn_bwd_dq).
    O, dO and dQ are dense [B, S, Hq, D]; stats as written by attn_fwd.
    logits, if given, the ones attn_fwd kept for the same inputs
    (attn_bwd_dq_logits: the same bits, one product fewer)."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    for t, n in ((O, "O"), (dO, "dO")):
        _f32(t, n)
        if t.shape != Q.shape:
            raise ValueError(f"{n} must have Q's shape")
    if stats.shape != (B, S, Hq, 2) or stats.dtype != torch.float32:
        raise ValueError("stats must be float32 [B, S, Hq, 2]")
    if dQ is None:
        dQ = torch.empty((B, S, Hq, D), dtype=torch.float32, device=Q.device)
    q, ldq = _heads_view(Q, "Q")
    k, ldk = _heads_view(K, "K")
    v, ldv = _heads_view(V, "V")
    ld = Hq * D
    if logits is None:
        _check(lib().attn_bwd_dq(q, k, v, _ptr(O), _ptr(dO), _ptr(stats), B, S, Hq, Hkv, D, ldq, ldk, ldv, ld,
                                 int(window), float(s_v), _ptr(dQ), _stream(stream)))
    else:
        lp, lb = _logits_arg(logits, B, S, Hq, window)
        _check(lib().attn_bwd_dq_logits(q, k, v, _ptr(O), _ptr(dO), _ptr(stats), lp, lb, B, S, Hq, Hkv, D, ldq, ldk,
                                        ldv, ld, int(window), float(s_v), _ptr(dQ), _stream(stream)))
    return dQ


def attn_bwd_dkdv(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, O: torch.Tensor, dO: torch.Tensor,
                  stats: torch.Tensor, window: int, s_v: float, dK: Optional[torch.Tensor] = None,
                  dV: Optional[torch.Tensor] = None, stream=None, logits: Optional[torch.Tensor] = None):
    """dK and dV of attn_fwd with 64-bit fixed-point accumulation
    (attn_bwd_dkdv).  O and dO dense [B, S, Hq, D]; stats as written by
    attn_fwd; dK and dV [B, S, Hkv, D] views sharing one row stride (column
    slices of a QKV gradient buffer work).  logits, if given, the ones
    attn_fwd kept (attn_bwd_dkdv_logits).  Returns (dK, dV)."""
    B, S, Hq, D = Q.shape
    Hkv = K.shape[2]
    for t, n in ((O, "O"), (dO, "dO")):
        _f32(t, n)
        if t.shape != Q.shape or not t.is_contiguous():
            raise ValueError(f"{n} must be a dense tensor of Q's shape")
    if stats.shape != (B, S, Hq, 2) or stats.dtype != torch.float32 or not stats.is_contiguous():
        raise ValueError("stats must be a dense float32 [B, S, Hq, 2] tensor")
    if dK is None and dV is None:
        g = torch.empty((B, S, 2, Hkv, D), dtype=torch.float32, device=Q.device)
        dK, dV = g[:, :, 0], g[:, :, 1]
    elif dK is None or dV is None:
        raise ValueError("give both dK and dV or neither")
    for t, n in ((dK, "dK"), (dV, "dV")):
        if t.shape != K.shape:
            raise ValueError(f"{n} must have K's shape")
    pk, ldg = _heads_view(dK, "dK")
    pv, ldg2 = _heads_view(dV, "dV")
    if ldg != ldg2:
        raise ValueError("dK and dV must share one row stride")
    q, ldq = _heads_view(Q, "Q")
    k, ldk = _heads_view(K, "K")
    v, ldv = _heads_view(V, "V")
    if logits is None:
        _check(lib().attn_bwd_dkdv(q, k, v, _ptr(O), _ptr(dO), _ptr(stats), B, S, Hq, Hkv, D, ldq, ldk, ldv, Hq * D,
                                   int(window), float(s_v), pk, pv, ldg, _stream(stream)))
    else:
        lp, lb = _logits_arg(logits, B, S, Hq, window)
        _check(lib().attn_bwd_dkdv_logits(q, k, v, _ptr(O), _ptr(dO), _ptr(stats), lp, lb, B, S, Hq, Hkv, D, ldq,
                                          ldk, ldv, Hq * D, int(window), float(s_v), pk, pv, ldg, _stream(stream)))
    return dK, dV


STREAM_WINDOW = 4097


class _StreamSource(C.Structure):
    _fields_ = [("name", C.c_char_p), ("weight", C.c_int64), ("n_shards", C.c_int32),
                ("shard_docs", C.c_void_p), ("doc_offsets", C.c_void_p), ("tokens", C.c_void_p)]


class DataStream:
    """The topology-invariant data stream (brl_stream_*), host side.  corpus:
    list of (name, weight, shards), each shard a list of int32 token arrays;
    the flattened copy made here lives as long as the stream."""

    def __init__(self, seed: int, separator: int, corpus):
        import numpy as np
        self._keep = []
        srcs = (_StreamSource * len(corpus))()
        for k, (name, weight, shards) in enumerate(corpus):
            docs = [np.ascontiguousarray(d, np.int32) for sh in shards for d in sh]
            tokens = np.concatenate(docs) if docs else np.zeros(1, np.int32)
            offs = np.zeros(len(docs) + 1, np.int64)
            offs[1:] = np.cumsum([d.size for d in docs])
            counts = np.array([len(sh) for sh in shards], np.int64)
            bname = name.encode("utf-8")
            self._keep += [tokens, offs, counts, bname]
            srcs[k] = _StreamSource(bname, int(weight), len(shards), counts.ctypes.data, offs.ctypes.data,
                                    tokens.ctypes.data)
        self._keep.append(srcs)
        h = C.c_void_p()
        _check(lib().brl_stream_create(int(seed) & (2 ** 64 - 1), int(separator), srcs, len(corpus), C.byref(h)))
        self._h = h

    def next(self, count: int):
        """(index of the first window, int32 [count, 4097])."""
        import numpy as np
        out = np.empty((count, STREAM_WINDOW), np.int32)
        first = C.c_int64()
        _check(lib().brl_stream_next(self._h, count, out.ctypes.data, C.byref(first)))
        return first.value, out

    def step(self, global_batch: int, ranks: int, rank: int):
        import numpy as np
        out = np.empty((global_batch // max(ranks, 1), STREAM_WINDOW), np.int32)
        _check(lib().brl_stream_step(self._h, global_batch, ranks, rank, out.ctypes.data))
        return out

    def save(self) -> bytes:
        n = lib().brl_stream_record_bytes(self._h)
        buf = (C.c_uint8 * n)()
        _check(lib().brl_stream_save(self._h, buf, n))
        return bytes(buf)

    def load(self, record: bytes) -> None:
        buf = (C.c_uint8 * len(record)).from_buffer_copy(record)
        _check(lib().brl_stream_load(self._h, buf, len(record)))

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().brl_stream_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def philox_u32(key: int, stream: int, first: int, n: int, out: Optional[torch.Tensor] = None,
               hip_stream=None) -> torch.Tensor:
    """Device draws out[k] = draw(key, stream, first + k) as int32 bit patterns."""
    if out is None:
        out = torch.empty(n, dtype=torch.int32, device="cuda")
    _check(lib().brl_philox_u32(int(key) & (2 ** 64 - 1), int(stream) & 0xFFFFFFFF, int(first), n, _ptr(out),
                                _stream(hip_stream)))
    return out


def probe_f32(op: str, a: torch.Tensor, b: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    out = torch.empty_like(a)
    _check(lib().brl_probe_f32(PROBE_OPS[op], _ptr(a), _ptr(b), _ptr(out), a.numel(), _stream(stream)))
    return out


RATE_UNITS = {"v_add_f32": 0, "v_mul_f32": 1, "mfma_k1_f32": 2, "mfma_i8": 3, "valu_u32": 4,
              "v_add_f32_sgpr": 5, "k1_engine": 6, "mfma_i8_data": 7, "k1_engine_data": 8}
# operations each thread performs per step of the rate probe (per lane: the
# MFMA counts are per wave, divided over its 64 lanes; k1_engine counts
# multiply-adds, a matrix-core product and a VALU add each)
RATE_OPS_PER_STEP = {"v_add_f32": 8, "v_mul_f32": 8, "mfma_k1_f32": 8 * 1024 / 64, "mfma_i8": 8 * 65536 / 64,
                     "valu_u32": 16, "v_add_f32_sgpr": 8, "k1_engine": 4 * 1024 / 64,
                     "mfma_i8_data": 32 * 65536 / 64, "k1_engine_data": 16 * 1024 / 64}


def probe_rate(unit: str, iters: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Launch the sustained-rate probe of one unit (brl_probe_rate); time it
    with events around the call.  Returns the output buffer."""
    n = int(lib().brl_probe_rate_threads())
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device="cuda")
    _check(lib().brl_probe_rate(RATE_UNITS[unit], int(iters), _ptr(out), out.numel(), _stream(stream)))
    return out
