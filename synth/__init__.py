"""Seeded synthetic inputs for the bitwise-reproducible int8 LSQ linear layer
and the gradient-reduction replay.

This module only draws random numbers; it holds none of the method's
arithmetic.  The same bytes feed the HIP library and the CPU oracle.

Stand-in for the pages' workload: Open-1B activations and weights at the
per-GPU microbatch of 4 sequences x 4096 tokens (onedev.kr summary, "Limits",
recipe paragraph).  The corpus and trained weights are not available, so
seeded Gaussians of the stated shapes stand in.

Generators:
  * linear-layer tensors: numpy's Philox4x32-10 bit generator keyed by
    (seed, tensor id), standard normals drawn in float64, scaled by the
    standard deviation and rounded to float32;
  * replay partials: one vector per virtual rank, drawn on the device by
    torch's Philox-based generator seeded with seed * 1000 + v (fast at
    201M elements per rank); the oracle receives a byte copy.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

S_X = 0.05          # activation step: a caller constant, one value for every layer

TENSOR_ID = {"X": 1, "W": 2, "dY": 3, "gate": 4, "lin": 5, "mask": 6, "sub": 7, "addend": 8,
             "Q": 9, "K": 10, "V": 11}


@dataclass(frozen=True)
class LinearCase:
    name: str
    seed: int
    M: int
    K: int
    N: int
    x_kind: str = "normal"        # "normal" or "silu_x_normal"
    w_std: float = 0.02
    dy_std: float = 1e-3
    subnormal_frac: float = 0.0   # fraction of dY entries replaced by subnormals
    swiglu: bool = False          # N is gate+up stacked; dY is [M, N/2]
    microbatches: int = 1
    s_x: float = S_X


@dataclass(frozen=True)
class ReplayCase:
    name: str
    seed: int
    replicas: int
    shards: int
    length: int
    std: float = 1e-4
    max_norm: float = 1.0


CASES = {
    "tiny": LinearCase("tiny", 42, 256, 512, 512, subnormal_frac=0.01),
    "qkv": LinearCase("qkv", 1, 16384, 2048, 3072),
    "swiglu_gate_up": LinearCase("swiglu_gate_up", 2, 16384, 2048, 11264, swiglu=True),
    "down_proj": LinearCase("down_proj", 3, 16384, 5632, 2048, x_kind="silu_x_normal",
                            microbatches=4),
}
REPLAY = ReplayCase("replay_6x8", 4, 6, 8, 201_326_592)


def _rng(seed: int, tensor: str) -> np.random.Generator:
    key = (int(seed) << 32) | TENSOR_ID[tensor]
    return np.random.Generator(np.random.Philox(key=key))


def normal(seed: int, tensor: str, shape, std: float) -> np.ndarray:
    g = _rng(seed, tensor)
    return (g.standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def silu_x_normal(seed: int, shape) -> np.ndarray:
    """SiLU(a) * b with a, b ~ N(0,1), in float64 (shapes the down-projection
    input like a SwiGLU output), rounded to float32."""
    a = _rng(seed, "X").standard_normal(shape, dtype=np.float64)
    b = _rng(seed, "gate").standard_normal(shape, dtype=np.float64)
    return (a / (1.0 + np.exp(-a)) * b).astype(np.float32)


def inject_subnormals(x: np.ndarray, seed: int, frac: float) -> np.ndarray:
    """Replace a fraction of entries by random subnormals (random sign,
    mantissa uniform in [1, 2^23 - 1])."""
    if frac <= 0:
        return x
    g = _rng(seed, "mask")
    pick = g.random(x.shape) < frac
    h = _rng(seed, "sub")
    mant = h.integers(1, 1 << 23, size=x.shape, dtype=np.uint32)
    sign = h.integers(0, 2, size=x.shape, dtype=np.uint32) << np.uint32(31)
    bits = x.view(np.uint32).copy()
    bits[pick] = (sign | mant)[pick]
    return bits.view(np.float32)


@dataclass
class LinearInputs:
    case: LinearCase
    X: np.ndarray
    W: np.ndarray
    dY: np.ndarray            # output gradient ([M,N], or [M,N/2] after SwiGLU)
    extra: dict = field(default_factory=dict)


def linear_inputs(case: LinearCase, M: int | None = None) -> LinearInputs:
    """Host arrays for a linear-layer case; M overrides the row count
    (prefix rows of the same stream are not guaranteed, so sub-sized
    problems use their own draw)."""
    M = case.M if M is None else M
    K, N = case.K, case.N
    if case.x_kind == "silu_x_normal":
        X = silu_x_normal(case.seed, (M, K))
    else:
        X = normal(case.seed, "X", (M, K), 1.0)
    W = normal(case.seed, "W", (N, K), case.w_std)
    n_out = N // 2 if case.swiglu else N
    dY = normal(case.seed, "dY", (M, n_out), case.dy_std)
    dY = inject_subnormals(dY, case.seed, case.subnormal_frac)
    return LinearInputs(case, X, W, dY)


@dataclass(frozen=True)
class AttentionCase:
    """Attention of one Open-1B layer at the per-GPU microbatch: 4 sequences
    of 4096 tokens, 16 query heads over 4 KV heads of 128 (onedev.kr summary,
    "Use"); window 512 on most layers, 0 (full causal) on every fifth and the
    last.  Q and K ~ N(0, 1) stand in for the QK-normalised (unit RMS, no gain)
    projections, V ~ N(0, 1)."""
    name: str
    seed: int
    B: int = 4
    S: int = 4096
    Hq: int = 16
    Hkv: int = 4
    window: int = 512
    s_v: float = S_X


ATTENTION_CASES = {
    "attn_window": AttentionCase("attn_window", 5),
    "attn_causal": AttentionCase("attn_causal", 6, window=0),
}


def attention_inputs(case: AttentionCase, S: int | None = None):
    """Host Q [B,S,Hq,128], K and V [B,S,Hkv,128] for an attention case."""
    S = case.S if S is None else S
    Q = normal(case.seed, "Q", (case.B, S, case.Hq, 128), 1.0)
    K = normal(case.seed, "K", (case.B, S, case.Hkv, 128), 1.0)
    V = normal(case.seed, "V", (case.B, S, case.Hkv, 128), 1.0)
    return Q, K, V


def small_case(name: str, seed: int, M: int, K: int, N: int, **kw) -> LinearCase:
    return LinearCase(name, seed, M, K, N, **kw)


def replay_partial(case: ReplayCase, v: int, device="cuda", length: int | None = None):
    """Partial gradient of virtual rank v as a float32 torch tensor on device."""
    import torch
    L = case.length if length is None else length
    g = torch.Generator(device=device)
    g.manual_seed(case.seed * 1000 + v)
    t = torch.randn(L, generator=g, device=device, dtype=torch.float32)
    t.mul_(case.std)
    return t


def replay_partial_host(seed: int, v: int, length: int, std: float = 1e-4) -> np.ndarray:
    """Host-side partial for small CPU-only replay cases."""
    g = np.random.Generator(np.random.Philox(key=(int(seed) << 32) | (1000 + v)))
    return (g.standard_normal(length, dtype=np.float64) * std).astype(np.float32)


# ---- synthetic corpus for the data stream -------------------------------------------
SEPARATOR = 0
VOCAB = 50304


def corpus(seed: int = 7, scale: int = 1):
    """Sources standing in for a training mix (the pages' corpus is not
    available): (name, weight, shards), each shard a list of int32 token
    arrays.  Document lengths are log-normal (median ~660 tokens, a long
    tail up to 20000), tokens uniform in [1, VOCAB) (0 is the separator)."""
    g = np.random.default_rng(seed)
    spec = [("web/cc-2024", 6, 4, 30), ("code/github", 2, 3, 20), ("math/proofs", 1, 2, 12),
            ("books/long", 1, 1, 4)]
    out = []
    for name, weight, n_shards, n_docs in spec:
        shards = []
        for _ in range(n_shards):
            docs = []
            for _ in range(int(g.integers(max(1, n_docs // 2), n_docs * scale + 1))):
                mu = 9.0 if name.startswith("books") else 6.5
                n = int(min(20000, max(1, round(g.lognormal(mu, 1.0)))))
                docs.append(g.integers(1, VOCAB, n).astype(np.int32))
            shards.append(docs)
        out.append((name, weight, shards))
    return out
