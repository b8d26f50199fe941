"""Benchmark of the bit-exact int8 LSQ linear layer and the ordered gradient
reduction on one MI355X.

One step = the whole hot path on synthetic inputs already resident in HBM:
  (1) qat_linear_fwd + qat_linear_bwd of the three linear layers of one
      Open-1B block at the per-GPU microbatch of 16384 tokens:
        - attention QKV projection (GQA 16 query / 4 KV heads of 128):
          X [16384, 2048], W [3072, 2048], dY [16384, 3072], seed 1;
        - SwiGLU gate+up projection with its activation: X [16384, 2048],
          W [11264, 2048] (gate and up stacked), dA [16384, 5632], seed 2;
        - down projection: H [16384, 5632], W [2048, 5632], dY [16384,
          2048], seed 3, backward over 4 microbatches of 4096 rows with dW
          accumulated in ascending order (the forward is row by row, so it
          runs as one call);
  (2) the single-device replay of one step's gradient reduction: 48 virtual
      ranks (6 replicas x 8 shards) of 201,326,592 fp32 each, fed in mesh
      order to ordered_reduce, then grad_l2norm_clip (max norm 1.0).
value = fwd+bwd int8-QAT linear throughput of the three layers in TOPS
(sum of 6*M*N*K over the layers / their time); per-layer figures, each
phase against its roofline, are under "configs".
ordered_reduce_GBps = algorithmic replay bytes / replay time.

Prints one JSON line.  --gpus above 1 is refused (one GPU).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bit-exact int8 QAT linear TOPS fwd+bwd (M=16384); ordered-reduce GB/s"

# MI355X published peaks (dense) and the derived fp32 VALU rate without FMA
# or packed instructions: 256 CU x 4 SIMD x 32 lanes per clock x 2.4 GHz
# (a wave64 v_add_f32 / v_mul_f32 with vector-register operands issues in two
# clocks; the published 157.3 TFLOP/s counts each FMA as two operations).
# The library's rate probe (brl_probe_rate, timed under "measured_peaks")
# sustains 67 T ops/s for those, 37 with a scalar-register operand, 71 for
# 32-bit integer ops, 77.7 T products/s on the K=1 fp32 MFMA and 4970 TOPS on
# the i8 MFMA with fixed operands, but 3530 TOPS when the operands change from
# one MFMA to the next as a GEMM's do (the chip lowers its clock under the
# higher power; the forward reports its fraction of that too).  dX and dW pair each matrix-core product with one VALU add (2
# ops); the probe of that pattern alone, with no memory traffic, sustains
# about 35 T multiply-adds/s = 70 T ops/s (the two units do not overlap in
# it), reported beside the published-rate fraction as "frac_of_engine".
PEAK_HBM_GBPS = 8000.0
PEAK_I8_TOPS = 5030.0
PEAK_VALU_F32_TOPS = 256 * 128 * 2.4e9 / 1e12         # 78.64 T ops/s

# Replay bytes per element index that the method must move with one
# replica's partials resident at a time (the bench keeps all 48 resident):
# each of the first 5 replicas reads its 8 partials and writes A_r (36 B);
# the last replica's running sum is formed inside the TreeFold, which reads
# A_0..A_4 and the 8 partials and writes T (56 B; the squared-norm CanonSum
# could ride on that pass, so it adds nothing); clip reads and writes T (8 B).
# (With at most two partials resident -- one add pass per shard -- it would
# be 6 * 7 * 12 + 28 + 8 = 540 B.)
REPLAY_R, REPLAY_S = 6, 8
REPLAY_BYTES_PER_ELEM = (REPLAY_R - 1) * (REPLAY_S + 1) * 4 + (REPLAY_R - 1 + REPLAY_S + 1) * 4 + 8   # 244
RUNSUM_BYTES_PER_ELEM = (REPLAY_S + 1) * 4                                                              # 36

# State hash (the next row after the hot path, measured beside it, not part of
# `value`): the compiled SHA-256 block loop of the leaf kernel issues
# HASH_VALU_PER_BLOCK VALU instructions per 64-byte block, HASH_ALIGNBIT_PER_BLOCK
# of them v_alignbit_b32 (the rotations), which gfx950 issues at about half the
# rate of the other integer ops (34 T lane-ops/s measured, against 71 for
# shifts and xors in the rate probe).  A CPU test
# recounts both in the generated assembly.  VALU bound: 78.64e12 issue slots/s
# over (2 x alignbit + the rest) slots per block, times 64 bytes.
HASH_VALU_PER_BLOCK = 1561
HASH_ALIGNBIT_PER_BLOCK = 576
HASH_STATE_TENSORS = 8
# AdamW (the next row after the clip, measured beside the step): per parameter
# read p, g, m, v and write p, m, v.
ADAMW_BYTES_PER_ELEM = 28                                   # 8 x 805 MB = 6.44 GB
# Attention with int8 P.V (measured beside the step, not part of `value`): the
# method's logits are 2*D binary32 operations each (D products, D - 1 adds and
# the scale), counted once per (row, allowed key); the int8 P.V product is on
# the matrix cores and small beside them.
ATTN_D = 128
# the linear layers of one step (names of synth.CASES), in the order they run
LAYERS = ("qkv", "swiglu_gate_up", "down_proj")


def stream_bench(torch, brl, dev, with_cpu: bool):
    """The data stream (host, C++) on the synthetic corpus, and the device
    Philox draws (16 B written per 4-word block)."""
    import synth
    corpus = synth.corpus(7, scale=8)
    st = brl.DataStream(1, synth.SEPARATOR, corpus)
    st.next(8)
    t0 = time.perf_counter()
    n_win = 400
    st.next(n_win)
    dt = time.perf_counter() - t0
    out = {"data_stream": {"windows": n_win, "s": round(dt, 4), "windows_per_s": round(n_win / dt, 1),
                           "tokens_per_s": round(n_win * brl.STREAM_WINDOW / dt, 1), "threads": 1}}
    if with_cpu:
        from oracle import datastream as ds
        orc = ds.Stream(1, [ds.Source(n, w, sh) for n, w, sh in corpus], synth.SEPARATOR)
        t0 = time.perf_counter()
        for _ in range(20):
            orc.next_window()
        out["data_stream"]["oracle_windows_per_s"] = round(20 / (time.perf_counter() - t0), 2)
    n = 1 << 28
    buf = torch.empty(n, dtype=torch.int32, device=dev)
    brl.philox_u32(5, 0, 0, n, out=buf)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(3):
        brl.philox_u32(5, 0, 0, n, out=buf)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / 3
    gbps = 4.0 * n / (ms * 1e-3) / 1e9
    out["philox"] = {"draws": n, "ms": round(ms, 4), "draws_per_s": round(n / (ms * 1e-3), 1),
                     "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(gbps / PEAK_HBM_GBPS, 4),
                                  "note": "4 B written per draw; about 140 VALU issue slots per 4-word block "
                                          "(10 rounds of two 32x32->64 multiplies), close to the HBM ridge"}}
    del buf
    return out


def attention_bench(torch, brl, dev):
    """attn_fwd, attn_bwd_dq and attn_bwd_dkdv on one Open-1B layer's
    microbatch (4 x 4096 tokens, 16 query / 4 KV heads of 128), window 512 and
    full causal; device-generated inputs (parity at this size is a GPU test).
    Each kernel is timed on its own (the backward forming the logits again),
    then the training path: the forward keeping its logits and the backward
    reading them."""
    B, S, Hq, Hkv = 4, 4096, 16, 4
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    Q = torch.randn(B, S, Hq, ATTN_D, generator=g, device=dev)
    K = torch.randn(B, S, Hkv, ATTN_D, generator=g, device=dev)
    V = torch.randn(B, S, Hkv, ATTN_D, generator=g, device=dev)
    O = torch.empty_like(Q)
    dO = torch.randn(B, S, Hq, ATTN_D, generator=g, device=dev).mul_(1e-3)
    dQ = torch.empty_like(Q)
    dK, dV = torch.empty_like(K), torch.empty_like(V)
    stats = torch.empty(B, S, Hq, 2, device=dev)
    out = {"shape": {"B": B, "S": S, "Hq": Hq, "Hkv": Hkv, "D": ATTN_D, "s_v": 0.05}}

    def timed(fn, reps=3):
        fn()
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def line(ms, ops, note):
        return {"ms": round(ms, 4),
                "roofline": {"bound": "alu", "achieved": round(ops / (ms * 1e-3) / 1e12, 3),
                             "peak": round(PEAK_VALU_F32_TOPS, 2), "unit": "TFLOP/s",
                             "frac": round(ops / (ms * 1e-3) / 1e12 / PEAK_VALU_F32_TOPS, 4), "note": note}}

    for name, window in (("window_512", 512), ("causal", 0)):
        logits = B * Hq * sum(min(i + 1, window) if window > 0 else i + 1 for i in range(S))
        ops = 2.0 * ATTN_D * logits             # one binary32 product and add per (row, key, d)
        ms = timed(lambda: brl.attn_fwd(Q, K, V, window, 0.05, O=O), reps=10)
        out[name] = line(ms, ops, "2*D binary32 ops per allowed logit, counted once")
        out[name]["logits"] = logits
        # dQ with 64-bit fixed-point accumulation: logits, dP and the dS.K products
        brl.attn_fwd(Q, K, V, window, 0.05, O=O, stats=stats)
        ms_dq = timed(lambda: brl.attn_bwd_dq(Q, K, V, O, dO, stats, window, 0.05, dQ=dQ))
        out[name]["dq"] = line(ms_dq, 3 * ops, "3 * 2*D binary32 ops per allowed (row, key)")
        # dK and dV: logits, dP, P.dO and dS.Q
        ms_kv = timed(lambda: brl.attn_bwd_dkdv(Q, K, V, O, dO, stats, window, 0.05, dK=dK, dV=dV))
        out[name]["dkdv"] = line(ms_kv, 4 * ops, "4 * 2*D binary32 ops per allowed (row, key)")
        # the training path: the forward keeps its logits (attn_fwd_keep_logits), the
        # backward reads them (attn_bwd_dq_logits, attn_bwd_dkdv_logits)
        L = brl.attn_logits_buffer(B, S, Hq, window, dev)
        ms_fk = timed(lambda: brl.attn_fwd(Q, K, V, window, 0.05, O=O, stats=stats, logits=L), reps=10)
        ms_dqk = timed(lambda: brl.attn_bwd_dq(Q, K, V, O, dO, stats, window, 0.05, dQ=dQ, logits=L))
        ms_kvk = timed(lambda: brl.attn_bwd_dkdv(Q, K, V, O, dO, stats, window, 0.05, dK=dK, dV=dV, logits=L))
        tot = ms_fk + ms_dqk + ms_kvk
        out[name]["kept_logits"] = {
            "bytes": L.numel() * 4,
            "fwd": line(ms_fk, ops, "2*D ops per allowed logit; the logits written to HBM for the backward"),
            "dq": line(ms_dqk, 2 * ops, "2 * 2*D ops per allowed (row, key): dP and dS.K"),
            "dkdv": line(ms_kvk, 3 * ops, "3 * 2*D ops per allowed (row, key): dP, P.dO and dS.Q"),
            "layer_fwd_bwd": line(tot, 5 * ops, "fwd + dQ + dK/dV against 5 * 2*D ops per allowed (row, key): "
                                               "the logits, dP, dS.K, P.dO and dS.Q, each once (dP is formed "
                                               "by both backward kernels, counted once)")}
        del L
        torch.cuda.empty_cache()
    del Q, K, V, O, dO, dQ, dK, dV, stats
    return out


def measured_peaks(torch, brl):
    """Sustained rates of the units the rooflines price against, measured by
    the library's rate probe (full grid, 8 independent chains per thread):
    binary32 adds and multiplies on the VALU, products of the K=1 fp32 MFMA,
    and integer ops (2 per multiply-accumulate) of the i8 MFMA 32x32x32."""
    out = {}
    iters = {"v_add_f32": 100000, "v_mul_f32": 100000, "v_add_f32_sgpr": 50000, "valu_u32": 50000,
             "mfma_k1_f32": 20000, "k1_engine": 20000, "k1_engine_data": 5000, "mfma_i8": 8000,
             "mfma_i8_data": 2000}
    buf = torch.empty(int(brl.lib().brl_probe_rate_threads()), dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    for unit, n in iters.items():
        brl.probe_rate(unit, 16, buf)
        ms = []
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            brl.probe_rate(unit, n, buf)
            e1.record(st)
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        ops = buf.numel() * brl.RATE_OPS_PER_STEP[unit] * n
        out[unit] = {"T_ops_per_s": round(ops / (min(ms) * 1e-3) / 1e12, 2), "ms": round(min(ms), 3), "iters": n}
    out["note"] = ("v_add_f32 / v_mul_f32: binary32 operations with vector-register operands (_sgpr: one "
                   "scalar-register operand); valu_u32: 32-bit shifts and xors; mfma_k1_f32: products of "
                   "v_mfma_f32_16x16x1_4b_f32; k1_engine: multiply-adds of that MFMA (-0 accumulator) "
                   "followed by a v_add_f32 per product, no memory traffic; k1_engine_data: the same on "
                   "operands that change from one MFMA to the next; mfma_i8: integer ops of "
                   "v_mfma_i32_32x32x32_i8 on fixed operands; mfma_i8_data: the same with operands that change "
                   "from one MFMA to the next, as in a GEMM")
    return out


def measured_traffic(kernels, weights=None):
    """HBM bytes per dispatch from the committed rocprofv3 counter summary
    (FETCH_SIZE and WRITE_SIZE passes, calibrated with a copy kernel of known
    size): the dispatch-weighted average over `kernels` (entries of the
    summary), or None when a source or compiler flag of the library changed
    since the counters were taken."""
    import hashlib
    from bitwise_reproducible_lsq_amd import build as brl_build
    path = os.path.join(ROOT, "profiles", "hbm_traffic_bench_step.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    for src, digest in rec.get("sources_sha256", {}).items():
        f = os.path.join(ROOT, src)
        if not os.path.exists(f) or hashlib.sha256(open(f, "rb").read()).hexdigest() != digest:
            return None
    # compiler flags of every unit (include paths left out: they differ between machines)
    flags = {u: [f for f in brl_build.FLAGS + brl_build.EXTRA.get(u, []) if not f.startswith("-I")]
             for u in brl_build.SOURCES}
    if hashlib.sha256(json.dumps(flags, sort_keys=True).encode()).hexdigest() != rec.get("flags_sha256"):
        return None
    weights = weights or [1] * len(kernels)
    total = 0.0
    for k, w in zip(kernels, weights):
        e = rec.get("kernels", {}).get(k)
        if e is None:
            return None
        total += w * e["bytes"]
    return int(round(total / sum(weights)))


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=2)
    p.add_argument("--replay-length", type=int, default=None, help="override the partial length")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=20.0, help="rough budget for the oracle sample")
    return p.parse_args()


class Timer:
    """HIP events on the current stream around a region; summed per name."""

    def __init__(self, torch):
        self.torch = torch
        self.t = {}
        self.counts = {}

    def region(self, name):
        torch = self.torch
        timer = self

        class _R:
            def __enter__(self):
                self.a = torch.cuda.Event(enable_timing=True)
                self.b = torch.cuda.Event(enable_timing=True)
                self.a.record()
                return self

            def __exit__(self, *exc):
                self.b.record()
                timer.t.setdefault(name, []).append((self.a, self.b))
                return False

        return _R()

    def ms(self, name):
        pairs = self.t.get(name, [])
        if not pairs:
            return 0.0, 0
        return sum(a.elapsed_time(b) for a, b in pairs), len(pairs)

    def count(self, name, n):
        self.counts[name] = self.counts.get(name, 0) + n

    def clear(self):
        self.t.clear()
        self.counts.clear()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the replay of the "
              "cluster's reduction is itself a single-device computation", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bitwise_reproducible_lsq_amd as brl
    import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rcase = synth.REPLAY
    L = args.replay_length or rcase.length
    R, S = rcase.replicas, rcase.shards

    # ---- inputs, resident before timing ------------------------------------------
    layers = []
    for name in LAYERS:
        case = synth.CASES[name]
        inp = synth.linear_inputs(case)
        M, K, N = case.M, case.K, case.N
        epi = brl.EPILOGUE_SWIGLU if case.swiglu else brl.EPILOGUE_NONE
        lay = {"name": name, "case": case, "inp": inp, "M": M, "K": K, "N": N, "epi": epi,
               "mb": case.microbatches,
               "X": torch.from_numpy(inp.X).to(dev), "W": torch.from_numpy(inp.W).to(dev),
               "dY": torch.from_numpy(inp.dY).to(dev),
               "Y": torch.empty((M, N // 2 if case.swiglu else N), dtype=torch.float32, device=dev),
               "Ypre": torch.empty((M, N), dtype=torch.float32, device=dev) if case.swiglu else None,
               "dX": torch.empty((M, K), dtype=torch.float32, device=dev),
               "dW": torch.empty((N, K), dtype=torch.float32, device=dev),
               "ws_f": brl.workspace(brl.OP_FWD, M, K, N, dev),
               "ws_b": brl.workspace(brl.OP_BWD, M // case.microbatches, K, N, dev)}
        layers.append(lay)
    partials = [synth.replay_partial(rcase, v, device=dev, length=L) for v in range(R * S)]
    # all partials stay resident, so each replica's first two shards combine in one pass
    # all partials stay resident, so each replica's running sum is one pass
    # over its 8 partials (the last replica's inside the TreeFold)
    assert (R, S) == (REPLAY_R, REPLAY_S)
    state = brl.ReduceState(R, S, L, device=dev, replica_resident=True)
    out = torch.empty(L, dtype=torch.float32, device=dev)
    ws_n = brl.workspace(brl.OP_NORM, L, 0, 0, dev)
    torch.cuda.synchronize()

    peaks = measured_peaks(torch, brl)
    engine_tops = 2 * peaks["k1_engine"]["T_ops_per_s"]
    i8_data_tops = peaks["mfma_i8_data"]["T_ops_per_s"]
    timer = Timer(torch)

    def fwd(lay):
        brl.qat_linear_fwd(lay["X"], lay["W"], synth.S_X, epilogue=lay["epi"], Y=lay["Y"], ws=lay["ws_f"],
                           Ypre=lay["Ypre"])

    def bwd(lay, need_dX=True, need_dW=True):
        M, mb = lay["M"], lay["mb"]
        rows = M // mb
        for b in range(mb):
            sl = slice(b * rows, (b + 1) * rows)
            brl.qat_linear_bwd(lay["dY"][sl], lay["X"][sl], lay["W"], synth.S_X,
                               Ypre=lay["Ypre"][sl] if lay["Ypre"] is not None else None, epilogue=lay["epi"],
                               need_dX=need_dX, need_dW=need_dW,
                               dX=lay["dX"][sl] if need_dX else None, dW=lay["dW"] if need_dW else None,
                               dW_accumulate=need_dW and b > 0, ws=lay["ws_b"])

    def step(timed: bool):
        with timer.region("linear"):
            for lay in layers:
                with timer.region(lay["name"] + ".fwd"):
                    fwd(lay)
                with timer.region(lay["name"] + ".bwd"):
                    bwd(lay)
        state.reset()
        with timer.region("replay"):
            for r in range(R):
                # a replica's calls launch nothing until its last shard's,
                # which launches its running sum (or, for the last replica,
                # the TreeFold): one event pair around the replica's calls
                # times that one kernel
                with timer.region("runsum" if r < R - 1 else "fold"):
                    for s in range(S):
                        brl.ordered_reduce(state, partials[r * S + s], out=out)
                if r < R - 1:
                    timer.count("runsum_launches", 1)
            with timer.region("norm_clip"):
                brl.grad_l2norm_clip(out, rcase.max_norm, ws=ws_n)

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    timer.clear()

    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    K_ = args.steps
    lin_ms = timer.ms("linear")[0] / K_
    rep_ms = timer.ms("replay")[0] / K_
    acc_ms = timer.ms("runsum")[0]
    acc_n = timer.counts.get("runsum_launches", 0)
    fold_ms = timer.ms("fold")[0] / K_
    nc_ms = timer.ms("norm_clip")[0] / K_
    acc_avg_ms = acc_ms / max(acc_n, 1)

    # phase split of each layer (separate, after the timed steps)
    def avg_call(fn, reps=3):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    def frac(v, peak):
        return round(v / peak, 4)

    configs = {}
    total_ops = 0.0
    for lay in layers:
        M, K, N, name = lay["M"], lay["K"], lay["N"], lay["name"]
        ops = 2.0 * M * N * K
        total_ops += 3 * ops
        f_ms = timer.ms(name + ".fwd")[0] / K_
        b_ms = timer.ms(name + ".bwd")[0] / K_
        pre_ms = avg_call(lambda: bwd(lay, need_dX=False, need_dW=False))
        dx_ms = avg_call(lambda: bwd(lay, need_dX=True, need_dW=False)) - pre_ms
        dw_ms = avg_call(lambda: bwd(lay, need_dX=False, need_dW=True)) - pre_ms
        t_fwd = ops / (f_ms * 1e-3) / 1e12
        t_dx = ops / (dx_ms * 1e-3) / 1e12
        t_dw = ops / (dw_ms * 1e-3) / 1e12
        t_all = 3 * ops / ((f_ms + b_ms) * 1e-3) / 1e12
        # combined roofline: the forward at the i8 peak plus dX and dW at the VALU ceiling
        t_min = ops / (PEAK_I8_TOPS * 1e12) + 2 * ops / (PEAK_VALU_F32_TOPS * 1e12)
        configs[name] = {
            "M": M, "K": K, "N": N, "seed": lay["case"].seed,
            "epilogue": "swiglu" if lay["epi"] else "none", "bwd_microbatches": lay["mb"],
            "ms": {"fwd": round(f_ms, 4), "bwd": round(b_ms, 4), "bwd_prelude": round(pre_ms, 4),
                   "dX": round(dx_ms, 4), "dW": round(dw_ms, 4), "fwd_bwd": round(f_ms + b_ms, 4)},
            "fwd": {"bound": "mfma", "achieved": round(t_fwd, 2), "peak": PEAK_I8_TOPS, "unit": "TOPS",
                    "frac": frac(t_fwd, PEAK_I8_TOPS),
                    "frac_of_measured_data_peak": frac(t_fwd, i8_data_tops)},
            "dX": {"bound": "alu", "achieved": round(t_dx, 3), "peak": round(PEAK_VALU_F32_TOPS, 2),
                   "unit": "TFLOP/s", "frac": frac(t_dx, PEAK_VALU_F32_TOPS),
                   "frac_of_engine": frac(t_dx, engine_tops)},
            "dW": {"bound": "alu", "achieved": round(t_dw, 3), "peak": round(PEAK_VALU_F32_TOPS, 2),
                   "unit": "TFLOP/s", "frac": frac(t_dw, PEAK_VALU_F32_TOPS),
                   "frac_of_engine": frac(t_dw, engine_tops)},
            "fwd_bwd": {"achieved": round(t_all, 3), "unit": "TOPS",
                        "combined_peak": round(3 * ops / t_min / 1e12, 2),
                        "frac": round(t_all / (3 * ops / t_min / 1e12), 4),
                        "frac_of_i8_peak": frac(t_all, PEAK_I8_TOPS)},
        }

    # the dominant kernel by time per step: the matrix-core product kernel of
    # dX (ste_mfma_kernel<true, 7>), one launch per microbatch of each layer;
    # its dW twin takes about 2% less.  achieved = the launches' algorithmic
    # operations (a product and an add per reduction step) over their time
    # time: each layer's backward inside the timed steps, less its operand
    # preparation, split between dX and dW in the ratio of the dX-only and
    # dW-only calls timed after the steps (those standalone calls alone run
    # a few percent faster than inside the step)
    dx_ops = sum(2.0 * lay["M"] * lay["N"] * lay["K"] for lay in layers)
    dx_ms_sum = 0.0
    for lay in layers:
        c = configs[lay["name"]]["ms"]
        dx_ms_sum += (c["bwd"] - c["bwd_prelude"]) * c["dX"] / (c["dX"] + c["dW"])
    dx_launches = sum(lay["mb"] for lay in layers)
    dx_rate = dx_ops / (dx_ms_sum * 1e-3) / 1e12
    dx_traffic = measured_traffic(["brl::ste_mfma_kernel<true, 7> [qkv dX]",
                                   "brl::ste_mfma_kernel<true, 7> [swiglu_gate_up dX]",
                                   "brl::ste_mfma_kernel<true, 7> [down_proj dX]"], weights=[1, 1, 4])
    dx_alg = sum(4.0 * (lay["M"] * lay["N"] + lay["N"] * lay["K"] * lay["mb"] + lay["M"] * lay["K"])
                 for lay in layers) / dx_launches
    dx_roofline = {
        "kernel": f"ste_mfma_kernel<true, 7> (dX: K=1 fp32 MFMA products, ordered binary32 adds; "
                  f"{dx_launches} launches per step: QKV 1, SwiGLU gate+up 1, down projection 4 microbatches)",
        "bound": "alu", "achieved": round(dx_rate, 3), "peak": round(PEAK_VALU_F32_TOPS, 2), "unit": "TFLOP/s",
        "frac": round(dx_rate / PEAK_VALU_F32_TOPS, 4), "frac_of_engine": round(dx_rate / engine_tops, 4),
        "ops_per_launch": round(dx_ops / dx_launches), "ms_per_step": round(dx_ms_sum, 4),
        "timing": "each layer's qat_linear_bwd time in the timed steps (HIP events on the call stream) less "
                  "its operand preparation, split between dX and dW in the ratio of dX-only and dW-only calls "
                  "timed after the steps (the step's calls form dX and dW together); the finish pass over "
                  "chunk roots is included (about 1% on gate+up)",
        "traffic": dx_traffic, "traffic_unit": "bytes per launch (average over the step's launches)",
        "algorithmic_bytes": round(dx_alg),
    }
    tops = total_ops / (lin_ms * 1e-3) / 1e12
    replay_bytes = REPLAY_BYTES_PER_ELEM * L
    replay_gbps = replay_bytes / (rep_ms * 1e-3) / 1e9
    acc_bytes = float(RUNSUM_BYTES_PER_ELEM) * L
    acc_gbps = acc_bytes / (acc_avg_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(tops, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": K_,
        "warmup": args.warmup,
        "ms_per_step": round(wall / K_ * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8->i32 fwd GEMM; f32 bwd and replay",
        "data": "synthetic (seeded Philox Gaussians; device-generated replay partials)",
        "config": {
            "workload": "Open-1B block linears at M=16384 fwd+bwd: QKV 2048->3072 (seed 1), SwiGLU gate+up "
                        "2048->2x5632 with activation (seed 2), down 5632->2048 with 4 microbatches (seed 3); "
                        f"+ replay 6x8 ranks x {L} fp32 (seed 4), clip 1.0",
            "layers": {lay["name"]: [lay["M"], lay["K"], lay["N"]] for lay in layers},
            "s_x": synth.S_X, "replicas": R, "shards": S, "replay_length": L,
        },
        "ordered_reduce_GBps": round(replay_gbps, 1),
        "ordered_reduce_bytes_per_element": REPLAY_BYTES_PER_ELEM,
        "phases_ms": {
            "linear_fwd_bwd": round(lin_ms, 4), "replay": round(rep_ms, 4),
            "runsum_avg": round(acc_avg_ms, 5), "fold": round(fold_ms, 4), "norm_clip": round(nc_ms, 4),
        },
        "configs": configs,
        "roofline": dx_roofline,
        "rooflines_other": {
            "running_sum": {
                "kernel": f"runsum_v4_kernel (a replica's running sum over its {S} resident partials in one pass, "
                          f"{acc_n // max(K_, 1)} launches per step, each timed with one event pair around the "
                          "replica's calls)",
                "bound": "hbm", "achieved": round(acc_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(acc_gbps / PEAK_HBM_GBPS, 4), "algorithmic_bytes": int(acc_bytes),
                "traffic": measured_traffic(["brl::runsum_v4_kernel"]) if L == rcase.length else None,
                "traffic_unit": "bytes per launch"},
            "replay_total": {"bound": "hbm", "achieved": round(replay_gbps, 1), "peak": PEAK_HBM_GBPS,
                             "unit": "GB/s", "frac": round(replay_gbps / PEAK_HBM_GBPS, 4)},
            "fwd_call": dict(configs["qkv"]["fwd"], layer="qkv"),
            "dX": dict(configs["qkv"]["dX"], layer="qkv"),
            "dW": dict(configs["qkv"]["dW"], layer="qkv"),
        },
    }
    # AdamW over the reduced, clipped gradient (L parameters; p, m, v synthetic)
    ap = synth.replay_partial(rcase, 100, device=dev, length=L)
    am = torch.zeros(L, dtype=torch.float32, device=dev)
    av = torch.zeros(L, dtype=torch.float32, device=dev)
    asc = brl.adamw_scalars_for_step(1000, 3.0e9)
    adamw_ms = avg_call(lambda: brl.adamw_step(ap, out, am, av, asc), reps=3)
    adamw_gbps = ADAMW_BYTES_PER_ELEM * L / (adamw_ms * 1e-3) / 1e9
    del ap, am, av
    # state hash of a 6.44 GB state (the first 8 replay partials as its tensors)
    hstate = partials[:HASH_STATE_TENSORS]
    hash_bytes = sum(t.numel() * 4 for t in hstate)
    hash_ms = avg_call(lambda: brl.state_hash(hstate), reps=3)
    result["adamw"] = {
        "params": L, "ms": round(adamw_ms, 4),
        "roofline": {"bound": "hbm", "achieved": round(adamw_gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(adamw_gbps / PEAK_HBM_GBPS, 4),
                     "note": f"{ADAMW_BYTES_PER_ELEM} B per parameter (read p, g, m, v; write p, m, v)"},
    }
    hash_gbps = hash_bytes / (hash_ms * 1e-3) / 1e9
    hash_slots = HASH_VALU_PER_BLOCK + HASH_ALIGNBIT_PER_BLOCK
    hash_peak = PEAK_VALU_F32_TOPS * 1e12 / hash_slots * 64 / 1e9
    result["state_hash"] = {
        "bytes": hash_bytes, "ms": round(hash_ms, 4), "GBps": round(hash_gbps, 1),
        "roofline": {"bound": "alu", "achieved": round(hash_gbps, 1), "peak": round(hash_peak, 1),
                     "unit": "GB/s", "frac": round(hash_gbps / hash_peak, 4),
                     "note": (f"{HASH_VALU_PER_BLOCK} VALU instructions per 64-byte SHA-256 block, "
                              f"{HASH_ALIGNBIT_PER_BLOCK} of them half-rate rotations")},
    }
    del hstate
    result["measured_peaks"] = peaks
    result["attention"] = attention_bench(torch, brl, dev)
    if not args.no_cpu_baseline:
        result["attention"]["cpu_baseline"] = cpu_attention_rate()
    result.update(stream_bench(torch, brl, dev, not args.no_cpu_baseline))
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(layers[0]["inp"], args.cpu_seconds)
        result["cpu_baseline"]["state_hash_GBps"] = cpu_hash_rate([partials[0].cpu().numpy()])
    print(json.dumps(result), flush=True)


def cpu_hash_rate(tensors) -> float:
    """The state-hash oracle (hashlib, one thread, as it stands) on one 805 MB tensor."""
    from oracle import state_hash as sh
    t0 = time.perf_counter()
    sh.state_hash(tensors)
    dt = time.perf_counter() - t0
    return round(sum(t.nbytes for t in tensors) / dt / 1e9, 3)


def cpu_attention_rate():
    """The attention oracle on sampled rows of the window-512 layer: the same
    algorithmic ops per second as the GPU figure (2*D per allowed logit; dQ
    three such products, dK/dV four)."""
    import numpy as np

    import oracle
    import synth
    case = synth.ATTENTION_CASES["attn_window"]
    Q, K, V = synth.attention_inputs(case)
    g = np.random.default_rng(0)
    rows = np.sort(g.choice(case.B * case.S * case.Hq, 256, replace=False))
    keys = sum(min(int(r // case.Hq) % case.S + 1, case.window) for r in rows)
    t0 = time.perf_counter()
    O = oracle.attn_fwd_rows(Q, K, V, case.window, case.s_v, rows)
    t_fwd = time.perf_counter() - t0
    Ofull = np.zeros_like(Q).reshape(-1, ATTN_D)
    Ofull[rows] = O
    dO = synth.normal(case.seed, "dY", Q.shape, 1e-3)
    t0 = time.perf_counter()
    oracle.attn_bwd_dq(Q, K, V, Ofull.reshape(Q.shape), dO, case.window, case.s_v, rows=rows)
    t_dq = time.perf_counter() - t0
    kv_rows = np.sort(g.choice(case.B * case.S * case.Hkv, 8, replace=False))
    group = case.Hq // case.Hkv
    pairs = sum(group * min(case.S - int(r // case.Hkv) % case.S, case.window) for r in kv_rows)
    t0 = time.perf_counter()
    oracle.attn_bwd_dkdv(Q, K, V, Ofull.reshape(Q.shape), dO, case.window, case.s_v, rows=kv_rows)
    t_kv = time.perf_counter() - t0
    return {"kind": "oracle", "cores": oracle.num_threads(),
            "sample": "256 random rows (fwd, dQ) and 8 random key rows (dK/dV) of the window-512 layer",
            "fwd_T_ops_per_s": round(2.0 * ATTN_D * keys / t_fwd / 1e12, 6),
            "dq_T_ops_per_s": round(3 * 2.0 * ATTN_D * keys / t_dq / 1e12, 6),
            "dkdv_T_ops_per_s": round(4 * 2.0 * ATTN_D * pairs / t_kv / 1e12, 8)}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, budget_s: float):
    """The oracle, as it stands, on a bounded sample of the same workload:
    some rows of Y and dX and some rows of dW of the QKV layer, and the replay
    over a prefix of the element range."""
    import numpy as np

    import oracle
    import synth

    M, K = inp.X.shape
    N = inp.W.shape[0]
    s_w = oracle.weight_scale(inp.W)
    g = np.random.default_rng(0)

    def run(n_rows, n_wrows):
        rows = np.sort(g.choice(M, n_rows, replace=False))
        wr = np.sort(g.choice(N, n_wrows, replace=False))
        t0 = time.perf_counter()
        oracle.fwd_rows(inp.X, inp.W, synth.S_X, rows=rows, s_w=s_w)
        oracle.dx_rows(inp.dY[rows], inp.X, inp.W, synth.S_X, rows, s_w=s_w)
        oracle.dw_rows(np.ascontiguousarray(inp.dY[:, wr].T), inp.X, inp.W, synth.S_X, wr, s_w=s_w)
        dt = time.perf_counter() - t0
        return dt, 2.0 * K * N * n_rows * 2 + 2.0 * M * K * n_wrows

    # grow the sample until one run takes ~40-70% of the budget; that run is the measurement
    n_rows, n_wrows = 8, 2
    while True:
        t_lin, ops = run(n_rows, n_wrows)
        if t_lin > 0.4 * budget_s or n_rows >= M:
            break
        scale = min(16.0, max(1.5, 0.6 * budget_s / max(t_lin, 1e-3)))
        n_rows = int(min(M, n_rows * scale))
        n_wrows = int(min(N, max(n_wrows + 1, n_wrows * scale)))
    rows, wr = range(n_rows), range(n_wrows)
    # replay over 2^24 elements of each of the 48 ranks (8 distinct partials,
    # each fed to six ranks: the oracle's cost does not depend on the values)
    Ls = 1 << 24
    distinct = [synth.replay_partial_host(synth.REPLAY.seed, v, Ls) for v in range(8)]
    parts = [distinct[v % 8] for v in range(48)]
    # repeated until it has run for ~15% of the budget (a rate: repeats of one
    # sample measure the same thing as a longer sample)
    reps, t_rep = 0, 0.0
    while t_rep < 0.15 * budget_s and reps < 64:
        t0 = time.perf_counter()
        oracle.replay(parts, 6, 8)
        t_rep += time.perf_counter() - t0
        reps += 1
    # the tiny layer (256 x 512 x 512, seed 42, with subnormal dY) forward and
    # backward on one thread
    tiny = synth.linear_inputs(synth.CASES["tiny"])
    threads = oracle.num_threads()
    oracle.set_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.linear_fwd(tiny.X, tiny.W, synth.S_X)
        oracle.linear_bwd(tiny.dY, tiny.X, tiny.W, synth.S_X)
        t_tiny = time.perf_counter() - t0
    finally:
        oracle.set_threads(threads)
    tc = tiny.case
    return {
        "value": round(ops / t_lin / 1e12, 6),
        "unit": "TOPS",
        "cores": threads,
        "nproc": os.cpu_count(),
        "cpu_affinity": len(os.sched_getaffinity(0)),
        "cpu_model": _cpu_model(),
        "tiny_1thread": {"TOPS": round(6.0 * tc.M * tc.N * tc.K / t_tiny / 1e12, 6), "s": round(t_tiny, 3),
                         "shape": [tc.M, tc.K, tc.N]},
        "kind": "oracle",
        "sample": (f"QKV layer: {len(rows)} rows of Y and dX, {len(wr)} rows of dW "
                   f"({ops / 1e9:.1f} G ops, {t_lin:.1f} s); replay of 48 ranks x {Ls} elements "
                   f"(8 distinct partials reused), {reps} times ({t_rep:.2f} s)"),
        "ordered_reduce_GBps": round(REPLAY_BYTES_PER_ELEM * Ls * reps / t_rep / 1e9, 3),
    }


if __name__ == "__main__":
    main()
