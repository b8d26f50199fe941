"""CPU checks of the C-ABI library: it loads, exports every function that
include/brlsq.h declares, validates arguments before touching the device,
and its gfx950 code contains no fused or packed fp32 arithmetic outside the
correctly rounded division sequence.  No kernel is launched here."""
import ctypes as C
import subprocess
import os
import re

import pytest

import bitwise_reproducible_lsq_amd as brl
from bitwise_reproducible_lsq_amd import build as brl_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "brlsq.h")


def _declared():
    text = open(HEADER).read()
    return re.findall(r"BRL_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


def test_header_declares_the_four_calls():
    names = _declared()
    for n in ("qat_linear_fwd", "qat_linear_bwd", "ordered_reduce", "grad_l2norm_clip"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = C.CDLL(brl.LIB_PATH)
    missing = [n for n in _declared() if not hasattr(L, n)]
    assert not missing, missing


def test_workspace_query_is_host_only():
    assert brl.workspace_bytes(brl.OP_FWD, 256, 512, 512) > 0
    assert brl.workspace_bytes(brl.OP_BWD, 256, 512, 512) > 0
    assert brl.workspace_bytes(brl.OP_NORM, 1000, 0, 0) > 0
    assert brl.workspace_bytes(brl.OP_FWD, 256, 0, 512) == 0
    assert brl.workspace_bytes(7, 1, 1, 1) == 0


def _fwd(M=4, K=4, N=4, s_x=0.05, X=1, W=1, Y=1, ws=1, ws_bytes=1 << 20, epi=0):
    L = brl.lib()
    p = lambda v: C.c_void_p(0x10000) if v else None
    return L.qat_linear_fwd(p(X), p(W), M, K, N, s_x, None, epi, p(Y), None, None, p(ws), ws_bytes, None, None)


def test_fwd_rejects_bad_arguments_without_launching():
    assert _fwd(M=-1) == brl.BRL_ESHAPE
    assert _fwd(K=0) == brl.BRL_ESHAPE
    assert _fwd(K=200_000) == brl.BRL_ESHAPE
    assert _fwd(s_x=0.0) == brl.BRL_EINVAL
    assert _fwd(s_x=float("inf")) == brl.BRL_EINVAL
    assert _fwd(s_x=float("nan")) == brl.BRL_EINVAL
    assert _fwd(W=0) == brl.BRL_EINVAL
    assert _fwd(epi=3) == brl.BRL_EINVAL
    assert _fwd(N=5, epi=1) == brl.BRL_ESHAPE
    assert _fwd(ws_bytes=16) == brl.BRL_EWORKSPACE
    assert _fwd(ws=0) == brl.BRL_EWORKSPACE
    assert b"workspace" in brl.lib().brl_last_error()


def test_bwd_rejects_bad_arguments_without_launching():
    L = brl.lib()
    p = C.c_void_p(0x10000)
    assert L.qat_linear_bwd(p, p, p, None, 4, 4, 4, 0.05, 1, p, p, 0, p, 1 << 20, None, None) == brl.BRL_EINVAL
    assert L.qat_linear_bwd(p, p, p, None, 4, 4, 4, 0.05, 0, p, p, 2, p, 1 << 20, None, None) == brl.BRL_EINVAL
    assert L.qat_linear_bwd(p, p, p, None, 4, -4, 4, 0.05, 0, p, p, 0, p, 1 << 20, None, None) == brl.BRL_ESHAPE
    assert L.qat_linear_bwd(p, p, p, None, 4, 4, 4, 0.05, 0, p, p, 0, p, 8, None, None) == brl.BRL_EWORKSPACE
    # a workspace that is not 256-byte aligned
    assert L.qat_linear_bwd(p, p, p, None, 4, 4, 4, 0.05, 0, p, p, 0, C.c_void_p(0x10010), 1 << 20, None,
                            None) == brl.BRL_EINVAL


def test_state_hash_rejects_bad_arguments_without_launching():
    L = brl.lib()
    p = C.c_void_p(0x10000)

    def call(ptrs, lens, count, digest=p, ws=p, ws_bytes=1 << 20):
        P = (C.c_void_p * max(1, len(ptrs)))(*ptrs)
        N = (C.c_int64 * max(1, len(lens)))(*lens)
        return L.brl_state_hash(C.cast(P, C.c_void_p), C.cast(N, C.c_void_p), count, digest, ws, ws_bytes, None)

    assert call([], [], 0) == brl.BRL_EINVAL
    assert call([0x10000], [-1], 1) == brl.BRL_ESHAPE
    assert call([None], [16], 1) == brl.BRL_EINVAL                 # null data with bytes
    assert call([0x10002], [16], 1) == brl.BRL_EINVAL              # not 4-byte aligned
    assert call([0x10000], [16], 1, digest=None) == brl.BRL_EINVAL
    assert call([0x10000], [1 << 30], 1, ws_bytes=64) == brl.BRL_EWORKSPACE
    need = brl.workspace_bytes(brl.OP_HASH, (1 << 30) + 5, 2, 0)
    assert need >= 32 * ((1 << 30) // 16384 + 1)
    assert brl.workspace_bytes(brl.OP_HASH, 10, 0, 0) == 0


def test_reduce_state_order_is_enforced_on_the_host():
    L = brl.lib()
    st = brl.ReduceStateC()
    bufs = (C.c_void_p * 6)(*([0x10000] * 6))
    assert L.brl_reduce_init(C.byref(st), 0, 8, 16, C.cast(bufs, C.c_void_p)) == brl.BRL_ESHAPE
    assert L.brl_reduce_init(C.byref(st), 65, 8, 16, C.cast(bufs, C.c_void_p)) == brl.BRL_ESHAPE
    assert L.brl_reduce_init(C.byref(st), 6, 8, 16, C.cast(bufs, C.c_void_p)) == brl.BRL_OK
    assert st.next == 0 and st.replicas == 6 and st.shards == 8
    st.next = 48
    assert L.ordered_reduce(C.byref(st), C.c_void_p(0x10000), C.c_void_p(0x10000), None) == brl.BRL_EORDER
    st.next = 47
    assert L.ordered_reduce(C.byref(st), C.c_void_p(0x10000), None, None) == brl.BRL_EINVAL  # last needs out
    assert st.next == 47


def test_norm_rejects_bad_arguments():
    L = brl.lib()
    p = C.c_void_p(0x10000)
    assert L.grad_l2norm_clip(p, 16, 0.0, 0.0, None, p, 1 << 20, None, None) == brl.BRL_EINVAL
    assert L.grad_l2norm_clip(p, 16, 1.0, -1.0, None, p, 1 << 20, None, None) == brl.BRL_EINVAL
    assert L.grad_l2norm_clip(p, -1, 1.0, 0.0, None, p, 1 << 20, None, None) == brl.BRL_ESHAPE
    assert L.grad_l2norm_clip(p, 16, 1.0, 0.0, None, p, 4, None, None) == brl.BRL_EWORKSPACE


def test_tuning_is_per_call_and_checked():
    """Launch shapes travel with each call (no library state): bad values
    fail the call before any launch, the workspace query follows the chunk
    depth it is given, and a reduce state carries its own copy."""
    L = brl.lib()
    p = C.c_void_p(0x10000)
    bad = [brl.Tuning(bwd_chunk_log2=8), brl.Tuning(bwd_chunk_log2=-1), brl.Tuning(reduce_wg_blocks=100),
           brl.Tuning(stream_vec=3), brl.Tuning(bwd_engine=3)]
    for t in bad:
        assert L.qat_linear_bwd(p, p, p, None, 4, 4, 4, 0.05, 0, p, p, 0, p, 1 << 20, C.byref(t), None) \
            == brl.BRL_EINVAL
        assert L.qat_linear_fwd(p, p, 4, 4, 4, 0.05, None, 0, p, None, None, p, 1 << 20, C.byref(t), None) \
            == brl.BRL_EINVAL
        assert L.grad_l2norm_clip(p, 16, 1.0, 0.0, None, p, 1 << 20, C.byref(t), None) == brl.BRL_EINVAL
        assert brl.workspace_bytes(brl.OP_BWD, 4096, 64, 4096, t) == 0
    assert b"tuning" in L.brl_last_error()
    d = brl.workspace_bytes(brl.OP_BWD, 4096, 64, 4096)
    assert brl.workspace_bytes(brl.OP_BWD, 4096, 64, 4096, brl.Tuning(bwd_chunk_log2=1)) > d
    assert brl.workspace_bytes(brl.OP_BWD, 4096, 64, 4096, brl.Tuning(bwd_chunk_log2=4)) == d
    st = brl.ReduceStateC()
    bufs = (C.c_void_p * 2)(*([0x10000] * 2))
    assert L.brl_reduce_init(C.byref(st), 2, 2, 16, C.cast(bufs, C.c_void_p)) == brl.BRL_OK
    assert (st.tune.bwd_chunk_log2, st.tune.reduce_wg_blocks, st.tune.stream_vec, st.tune.bwd_engine) == (0, 0, 0, 0)
    st.tune.stream_vec = 3
    assert L.ordered_reduce(C.byref(st), p, None, None) == brl.BRL_EINVAL
    assert st.next == 0


def test_library_holds_no_writable_state():
    """The library's own writable symbols are only: the host handles of its
    kernels (registered with the HIP runtime), two constant tables computed
    once on first use (SHA-256 constants from integer roots) with their
    initialisation guards, the host shadow of a read-only device constant,
    the no-alloc norm's device scratch array with its per-device address
    table (set once per device), and the calling thread's last-error message
    (thread-local).  No tuning knob, cache or counter lives between calls."""
    out = subprocess.run(["nm", "-C", "--defined-only", brl.LIB_PATH], capture_output=True, text=True).stdout
    runtime = ("__hip_", "_DYNAMIC", "_GLOBAL_OFFSET_TABLE_", "__dso_handle", "DW.ref.", "__do_init", "__do_fini",
               "__init", "__fini", "completed.", "__TMC_END__", "__bss_start", "_edata", "_end")
    allowed = ("brl::sha_consts()::c", "brl::sha256_host(", "guard variable for brl::", "brl::kNegZero4",
               "brl::g_err", "scratch", "g_scratch_dev")
    ours = []
    for line in out.splitlines():
        parts = line.split(maxsplit=2)
        if len(parts) != 3 or parts[1] not in "bBdDvV":
            continue
        name = parts[2]
        if name.startswith(runtime) or ("_kernel" in name and "(" in name):
            continue
        if not name.startswith(allowed):
            ours.append(name)
    assert ours == [], ours
    tls = subprocess.run(["readelf", "-sW", brl.LIB_PATH], capture_output=True, text=True).stdout
    assert [l.split()[-1] for l in tls.splitlines() if " TLS " in l] == ["_ZN3brlL5g_errE"]


# ---- generated gfx950 code -------------------------------------------------------
FUSED = re.compile(r"v_(fma|fmac|fmamk|fmaak|mad|mac)_f32|v_pk_\w*f32|v_fma_mix|v_mad_mix|v_dot\w*f32")


def test_no_fused_or_packed_fp32_outside_division():
    """Every fp32 multiply-add in the device code sits inside the correctly
    rounded division sequence (between v_div_scale_f32 and v_div_fixup_f32);
    no packed fp32 instruction appears at all."""
    files = brl_build.asm_files()
    assert all(os.path.exists(f) for f in files), "build first"
    bad = {}
    for f in files:
        fn, in_div = None, False
        for line in open(f):
            m = re.match(r"^(_Z\w+):", line)
            if m:
                fn, in_div = m.group(1), False
                continue
            if not line.startswith("\t"):
                continue
            ins = line.strip().split(" ")[0]
            if ins.startswith("v_div_scale_f32"):
                in_div = True
            elif ins.startswith("v_div_fixup_f32"):
                in_div = False
            elif FUSED.match(ins) and not in_div:
                bad.setdefault(fn, []).append(line.strip())
    assert not bad, bad


def test_hot_loops_use_plain_mul_and_add():
    """The backward contraction kernels are made of v_mul_f32 + v_add_f32."""
    text = open([f for f in brl_build.asm_files() if "bwd" in f][0]).read()
    names = sorted(set(re.findall(r"^(_ZN3brl16ste_chunk_kernel\w+):", text, re.M)))
    assert len(names) >= 12, names
    for name in names:
        body = text.split(name + ":")[1].split("s_endpgm")[0]
        n_mul = len(re.findall(r"\tv_mul_f32", body))
        n_add = len(re.findall(r"\tv_add_f32", body))
        assert n_mul >= 512 and n_add >= 480, (name, n_mul, n_add)

def test_forward_preparation_waiters_leave_room_for_producers():
    """fwd_prep_kernel's waiting workgroups (at most 4 per CU, plus the tail)
    must be fewer than the kernel's workgroups a CU holds at once, so the
    workgroups they wait for can always run.  A 256-thread workgroup is one
    wave on each of the 4 SIMDs, so workgroups per CU = the compiler's
    occupancy figure (waves per SIMD); require at least 5."""
    text = open([f for f in brl_build.asm_files() if os.path.basename(f).startswith("fwd")][0]).read()
    body = text.split("_ZN3brl15fwd_prep_kernelENS_8PrepArgsE:")[1]
    m = re.search(r"; Occupancy: (\d+)", body)
    assert m, "no occupancy figure after fwd_prep_kernel"
    assert int(m.group(1)) >= 5, m.group(0)


def test_matrix_core_backward_keeps_products_in_vgprs():
    """The matrix-core backward forms products with the K=1 fp32 MFMA and adds
    them with v_add_f32 straight from VGPRs (no accumulator-register copies,
    no fused add)."""
    text = open([f for f in brl_build.asm_files() if "bwd" in f][0]).read()
    names = sorted(set(re.findall(r"^(_ZN3brl15ste_mfma_kernel\w+):", text, re.M)))
    assert len(names) >= 12, names
    for name in names:
        body = text.split(name + ":")[1].split("s_endpgm")[0]
        assert len(re.findall(r"\tv_mfma_f32_16x16x1_4b_f32", body)) >= 32, name
        assert len(re.findall(r"\tv_add_f32", body)) >= 512, name
        assert "v_accvgpr_read" not in body, name
        assert not re.search(r"\tv_mfma\S* a\[", body), name


def test_state_hash_block_instruction_count_matches_bench():
    """bench.py prices the state hash against the VALU bound of the compiled
    SHA-256 block loop; recount that loop's VALU instructions here (every
    basic block of the leaf kernel's first innermost loop)."""
    import sys
    sys.path.insert(0, ROOT)
    import bench
    text = open([f for f in brl_build.asm_files() if "hash" in f][0]).read()
    body = text.split("_ZN3brl16hash_leaf_kernelILb1EEEvNS_9HashBatchENS_9ShaConstsEPhPl:")[1].split("s_endpgm")[0]
    lines = body.splitlines()
    hdr = next(m.group(1) for m in (re.match(r"\.L(BB\d+_\d+):\s*;\s*=>This Inner Loop Header", l) for l in lines) if m)
    n_valu, n_align, inside = 0, 0, False
    for l in lines:
        m = re.match(r"\.L(BB\d+_\d+):(.*)", l)
        if m:
            inside = m.group(1) == hdr or f"Header={hdr} " in m.group(2) + " "
            continue
        if inside and re.match(r"\s+v_", l):
            n_valu += 1
            n_align += "v_alignbit_b32" in l
    assert n_valu == bench.HASH_VALU_PER_BLOCK, n_valu
    assert n_align == bench.HASH_ALIGNBIT_PER_BLOCK, n_align


def test_adamw_scalars_match_the_oracle():
    """brl_adamw_scalars_for_step (host code of the library) gives the oracle's
    binary32 scalars at warm-up, cosine and end-of-budget points."""
    import oracle
    for step, tokens in [(1, 0.0), (1, 1e6), (3, 1.05e9), (667, 2.1e9), (1000, 3e9), (60000, 2.01e11),
                         (120000, 4e11), (200000, 5e11)]:
        lib_s = brl.adamw_scalars_for_step(step, tokens).as_dict()
        want = oracle.adamw_scalars(step, tokens)
        for k, v in want.items():
            assert lib_s[k] == v, (step, tokens, k, lib_s[k], v)


def test_adamw_rejects_bad_arguments_without_launching():
    L = brl.lib()
    sc = brl.AdamWScalars()
    p = C.c_void_p(0x10000)
    assert L.adamw_step(p, p, p, p, -1, C.byref(sc), 1, None) == brl.BRL_ESHAPE
    assert L.adamw_step(p, p, p, p, 4, None, 1, None) == brl.BRL_EINVAL
    assert L.adamw_step(None, p, p, p, 4, C.byref(sc), 1, None) == brl.BRL_EINVAL
    assert L.adamw_step(C.c_void_p(0x10001), p, p, p, 4, C.byref(sc), 1, None) == brl.BRL_EINVAL
    assert L.brl_adamw_scalars_for_step(0, 1.0, None, C.byref(sc)) == brl.BRL_EINVAL
    assert L.brl_adamw_scalars_for_step(1, float("nan"), None, C.byref(sc)) == brl.BRL_EINVAL


def test_attention_rejects_bad_arguments_without_launching():
    L = brl.lib()
    p = C.c_void_p(0x10000)
    ok = dict(B=1, S=64, Hq=4, Hkv=2, D=128, ldq=512, ldk=256, ldv=256, ldo=512)

    def call(**kw):
        a = {**ok, **kw}
        ws = kw.get("ws", C.c_void_p(0x100000))
        return L.attn_fwd(kw.get("Q", p), p, p, a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["ldq"], a["ldk"],
                          a["ldv"], 0, 0.05, kw.get("O", p), a["ldo"], None, ws, kw.get("ws_bytes", 0), None)

    assert call(D=64) == brl.BRL_ESHAPE
    assert call(Hq=3) == brl.BRL_ESHAPE
    assert call(Hkv=0) == brl.BRL_ESHAPE
    assert call(S=133144) == brl.BRL_ESHAPE
    assert call(ldq=500) == brl.BRL_ESHAPE
    assert call(ldk=258) == brl.BRL_EINVAL
    assert call(Q=None) == brl.BRL_EINVAL
    assert call(O=C.c_void_p(0x10004)) == brl.BRL_EINVAL
    assert call(S=0) == brl.BRL_OK            # nothing to do, nothing launched
    need = L.attn_fwd_workspace_bytes(1, 64, 4, 2, 0)
    assert need >= 64 * 64 * 4 and L.attn_fwd_workspace_bytes(1, 64, 3, 2, 0) == 0
    assert call(ws_bytes=need - 1) == brl.BRL_EWORKSPACE
    assert call(ws=C.c_void_p(0x100010), ws_bytes=need) == brl.BRL_EINVAL     # not 256-byte aligned
    # the workspace holds one slot of 64 x 64 logits per key tile of the longest walk, per workgroup
    # (window 512 from a tile-aligned query block reaches back 511 keys: 9 tiles with its own), then
    # the int8 codes of V, 128 x 64 per key tile and KV head
    codes = 4 * 4 * 64 * 128 * 64
    assert L.attn_fwd_workspace_bytes(4, 4096, 16, 4, 512) == 512 * 9 * 64 * 64 * 4 + codes + 256
    assert L.attn_fwd_workspace_bytes(4, 4096, 16, 4, 0) == 512 * 64 * 64 * 64 * 4 + codes + 256
    assert L.attn_bwd_dq(p, p, p, p, p, p, 1, 64, 4, 2, 64, 512, 256, 256, 512, 0, 0.05, p, None) == brl.BRL_ESHAPE
    assert L.attn_bwd_dq(p, p, p, p, p, None, 1, 64, 4, 2, 128, 512, 256, 256, 512, 0, 0.05, p, None) == brl.BRL_EINVAL
    assert L.attn_bwd_dq(p, p, p, p, C.c_void_p(0x10008), p, 1, 64, 4, 2, 128, 512, 256, 256, 512, 0, 0.05, p,
                         None) == brl.BRL_EINVAL
    def kvcall(D=128, ldg=256, stats=p, dV=p, S=64):
        return L.attn_bwd_dkdv(p, p, p, p, p, stats, 1, S, 4, 2, D, 512, 256, 256, 512, 0, 0.05, p, dV, ldg, None)

    assert kvcall(D=64) == brl.BRL_ESHAPE
    assert kvcall(ldg=128) == brl.BRL_ESHAPE
    assert kvcall(ldg=258) == brl.BRL_EINVAL
    assert kvcall(stats=None) == brl.BRL_EINVAL
    assert kvcall(dV=None) == brl.BRL_EINVAL
    assert kvcall(dV=C.c_void_p(0x10004)) == brl.BRL_EINVAL
    assert kvcall(S=0) == brl.BRL_OK           # nothing to do, nothing launched


def test_noalloc_norm_rejects_before_any_device_call():
    """The no-alloc norm checks its arguments and the length bound of its
    scratch array on the host, before it touches a device."""
    L = brl.lib()
    p = C.c_void_p(0x10000)
    assert L.grad_l2norm_clip_noalloc(p, brl.NOALLOC_NORM_MAX_LEN + 1, 1.0, 0.0, None, None, None) == brl.BRL_ESHAPE
    assert b"scratch" in L.brl_last_error()
    assert L.grad_l2norm_clip_noalloc(p, 16, 0.0, 0.0, None, None, None) == brl.BRL_EINVAL
    assert L.grad_l2norm_clip_noalloc(p, -1, 1.0, 0.0, None, None, None) == brl.BRL_ESHAPE
    t = brl.Tuning(stream_vec=3)
    assert L.grad_l2norm_clip_noalloc(p, 16, 1.0, 0.0, None, C.byref(t), None) == brl.BRL_EINVAL
    # the bound is the longest length whose roots and scalars fit the 2 MiB array
    assert brl.workspace_bytes(brl.OP_NORM, brl.NOALLOC_NORM_MAX_LEN, 0, 0) <= 2 << 20
    assert brl.workspace_bytes(brl.OP_NORM, brl.NOALLOC_NORM_MAX_LEN + 1, 0, 0) > 2 << 20


def test_ctypes_structs_match_the_header(tmp_path):
    """The binding's ctypes mirrors of the ABI structs have the sizes and
    field offsets the C compiler gives the header's definitions (a mismatch
    would corrupt every call that passes one)."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    mirrors = {
        "brl_tuning": brl.Tuning,
        "brl_reduce_state": brl.ReduceStateC,
        "brl_adamw_config": brl.AdamWConfig,
        "brl_adamw_scalars": brl.AdamWScalars,
        "brl_stream_source": brl._StreamSource,
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "brlsq.h"', "int main(void) {"]
    for cname, py in mirrors.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run([cc, "-I", brl_build.INCLUDE, str(src), "-o", str(exe)], check=True, capture_output=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, what, val = line.split()
        got[(cname, what)] = int(val)
    for cname, py in mirrors.items():
        assert got[(cname, "size")] == C.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)
