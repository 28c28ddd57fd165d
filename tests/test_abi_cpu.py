"""The C ABI on the CPU: the library loads, exports every function the header
declares, and rejects every bad argument with the documented status before
any HIP call.  Pointers here are fake and never dereferenced: each call
fails validation first.  The one test that lets a valid call reach HIP runs
only where no GPU is visible, so that the launch itself fails."""

import ctypes

import pytest

from gemm_w4a16_group_amd import binding as B

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4, 5

# fake, distinct, 16-byte aligned addresses (never dereferenced)
Q, S, Z, X, C, WS = (ctypes.c_void_p(0x100000 * (i + 1)) for i in range(6))
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    return B.load_library()


def _gpu_count():
    try:
        import torch
        return torch.cuda.device_count()
    except Exception:
        return 0


def test_exports_every_header_function(lib):
    names = B.header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version(lib):
    assert lib.w4a16_status_string(OK) == b"ok"
    for st in (INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, HIPERR):
        assert lib.w4a16_status_string(st) not in (b"ok", b"unknown status")
    assert lib.w4a16_status_string(99) == b"unknown status"
    assert lib.w4a16_version() >= 100


def _gemm(lib, M=64, N=1, K=256, g=128, q=Q, s=S, z=Z, x=X, c=C, ws=NULL, wsb=0):
    return lib.w4a16_gemm(q, s, z, x, c, M, N, K, g, ws, wsb, NULL)


def test_gemm_dimension_checks(lib):
    assert _gemm(lib, g=64) == UNSUPPORTED
    assert b"group_size" in lib.w4a16_last_error()
    assert _gemm(lib, M=0) == INVALID
    assert _gemm(lib, N=0) == INVALID
    assert _gemm(lib, K=0) == INVALID
    assert _gemm(lib, K=200) == INVALID
    assert _gemm(lib, K=64) == INVALID
    assert _gemm(lib, M=1 << 31) == INVALID
    assert _gemm(lib, N=-3) == INVALID


def test_gemm_pointer_checks(lib):
    assert _gemm(lib, q=NULL) == INVALID
    assert _gemm(lib, c=NULL) == INVALID
    assert _gemm(lib, x=ctypes.c_void_p(0x300008)) == MISALIGNED
    assert _gemm(lib, s=ctypes.c_void_p(0x200002)) == MISALIGNED
    # output overlapping an input
    assert _gemm(lib, c=ctypes.c_void_p(0x100000 + 64)) == INVALID
    assert b"overlap" in lib.w4a16_last_error()


def test_workspace_checks(lib):
    # a narrow plan: it needs a workspace
    M, N, K = 12288, 16, 4096
    need = lib.w4a16_gemm_workspace_size(M, N, K, 128)
    assert need > 0
    big = 0x10000000
    q, s, z, x, c = (ctypes.c_void_p(big * (i + 1)) for i in range(5))
    ws = ctypes.c_void_p(big * 7)
    assert _gemm(lib, M=M, N=N, K=K, q=q, s=s, z=z, x=x, c=c) == WORKSPACE
    assert _gemm(lib, M=M, N=N, K=K, q=q, s=s, z=z, x=x, c=c, ws=ws, wsb=need - 1) == WORKSPACE
    assert _gemm(lib, M=M, N=N, K=K, q=q, s=s, z=z, x=x, c=c,
                 ws=ctypes.c_void_p(big * 7 + 4), wsb=need) == MISALIGNED
    assert _gemm(lib, M=M, N=N, K=K, q=q, s=s, z=z, x=x, c=c, ws=c, wsb=need) == INVALID


def test_plan_checks(lib):
    p = B.Plan()
    assert lib.w4a16_plan_default(12288, 1, 4096, 128, ctypes.byref(p)) == OK
    assert p.kernel == B.KERNEL_SKINNY and p.ncol == 1 and p.splitk == 1
    assert lib.w4a16_plan_default(12288, 4096, 4096, 128, ctypes.byref(p)) == OK
    assert p.kernel == B.KERNEL_TILED
    assert lib.w4a16_plan_default(12288, 1, 4096, 128, None) == INVALID

    def gp(**kw):
        pl = B.Plan.make(**kw)
        return lib.w4a16_gemm_plan(Q, S, Z, X, C, 64, kw.pop("N", 4), 1024, 128,
                                   ctypes.byref(pl), NULL, 0, NULL)
    assert gp(kernel=7, splitk=1) == UNSUPPORTED
    assert gp(kernel=1, ncol=2, rb=1, wm=1, wk=1, splitk=1) == UNSUPPORTED   # ncol != N
    assert gp(kernel=1, ncol=8, rb=1, wm=1, wk=1, splitk=1) == UNSUPPORTED   # ncol != N
    assert gp(kernel=1, ncol=12, rb=1, wm=1, wk=1, splitk=1, N=12) == UNSUPPORTED  # no 12-column kernel
    assert gp(kernel=1, ncol=4, rb=3, wm=1, wk=1, splitk=1) == UNSUPPORTED
    assert gp(kernel=1, ncol=4, rb=1, wm=4, wk=8, splitk=1) == UNSUPPORTED   # 32 waves
    assert gp(kernel=1, ncol=4, rb=1, wm=1, wk=1, splitk=1, N=4) != UNSUPPORTED  # valid plan
    assert gp(kernel=1, ncol=4, rb=1, wm=1, wk=1, splitk=9) == UNSUPPORTED   # > 8 groups
    assert gp(kernel=1, ncol=4, rb=1, wm=1, wk=1, splitk=2) == WORKSPACE
    assert gp(kernel=2, bm=64, bn=64, splitk=1) == UNSUPPORTED
    assert gp(kernel=2, bm=128, bn=64, splitk=9) == UNSUPPORTED             # > 8 groups
    assert gp(kernel=2, bm=128, bn=64, splitk=1, wm=2) == UNSUPPORTED       # 2 x 2 needs bn >= 128
    assert gp(kernel=2, bm=128, bn=128, splitk=1, wm=3) == UNSUPPORTED
    assert gp(kernel=2, bm=96, bn=64, splitk=1, wm=3, pf=2) == WORKSPACE      # three waves of 32 rows
    assert gp(kernel=2, bm=96, bn=128, splitk=1, wm=3) == UNSUPPORTED       # 96 rows: 64 columns only
    assert gp(kernel=2, bm=96, bn=64, splitk=1, wm=4) == UNSUPPORTED
    assert gp(kernel=2, bm=96, bn=64, splitk=1, wm=3, pf=4, xpf=2) == UNSUPPORTED
    assert gp(kernel=2, bm=512, bn=128, splitk=1, wm=8) == WORKSPACE        # valid eight-wave plan
    assert gp(kernel=2, bm=512, bn=128, splitk=1, wm=8, pf=2) == WORKSPACE
    assert gp(kernel=2, bm=256, bn=128, splitk=1, wm=4, pf=2) == WORKSPACE
    assert gp(kernel=2, bm=512, bn=128, splitk=1, wm=4) == UNSUPPORTED      # 512 rows need eight waves
    assert gp(kernel=2, bm=256, bn=128, splitk=1, wm=8) == UNSUPPORTED      # eight waves need 512 rows
    assert gp(kernel=2, bm=512, bn=64, splitk=1, wm=8) == UNSUPPORTED
    assert gp(kernel=2, bm=256, bn=128, splitk=1, wm=2, pf=2) == UNSUPPORTED  # 2 x 2 with a third set
    assert gp(kernel=2, bm=256, bn=128, splitk=1, wm=4, pf=3) == UNSUPPORTED

    # a tile's weight rows must fit 32-bit buffer offsets: bm * K / 2 < 2^31
    def gk(K, **kw):
        pl = B.Plan.make(kernel=2, bn=128, splitk=1, **kw)
        far = [ctypes.c_void_p((1 << 40) * (i + 1)) for i in range(5)]
        st = lib.w4a16_gemm_plan(*far, 64, 4, K, 128, ctypes.byref(pl), NULL, 0, NULL)
        return st, lib.w4a16_last_error()
    st, msg = gk(1 << 23, bm=512, wm=8)
    assert st == UNSUPPORTED and b"2^31" in msg
    assert gk((1 << 23) - 128, bm=512, wm=8)[0] == WORKSPACE
    assert gk(1 << 24, bm=256, wm=4)[0] == UNSUPPORTED
    assert gk((1 << 24) - 128, bm=256, wm=4)[0] == WORKSPACE
    assert gp(kernel=3, ncol=16, pf=8, splitk=1, rb=2) == WORKSPACE        # valid narrow plan
    assert gp(kernel=3, ncol=8, pf=8, splitk=1, rb=2) == UNSUPPORTED       # 16, 32 or 64 columns
    assert gp(kernel=3, ncol=16, pf=2, splitk=1, rb=2) == UNSUPPORTED      # ring of 4, 8 or 16
    assert gp(kernel=3, ncol=16, pf=8, splitk=1, rb=3) == UNSUPPORTED
    assert gp(kernel=3, ncol=16, pf=8, splitk=1, rb=2, wk=3) == UNSUPPORTED
    assert gp(kernel=3, ncol=16, pf=8, splitk=3, rb=2, wk=4) == UNSUPPORTED  # 12 > 8 groups
    assert gp(kernel=3, ncol=16, pf=8, splitk=2, rb=2, wk=4) == WORKSPACE
    assert gp(kernel=3, ncol=16, pf=8, splitk=9, rb=2) == UNSUPPORTED      # > 8 groups
    assert gp(kernel=3, ncol=16, pf=8, splitk=1, rb=2, N=17) == UNSUPPORTED  # N > ncol
    assert lib.w4a16_gemm_plan(Q, S, Z, X, C, 64, 4, 1024, 128, None, NULL, 0, NULL) == INVALID
    bad = B.Plan.make(kernel=2, bm=64, bn=64, splitk=1)
    assert lib.w4a16_workspace_size_plan(64, 4, 1024, 128, ctypes.byref(bad)) == 0


def test_default_plans_are_valid(lib):
    shapes = [(4096, 4096), (12288, 4096), (22016, 4096), (4096, 11008), (1, 128), (17, 384),
              (5, 32768)]
    for (M, K) in shapes:
        for N in (1, 2, 3, 4, 8, 16, 17, 32, 33, 64, 65, 128, 256, 1000, 4096):
            p = B.Plan()
            assert lib.w4a16_plan_default(M, N, K, 128, ctypes.byref(p)) == OK
            ws = lib.w4a16_workspace_size_plan(M, N, K, 128, ctypes.byref(p))
            assert ws == lib.w4a16_gemm_workspace_size(M, N, K, 128)
            needs = p.kernel in (2, 3) or p.splitk > 1
            assert (ws == 0) == (not needs), (M, N, K, p.as_dict())
            if p.kernel in (2, 3):
                # x is read in place for N a multiple of 8 (no chunk area)
                assert ws >= 65536 + (K * N * 2 if N % 8 else 0)
            # a valid plan passes every check: with fake pointers the call
            # then fails only on the workspace (if any), never on the plan
            far = [ctypes.c_void_p((1 << 40) * (i + 1)) for i in range(5)]
            st = lib.w4a16_gemm_plan(*far, M, N, K, 128, ctypes.byref(p), NULL, 0, NULL) \
                if ws else None
            if ws:
                assert st == WORKSPACE, (M, N, K, p.as_dict(), lib.w4a16_last_error())


def test_default_split_fills_the_cus(lib):
    # 64-column tiles are split along K up to 256 workgroups while every
    # split keeps 8 groups of 128 k
    def plan(M, N, K):
        p = B.Plan()
        assert lib.w4a16_plan_default(M, N, K, 128, ctypes.byref(p)) == OK
        return p
    p = plan(4096, 64, 11008)           # 32 tiles, 86 groups
    assert (p.kernel, p.bm, p.bn, p.splitk) == (2, 128, 64, 8)
    p = plan(4096, 128, 4096)           # 64 tiles, 32 groups
    assert (p.kernel, p.bm, p.bn, p.splitk) == (2, 128, 64, 4)
    p = plan(2048, 128, 4096)           # 32 tiles: 8 groups per split stops it at 4
    assert (p.kernel, p.bm, p.bn, p.splitk) == (2, 128, 64, 4)
    p = plan(12288, 64, 4096)           # 96-row tiles, two splits
    assert (p.kernel, p.bm, p.wm, p.splitk) == (2, 96, 3, 2)


def test_gemv_checks(lib):
    assert lib.w4a16_gemv(Q, S, Z, X, C, 64, 256, 32, NULL) == UNSUPPORTED
    assert lib.w4a16_gemv(Q, S, Z, NULL, C, 64, 256, 128, NULL) == INVALID
    assert lib.w4a16_gemv(Q, S, Z, X, ctypes.c_void_p(0x500004), 64, 256, 128, NULL) == MISALIGNED


def test_pack_checks(lib):
    P1, P2 = ctypes.c_void_p(0x700000), ctypes.c_void_p(0x800000)
    assert lib.w4a16_pack(NULL, NULL, 4, 256, 128, P1, P2, NULL) == INVALID
    assert lib.w4a16_pack(Q, NULL, 4, 256, 128, NULL, NULL, NULL) == INVALID
    assert lib.w4a16_pack(Q, Z, 4, 256, 64, P1, P2, NULL) == UNSUPPORTED
    assert lib.w4a16_pack(Q, Z, 4, 200, 128, P1, P2, NULL) == INVALID
    assert lib.w4a16_pack(ctypes.c_void_p(0x100001), NULL, 4, 256, 128, P1, NULL, NULL) == MISALIGNED
    assert lib.w4a16_pack(Q, NULL, 4, 256, 128, Q, NULL, NULL) == INVALID   # output overlaps input


@pytest.mark.skipif(_gpu_count() != 0, reason="needs a machine with no GPU: the launch must fail")
def test_valid_call_without_gpu_reports_hip_error(lib):
    st = _gemm(lib)
    assert st == HIPERR
    assert len(lib.w4a16_last_error()) > 0


def test_kernel_name_follows_the_plan(lib):
    # eight waves along K, four groups each: four weight groups in flight per wave
    assert B.kernel_name(12288, 1, 4096) == "skinny_kernel<1, 4>"
    assert B.kernel_name(4096, 1, 11008) == "skinny_kernel<1, 8>"
    # 512-row tiles where they load the 256 CUs as evenly as 256-row tiles
    # (768 = 3 x 256 tiles at N = 4096, 192 at N = 1024), not at N = 2048
    assert B.kernel_name(12288, 4096, 4096) == "tiled_dx_kernel<512, 128, 8, 8, 2, 1>"
    assert B.kernel_name(12288, 1024, 4096) == "tiled_dx_kernel<512, 128, 8, 8, 2, 1>"
    assert B.kernel_name(12288, 2048, 4096) == "tiled_dx_kernel<256, 128, 4, 4, 1, 1>"
    assert B.kernel_name(12288, 512, 4096) == "tiled_dx_kernel<128, 128, 4, 4, 1, 1>"
    # 96-row tiles of three waves where 128-row ones leave CUs idle; the
    # few-column tiles read [K, N] activations in place (the _dx kernels)
    # when N is a multiple of 8, else through xpack_col_kernel
    assert B.kernel_name(12288, 64, 4096) == "tiled_dx_kernel<96, 64, 3, 3, 2, 1>"
    assert B.kernel_name(12288, 60, 4096) == "tiled_kernel<96, 64, 3, 3, 2, 1>"
    assert B.kernel_name(11008, 128, 4096) == "tiled_dx_kernel<96, 64, 3, 3, 2, 1>"
    assert B.kernel_name(4096, 64, 11008) == "tiled_dx_kernel<128, 64, 4, 4, 2, 1>"
    # two K slices of 128 x 128 tiles from 160 tiles on (22016 rows, N = 128),
    # never at N <= 64 (half of each tile would be empty)
    assert B.kernel_name(22016, 128, 4096) == "tiled_k2_dx_kernel<128, 128, 4, 4, 1, 1>"
    assert B.kernel_name(22016, 64, 4096) == "tiled_dx_kernel<96, 64, 3, 3, 2, 1>"
    assert B.kernel_name(24576, 64, 4096) != "tiled_k2_dx_kernel<128, 128, 4, 4, 1, 1>"
    # long K below N = 1024: 128-column tiles split along K
    assert B.kernel_name(4096, 384, 11008) == "tiled_dx_kernel<128, 128, 4, 4, 2, 1>"
    assert B.kernel_name(4096, 384, 4096) == "tiled_dx_kernel<128, 64, 4, 4, 2, 1>"
    p = B.Plan.make(kernel=2, bm=128, bn=256, splitk=1, wm=2)
    assert B.kernel_name(300, 300, 1024, p) == "tiled_kernel<128, 256, 2, 4, 1, 1>"
    # narrow plans read [K, N] activations in place when N is a multiple of 8
    # (last template argument true) and re-laid by xpack_col_kernel otherwise
    assert B.kernel_name(12288, 16, 4096) == "narrow_kernel<1, 4, 1, 1, 4, true>"
    assert B.kernel_name(12288, 8, 4096) == "narrow_kernel<1, 4, 1, 1, 4, true>"
    assert B.kernel_name(12288, 12, 4096) == "narrow_kernel<1, 4, 1, 1, 4, false>"
    # 32 staged columns: 128-row workgroups where 64-row tiles times the
    # smallest split reach 256 (96-row ones of three waves where those fit
    # one per CU), 64-row ones otherwise
    assert B.kernel_name(12288, 32, 4096) == "narrow_kernel<2, 4, 2, 1, 3, true>"
    assert B.kernel_name(4096, 24, 11008) == "narrow_kernel<2, 4, 2, 1, 4, true>"
    assert B.kernel_name(4096, 32, 4096) == "narrow_kernel<2, 4, 1, 1, 4, true>"
    assert B.kernel_name(22016, 32, 4096) == "narrow_kernel<2, 4, 2, 1, 4, true>"
    # 128-row workgroups when 64-row tiles outnumber the CUs; one wave along
    # K; the skinny kernel for N = 8 on a small matrix
    assert B.kernel_name(22016, 16, 4096) == "narrow_kernel<1, 4, 2, 1, 3, true>"
    assert B.kernel_name(4096, 8, 11008) == "narrow_kernel<1, 4, 1, 1, 4, true>"
    assert B.kernel_name(4096, 8, 4096) == "skinny_kernel<8, 4>"
    assert B.kernel_name(4096, 16, 4096) == "skinny_kernel<16, 4>"
    buf = ctypes.create_string_buffer(8)
    assert lib.w4a16_kernel_name(64, 1, 1024, 128, None, None, 8) == INVALID
    assert lib.w4a16_kernel_name(64, 1, 1000, 128, None, buf, 8) == INVALID      # K % 128
    assert lib.w4a16_kernel_name(64, 1, 1024, 128, None, buf, 8) == OK           # truncated
    assert buf.value == b"skinny_"


def test_quantize_argument_checks(lib):
    w, q, s, z = (ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(4))
    assert lib.w4a16_quantize(w, 64, 1024, 64, q, s, z, NULL) == UNSUPPORTED     # group size
    assert lib.w4a16_quantize(w, 64, 1000, 128, q, s, z, NULL) == INVALID       # K % 128
    assert lib.w4a16_quantize(NULL, 64, 1024, 128, q, s, z, NULL) == INVALID
    assert lib.w4a16_quantize(w, 64, 1024, 128, ctypes.c_void_p(0x20000008), s, z, NULL) == MISALIGNED
    # packed codes on top of the input
    assert lib.w4a16_quantize(w, 64, 1024, 128, ctypes.c_void_p(0x10000000 + 4096), s, z, NULL) == INVALID
    assert b"overlap" in lib.w4a16_last_error()


def test_token_layout_plans_and_checks(lib):
    def plan_ex(M, N, K, layout):
        p = B.Plan()
        st = lib.w4a16_plan_default_ex(M, N, K, 128, layout, ctypes.byref(p))
        return st, p

    # N = 1: both layouts are the same memory and take the same plan
    for M, K in ((4096, 4096), (12288, 4096), (100, 256)):
        st, p = plan_ex(M, 1, K, B.LAYOUT_TOKEN)
        assert st == OK
        q = B.Plan()
        assert lib.w4a16_plan_default(M, 1, K, 128, ctypes.byref(q)) == OK
        assert p.as_dict() == q.as_dict()
    # the skinny kernel only up to N = 8; the chunk-staging kernels need a
    # workspace for the rewritten activations
    for N in (2, 5, 7, 8, 16, 17, 32, 33, 64, 200, 4096):
        for M, K in ((4096, 4096), (11008, 4096), (4096, 11008), (96, 128), (96, 1152)):
            st, p = plan_ex(M, N, K, B.LAYOUT_TOKEN)
            assert st == OK, (M, N, K)
            need = lib.w4a16_workspace_size_ex(M, N, K, 128, B.LAYOUT_TOKEN, ctypes.byref(p))
            assert lib.w4a16_workspace_size_ex(M, N, K, 128, B.LAYOUT_TOKEN, None) == need
            if N > 8:
                assert p.kernel in (B.KERNEL_NARROW, B.KERNEL_TILED), (M, N, K, p.as_dict())
            if p.kernel != B.KERNEL_SKINNY:
                assert need >= K * N * 2
    # the default of the KN layout through the _ex calls equals the plain calls
    for M, N, K in ((4096, 3, 4096), (4096, 16, 4096), (4096, 4096, 4096)):
        st, p = plan_ex(M, N, K, B.LAYOUT_KN)
        q = B.Plan()
        assert st == OK and lib.w4a16_plan_default(M, N, K, 128, ctypes.byref(q)) == OK
        assert p.as_dict() == q.as_dict()
        assert (lib.w4a16_workspace_size_ex(M, N, K, 128, B.LAYOUT_KN, None)
                == lib.w4a16_gemm_workspace_size(M, N, K, 128))
    # unknown layout
    assert plan_ex(64, 4, 256, 2)[0] == INVALID
    assert b"layout" in lib.w4a16_last_error()
    assert lib.w4a16_workspace_size_ex(64, 4, 256, 128, -1, None) == 0
    assert lib.w4a16_gemm_ex(Q, S, Z, X, C, 64, 4, 256, 128, 7, None, NULL, 0, NULL) == INVALID
    # a 16-column skinny plan under the token layout is refused
    sk = B.Plan.make(kernel=B.KERNEL_SKINNY, ncol=16, rb=1, wm=1, wk=4, splitk=1)
    assert lib.w4a16_workspace_size_plan(64, 16, 1152, 128, ctypes.byref(sk)) == 0   # valid, no workspace
    assert lib.w4a16_kernel_name(64, 16, 1152, 128, ctypes.byref(sk), ctypes.create_string_buffer(64), 64) == OK
    assert (lib.w4a16_gemm_ex(Q, S, Z, X, C, 64, 16, 1152, 128, B.LAYOUT_TOKEN, ctypes.byref(sk), NULL, 0, NULL)
            == UNSUPPORTED)
    assert b"token-major" in lib.w4a16_last_error()
    assert lib.w4a16_workspace_size_ex(64, 16, 1152, 128, B.LAYOUT_TOKEN, ctypes.byref(sk)) == 0
    # token layout on a chunk-staging plan, no workspace
    nr = B.Plan.make(kernel=B.KERNEL_NARROW, ncol=16, pf=8, splitk=1, rb=1, wk=1)
    assert (lib.w4a16_gemm_ex(Q, S, Z, X, C, 64, 4, 256, 128, B.LAYOUT_TOKEN, ctypes.byref(nr), NULL, 0, NULL)
            == WORKSPACE)
    # dimension and pointer checks are the same as w4a16_gemm's
    assert lib.w4a16_gemm_ex(Q, S, Z, X, C, 64, 0, 256, 128, B.LAYOUT_TOKEN, None, NULL, 0, NULL) == INVALID
    assert lib.w4a16_gemm_ex(NULL, S, Z, X, C, 64, 1, 256, 128, B.LAYOUT_TOKEN, None, NULL, 0, NULL) == INVALID
    assert (lib.w4a16_gemm_ex(Q, S, Z, ctypes.c_void_p(0x400008), C, 64, 1, 256, 128, B.LAYOUT_TOKEN, None,
                              NULL, 0, NULL) == MISALIGNED)


def test_add_rmsnorm_checks(lib):
    R, G_, H, Y = (ctypes.c_void_p(0x1000000 * (i + 1)) for i in range(4))
    f = lib.w4a16_add_rmsnorm
    # dimensions, eps, pointers, alignment
    assert f(X, R, G_, 1e-6, H, Y, 0, 4096, NULL) == INVALID
    assert f(X, R, G_, 1e-6, H, Y, 2, 4, NULL) == INVALID
    assert f(X, R, G_, 1e-6, H, Y, 2, 4100, NULL) == INVALID
    assert f(X, R, G_, -1.0, H, Y, 2, 4096, NULL) == INVALID
    assert f(X, R, G_, float("nan"), H, Y, 2, 4096, NULL) == INVALID
    assert f(X, R, G_, float("inf"), H, Y, 2, 4096, NULL) == INVALID
    assert b"eps" in lib.w4a16_last_error()
    assert f(X, R, NULL, 1e-6, H, Y, 2, 4096, NULL) == INVALID
    assert f(X, R, G_, 1e-6, ctypes.c_void_p(0x2000008), Y, 2, 4096, NULL) == MISALIGNED
    # y overlapping an input; h partially overlapping the residual
    assert f(X, R, G_, 1e-6, H, ctypes.c_void_p(0x1000000 + 4096), 2, 4096, NULL) == INVALID
    assert f(X, R, G_, 1e-6, ctypes.c_void_p(0x1000000 + 16), Y, 2, 4096, NULL) == INVALID
    assert b"h overlaps" in lib.w4a16_last_error()
    assert f(X, R, G_, 1e-6, X, Y, 2, 4096, NULL) == INVALID


def test_gemm_add_rmsnorm_checks(lib):
    R, G_, H = (ctypes.c_void_p(0x10000000 * (i + 8)) for i in range(3))
    q, s, z, x, c = (ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(5))
    ws = ctypes.c_void_p(0x10000000 * 12)
    M, N, K = 4096, 16, 4096

    def call(eps=1e-6, h=H, cc=c, wsp=ws, wsb=1 << 26, plan=None, n=N):
        return lib.w4a16_gemm_add_rmsnorm(q, s, z, x, R, G_, eps, h, cc, M, n, K, 128, plan, wsp, wsb, NULL)

    for n in (1, 3, 8, 16, 32, 100, 4096):
        need = lib.w4a16_gemm_add_rmsnorm_workspace_size(M, n, K, 128, None)
        assert need >= K * n * 2, n    # the normalized rows always live in the workspace
    need = lib.w4a16_gemm_add_rmsnorm_workspace_size(M, N, K, 128, None)
    assert call(wsp=NULL, wsb=0) == WORKSPACE
    assert call(wsb=need - 1) == WORKSPACE
    assert call(eps=-1e-3) == INVALID
    assert call(h=NULL) == INVALID
    assert call(h=ctypes.c_void_p(0x10000000 * 8 + 16)) == INVALID      # partial overlap of the residual
    assert call(h=x) == INVALID
    assert call(cc=ctypes.c_void_p(0x10000000 * 9 + 64)) == INVALID     # c over gamma
    assert call(wsp=ctypes.c_void_p(0x10000000 * 10 - 4096)) == INVALID  # workspace runs into h
    sk = B.Plan.make(kernel=B.KERNEL_SKINNY, ncol=16, rb=1, wm=1, wk=4, splitk=1)
    assert call(plan=ctypes.byref(sk)) == UNSUPPORTED                    # token-major skinny needs N <= 8
    assert lib.w4a16_gemm_add_rmsnorm_workspace_size(M, N, K, 128, ctypes.byref(sk)) == 0
    assert lib.w4a16_gemm_add_rmsnorm_workspace_size(M, N, K, 64, None) == 0


def test_decode_attention_checks(lib):
    qkv, kc, vc, pos, out = (ctypes.c_void_p(0x10000000 * (i + 1)) for i in range(5))
    ws = ctypes.c_void_p(0x10000000 * 9)

    def call(B=1, H=32, D=128, S=2048, L=2048, base=10000.0, scale=0.088, o=out, k=kc, p=pos, w=ws, wb=1 << 24):
        return lib.w4a16_decode_attention(qkv, k, vc, p, o, B, H, D, S, L, base, scale, w, wb, NULL)

    assert call(D=64) == UNSUPPORTED
    assert call(S=300000, L=300000) == UNSUPPORTED   # more than 1024 splits along the keys
    assert call(B=0) == INVALID
    assert call(H=70000) == INVALID
    assert call(L=4096) == INVALID           # max_len above the capacity
    assert call(L=0) == INVALID
    assert call(base=0.0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(o=NULL) == INVALID
    assert call(p=ctypes.c_void_p(0x40000002)) == MISALIGNED
    assert call(o=ctypes.c_void_p(0x10000000 * 2 + 256)) == INVALID   # out inside the key cache
    assert call(k=ctypes.c_void_p(0x10000000 * 3 - 4096)) == INVALID  # key cache runs into the value cache
    need = lib.w4a16_decode_attention_workspace_size(1, 32, 128, 2048, 2048)
    assert need > 0                          # one sequence: split along the keys
    assert call(w=NULL, wb=0) == WORKSPACE
    assert call(wb=need - 1) == WORKSPACE
    # many sequences fill the chip without a split: no workspace
    assert lib.w4a16_decode_attention_workspace_size(64, 32, 128, 64, 64) == 0
    assert lib.w4a16_decode_attention_workspace_size(1, 32, 64, 2048, 2048) == 0   # unsupported D


def test_tune_checks(lib):
    best = B.Plan()
    us = ctypes.c_float()
    n = ctypes.c_int32()

    def call(iters=5, bp=ctypes.byref(best), layout=0, flush=NULL, fb=0, g=128):
        return lib.w4a16_tune(Q, S, Z, X, C, 64, 4, 256, g, layout, WS, 1 << 20, flush, fb, iters, bp,
                              ctypes.byref(us), ctypes.byref(n), NULL)

    assert call(iters=0) == INVALID
    assert call(bp=None) == INVALID
    assert call(layout=5) == INVALID
    assert call(g=64) == UNSUPPORTED
    assert call(flush=ctypes.c_void_p(0x700008), fb=4096) == INVALID
    assert call(flush=ctypes.c_void_p(0x700000), fb=0) == INVALID


def test_every_export_is_declared():
    """The library exports no w4a16_ function that the header does not declare."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", B.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted({ln.split()[-1] for ln in out.splitlines() if ln.split() and ln.split()[-1].startswith("w4a16_")})
    assert exported == B.header_functions()


def test_decode_layer_and_silu_checks(lib):
    assert lib.w4a16_silu_mul(X, C, 0, 64, NULL) == INVALID
    assert lib.w4a16_silu_mul(X, C, 4, 12, NULL) == INVALID
    assert lib.w4a16_silu_mul(X, ctypes.c_void_p(0x400008), 4, 64, NULL) == MISALIGNED
    assert lib.w4a16_silu_mul(X, ctypes.c_void_p(0x400000 + 64), 4, 64, NULL) == INVALID   # act inside gu
    # workspace sizes: valid shapes give a size, invalid ones 0
    assert lib.w4a16_decode_layer_workspace_size(1, 32, 128, 11008, 2048, 2048) > 0
    assert lib.w4a16_decode_layer_workspace_size(1, 32, 128, 11000, 2048, 2048) == 0   # I % 128
    assert lib.w4a16_decode_layer_workspace_size(1, 32, 64, 11008, 2048, 2048) == 0    # D
    layer = B.DecoderLayer()
    assert lib.w4a16_decode_layer(None, 1, 4, 128, 1024, 64, 64, X, 1e-6, 1e4, Q, S, WS, 1 << 30, NULL) == INVALID
    # a layer of null pointers fails its first step's checks before anything is enqueued
    need = lib.w4a16_decode_layer_workspace_size(1, 4, 128, 1024, 64, 64)
    assert (lib.w4a16_decode_layer(ctypes.byref(layer), 1, 4, 128, 1024, 64, 64, X, 1e-6, 1e4, Q, S, WS, need, NULL)
            == INVALID)
    assert (lib.w4a16_decode_layer(ctypes.byref(layer), 1, 4, 128, 1024, 64, 64, X, 1e-6, 1e4, Q, S, WS, need - 1,
                                   NULL) == WORKSPACE)


def test_gemm_silu_checks(lib):
    # output over the gate/up input's second half (gu is N x 2K)
    M, N, K = 64, 2, 256
    assert lib.w4a16_gemm_silu(Q, S, Z, X, ctypes.c_void_p(0x400000 + N * K * 2), M, N, K, 128, None, WS, 1 << 20,
                               NULL) == INVALID
    assert lib.w4a16_gemm_silu(Q, S, Z, X, C, M, N, K, 64, None, WS, 1 << 20, NULL) == UNSUPPORTED
    assert lib.w4a16_gemm_silu(NULL, S, Z, X, C, M, N, K, 128, None, WS, 1 << 20, NULL) == INVALID
    sk = B.Plan.make(kernel=B.KERNEL_SKINNY, ncol=16, rb=1, wm=1, wk=4, splitk=1)
    assert lib.w4a16_gemm_silu(Q, S, Z, X, C, M, 16, 1152, 128, ctypes.byref(sk), WS, 1 << 20, NULL) == UNSUPPORTED


def test_stream_read_probe_checks(lib):
    assert lib.w4a16_stream_read_sink_words(4096, 8, 4) == 8
    assert lib.w4a16_stream_read_sink_words(26181632, 8, 4) == 6392
    assert lib.w4a16_stream_read_sink_words(26181632, 4, 16) == 1600
    assert lib.w4a16_stream_read_sink_words(4100, 8, 4) == 0
    assert lib.w4a16_stream_read_sink_words(4096, 3, 4) == 0
    assert lib.w4a16_stream_read_sink_words(4096, 8, 3) == 0
    assert lib.w4a16_stream_read(NULL, 4096, C, 8, 4, NULL) == INVALID
    assert lib.w4a16_stream_read(Q, 4096, NULL, 8, 4, NULL) == INVALID
    assert lib.w4a16_stream_read(Q, 4100, C, 8, 4, NULL) == INVALID
    assert lib.w4a16_stream_read(Q, 0, C, 8, 4, NULL) == INVALID
    assert lib.w4a16_stream_read(Q, 4096, C, 3, 4, NULL) == INVALID
    assert lib.w4a16_stream_read(Q, 4096, C, 8, 32, NULL) == INVALID
    assert lib.w4a16_stream_read(ctypes.c_void_p(0x100008), 4096, C, 8, 4, NULL) == MISALIGNED
    assert lib.w4a16_stream_read(Q, 4096, ctypes.c_void_p(0x100000 + 64), 8, 4, NULL) == INVALID
    assert b"overlap" in lib.w4a16_last_error()
