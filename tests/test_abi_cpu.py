"""The C-ABI library loads, exports every function include/moe.h declares, and
rejects bad arguments on the host before anything is enqueued (no GPU needed:
every call here fails validation, so no HIP call is made)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")
LIB = os.path.join(ROOT, "mixture_experts_transformer_amd", "libmoe.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from mixture_experts_transformer_amd import build as B
        B.build()
    return C.CDLL(LIB)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["moe_route", "moe_permute", "moe_grouped_ffn", "moe_combine", "moe_layer_fwd"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings(lib):
    lib.moe_status_str.restype = C.c_char_p
    assert lib.moe_status_str(0) == b"ok"
    assert lib.moe_status_str(5) == b"workspace too small"
    assert lib.moe_abi_version() == 2


def _route(lib, T=4, d=32, E=8, k=2, h=1, W=1, ids=1, w=1, hdt=0):
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    lib.moe_route.argtypes = [vp, C.c_int, i64, i64, vp, C.c_float, i32, vp, vp, i32, i32, vp,
                              C.c_int, vp, vp, vp, vp]
    p = lambda x: None if not x else 4096 * x
    return lib.moe_route(p(h), hdt, T, d, None, 1e-5, 0, p(W), None, E, k, None, 0, None,
                         p(ids), p(w), None)


def test_route_rejects_bad_arguments(lib):
    assert _route(lib, k=9) == 2          # k > E
    assert _route(lib, E=513) == 2        # E above the limit
    assert _route(lib, k=17, E=64) == 2   # k above 16
    assert _route(lib, d=24) == 2         # d_r not a multiple of 16
    assert _route(lib, d=16) == 2         # d_r below 32
    assert _route(lib, h=0) == 1          # null input
    assert _route(lib, hdt=7) == 3        # bad dtype
    assert _route(lib, T=0, h=0, W=0, ids=0, w=0) == 0   # nothing to do


def test_permute_rejects_bad_arguments(lib):
    vp, i64, i32 = C.c_void_p, C.c_int64, C.c_int32
    lib.moe_permute.argtypes = [vp, i64, i32, i64, vp, C.c_int, i64, i32, vp, i64, vp, vp, vp, vp,
                                vp, vp, C.c_size_t, vp]
    lib.moe_permute_workspace_size.restype = C.c_size_t
    lib.moe_permute_workspace_size.argtypes = [i64, i32]
    a = 4096
    need = lib.moe_permute_workspace_size(1000, 16)
    assert need > 0
    call = lambda **kw: lib.moe_permute(
        kw.get("ids", a), kw.get("n", 1000), kw.get("E", 16), kw.get("cap", -1), kw.get("src"),
        1, kw.get("width", 0), 1, kw.get("dst"), kw.get("R", 1000), a, a, a, a, a,
        kw.get("ws", a), kw.get("wsb", need), None)
    assert call(E=0) == 2
    assert call(E=1025) == 2
    assert call(R=999) == 2                # fewer rows than could be kept
    assert call(wsb=need - 1) == 5         # workspace too small
    assert call(ws=0) == 5
    assert call(src=a) == 1                # src without dst
    assert call(src=a, dst=a, width=12) == 2   # row not a multiple of 16 bytes
    assert call(ids=4100) == 4             # misaligned


def test_layer_rejects_bad_descriptors(lib):
    import mixture_experts_transformer_amd.moe as B
    d = B.layer_desc(64, 128, 64, 8, 2, 64, 1, 64, "bf16")
    W = B.LayerWeights(4096, 0, 4096, 0, 4096, 4096, 4096, 4096, 4096)
    call = lambda desc, W=W, ws=4096, wsb=1 << 30: B._lib.moe_layer_fwd(
        C.byref(desc), C.byref(W), 4096, 8192, None, ws, wsb, None)
    bad = B.layer_desc(64, 128, 64, 8, 9, 64, 1, 64, "bf16")       # k > E
    assert call(bad) == 2
    bad = B.layer_desc(64, 100, 64, 8, 2, 64, 1, 64, "bf16")       # D not a multiple of 32
    assert call(bad) == 2
    bad = B.layer_desc(64, 128, 64, 8, 2, 96, 1, 64, "bf16")       # bf16 H: 192-byte rows
    assert call(bad) == 2
    ok_f32 = B.layer_desc(64, 128, 64, 8, 2, 96, 1, 64, "f32")     # f32 H = 96: 384 bytes
    assert call(ok_f32, ws=4096, wsb=16) == 5                       # passes the shape checks
    big = B.layer_desc(1 << 20, 4096, 2048, 8, 2, 64, 1, 64, "bf16")   # [T, L] input of 4 GiB
    assert call(big) == 2
    bad = B.layer_desc(64, 128, 64, 8, 2, 64, 4, 64, "bf16")       # too many shared experts
    assert call(bad) == 2
    assert call(d, wsb=16) == 5                                    # workspace too small
    W2 = B.LayerWeights(0, 0, 4096, 0, 4096, 4096, 4096, 4096, 4096)   # latent without W_dn
    assert call(d, W=W2) == 1
    need = B.moe_layer_workspace_size(d)
    assert need > 64 * 2 * 64 * 2


def test_backward_entry_points_reject_bad_arguments(lib):
    vp, i64, i32, sz = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t
    lib.moe_ragged_dot_dlhs.argtypes = [vp, vp, i32, i64, vp, i64, i64, C.c_int, vp, vp, sz, vp]
    lib.moe_ragged_dot_dlhs_workspace_size.restype = sz
    lib.moe_ragged_dot_dlhs_workspace_size.argtypes = [i32]
    lib.moe_ragged_dot_drhs.argtypes = [vp, vp, vp, i32, i64, i64, i64, C.c_int, vp, C.c_int, vp, sz,
                                        vp]
    lib.moe_ragged_dot_drhs_workspace_size.restype = sz
    lib.moe_ragged_dot_drhs_workspace_size.argtypes = [i32]
    lib.moe_grouped_ffn_bwd.argtypes = [vp, vp, vp, i32, i64, vp, vp, i64, i64, C.c_int, vp, vp, vp,
                                        C.c_int, vp, sz, vp]
    lib.moe_grouped_ffn_bwd_workspace_size.restype = sz
    lib.moe_grouped_ffn_bwd_workspace_size.argtypes = [i32, i64, i64, C.c_int]
    a = 4096
    need = lib.moe_ragged_dot_dlhs_workspace_size(8)
    assert need >= 9 * 4
    dlhs = lambda **kw: lib.moe_ragged_dot_dlhs(
        a, kw.get("off", a), kw.get("E", 8), 1000, kw.get("W", a), kw.get("N", 128),
        kw.get("K", 64), kw.get("dt", 1), a, kw.get("ws", a), kw.get("wsb", need), None)
    assert dlhs(E=0) == 2
    assert dlhs(N=100) == 2                 # not whole 128-byte steps
    assert dlhs(dt=7) == 3
    assert dlhs(W=0) == 1
    assert dlhs(off=a + 4) == 4             # misaligned
    assert dlhs(wsb=need - 1) == 5
    dneed = lib.moe_ragged_dot_drhs_workspace_size(8)
    assert dneed >= 9 * 8
    drhs = lambda **kw: lib.moe_ragged_dot_drhs(
        a, a, a, kw.get("E", 8), 1000, kw.get("N", 128), kw.get("K", 64), kw.get("dt", 1),
        kw.get("dW", a), kw.get("dw", 0), a, kw.get("wsb", dneed), None)
    assert drhs(wsb=dneed - 1) == 5
    assert drhs(K=96) == 2                  # bf16 rows of 192 bytes
    assert drhs(dt=0, dw=1) == 3            # float32 inputs, bfloat16 weight gradient
    assert drhs(dW=0) == 1
    assert drhs(E=1025) == 2
    wneed = lib.moe_grouped_ffn_bwd_workspace_size(8, 1000, 64, 1)
    assert wneed > 1000 * 64 * 2 * 5
    ffn = lambda **kw: lib.moe_grouped_ffn_bwd(
        a, a, a, 8, 1000, a, a, kw.get("d", 128), 64, 1, a, kw.get("dWgu", a), a, kw.get("dw", 0),
        a, kw.get("wsb", wneed), None)
    assert ffn(d=96) == 2
    assert ffn(dWgu=0) == 1
    assert ffn(dw=5) == 3
    assert ffn(wsb=wneed - 1) == 5


def test_forward_ragged_dot_and_fp8_entry_points_reject_bad_arguments(lib):
    vp, i64, i32, sz, f32 = C.c_void_p, C.c_int64, C.c_int32, C.c_size_t, C.c_float
    lib.moe_ragged_dot_workspace_size.restype = sz
    lib.moe_ragged_dot_workspace_size.argtypes = [i32]
    lib.moe_ragged_dot.argtypes = [vp, vp, i32, i64, vp, i64, i64, C.c_int, vp, C.c_int, vp, sz,
                                   vp]
    lib.moe_ragged_dot_e4m3.argtypes = [vp, vp, i32, i64, vp, i64, i64, vp, vp, vp, C.c_int, vp,
                                        sz, vp]
    lib.moe_quantize_e4m3.argtypes = [vp, C.c_int, i64, vp, vp, vp, vp]
    lib.moe_swiglu_quantize_e4m3.argtypes = [vp, C.c_int, vp, i32, i64, i64, vp, vp, vp, vp]
    lib.moe_grouped_ffn_e4m3.argtypes = [vp, vp, i32, i64, vp, vp, i64, i64, vp, vp, vp, vp, vp,
                                         C.c_int, vp, vp, sz, vp]
    lib.moe_grouped_ffn_e4m3_workspace_size.restype = sz
    lib.moe_grouped_ffn_e4m3_workspace_size.argtypes = [i32, i64, i64]
    lib.moe_fp8_scale_update.argtypes = [vp, i32, vp, vp, vp]
    a = 4096
    need = lib.moe_ragged_dot_workspace_size(8)
    assert need >= 9 * 4 and lib.moe_ragged_dot_workspace_size(0) == 0
    rd = lambda **kw: lib.moe_ragged_dot(
        a, a, kw.get("E", 8), 1000, kw.get("W", a), kw.get("N", 128), kw.get("K", 64),
        kw.get("dt", 1), a, kw.get("zdt", 1), a, kw.get("wsb", need), None)
    assert rd(E=0) == 2 and rd(E=1025) == 2
    assert rd(K=96) == 2                    # bf16 rows of 192 bytes
    assert rd(N=96) == 2                    # not whole 64-column blocks
    assert rd(dt=0, zdt=1) == 3             # float32 inputs, bfloat16 output
    assert rd(dt=2) == 3                    # E4M3 goes through its own entry point
    assert rd(W=0) == 1
    assert rd(wsb=need - 1) == 5
    f8 = lambda **kw: lib.moe_ragged_dot_e4m3(
        kw.get("X", a), a, 8, 1000, a, kw.get("N", 128), kw.get("K", 128), kw.get("sx", a),
        kw.get("sw", None), a, kw.get("zdt", 1), a, kw.get("wsb", need), None)
    assert f8(K=64) == 2                    # E4M3 rows of 64 bytes
    assert f8(N=32) == 2
    assert f8(zdt=2) == 3                   # no E4M3 output
    assert f8(sx=a + 2) == 4                # a scale is a 4-byte aligned float
    assert f8(X=a + 8) == 4
    assert f8(wsb=need - 1) == 5
    qz = lambda **kw: lib.moe_quantize_e4m3(
        kw.get("x", a), kw.get("dt", 1), kw.get("n", 100), kw.get("s", a), kw.get("q", a),
        kw.get("amax", a), None)
    assert qz(dt=2) == 3
    assert qz(n=-1) == 2
    assert qz(q=0) == 1
    assert qz(q=a + 1) == 4
    assert qz(amax=a + 2) == 4
    assert qz(s=a + 1) == 4
    sq = lambda **kw: lib.moe_swiglu_quantize_e4m3(
        a, kw.get("dt", 1), a, kw.get("E", 8), 1000, kw.get("H", 64), kw.get("s", None),
        kw.get("hq", a), None, None)
    assert sq(H=40) == 2                    # not whole 16-column groups
    assert sq(E=0) == 2
    assert sq(dt=2) == 3
    assert sq(hq=0) == 1
    assert sq(s=a + 3) == 4
    fneed = lib.moe_grouped_ffn_e4m3_workspace_size(8, 1000, 128)
    assert fneed >= 1000 * 128 * 5
    ff = lambda **kw: lib.moe_grouped_ffn_e4m3(
        a, a, 8, 1000, a, a, kw.get("d", 128), kw.get("H", 128), None, None, kw.get("sh", None),
        None, a, kw.get("ydt", 1), kw.get("amax", None), a, kw.get("wsb", fneed), None)
    assert ff(d=64) == 2 and ff(H=192) == 2  # multiples of 128
    assert ff(ydt=2) == 3
    assert ff(sh=a + 1) == 4 and ff(amax=a + 2) == 4
    assert ff(wsb=fneed - 1) == 5
    lib.moe_permute_e4m3.argtypes = [vp, i64, i32, i64, vp, C.c_int, i64, i32, vp, i64, vp, vp, vp,
                                     vp, vp, vp, vp, vp, sz, vp]
    lib.moe_permute_workspace_size.restype = sz
    lib.moe_permute_workspace_size.argtypes = [i64, i32]
    pneed = lib.moe_permute_workspace_size(1000, 8)
    pe = lambda **kw: lib.moe_permute_e4m3(
        a, 1000, 8, -1, kw.get("src", a), kw.get("dt", 1), kw.get("w", 64), kw.get("div", 1),
        kw.get("dst", a), kw.get("R", 1000), a, a, a, a, a, kw.get("s", None), None, a,
        kw.get("wsb", pneed), None)
    assert pe(w=40) == 2                    # not whole 16-byte code chunks
    assert pe(div=0) == 2
    assert pe(R=999) == 2                   # fewer rows than assignments, dropless
    assert pe(dt=2) == 3
    assert pe(dst=0) == 1 and pe(src=0) == 1
    assert pe(s=a + 1) == 4
    assert pe(wsb=pneed - 1) == 5
    lib.moe_dispatch_pack.argtypes = [vp, i64, i32, i32, i32, i64, vp, C.c_int, i64, vp, vp, i64,
                                      vp, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_dispatch_pack_workspace_size.restype = sz
    lib.moe_dispatch_pack_workspace_size.argtypes = [i64, i32]
    dneed2 = lib.moe_dispatch_pack_workspace_size(8000, 64)
    assert dneed2 >= 8000 * 4
    dp = lambda **kw: lib.moe_dispatch_pack(
        a, 1000, kw.get("k", 8), kw.get("E", 384), kw.get("P", 64), -1, a, 1, kw.get("w", 64), a,
        a, kw.get("R", 8000), a, a, a, a, a, a, kw.get("wsb", dneed2), None)
    assert dp(E=380) == 2                   # experts not a multiple of the peers
    assert dp(k=17) == 2
    assert dp(R=7999) == 2                  # fewer rows than assignments, no cap
    assert dp(w=4) == 2                     # 8-byte rows
    assert dp(wsb=dneed2 - 1) == 5
    su = lambda **kw: lib.moe_fp8_scale_update(kw.get("h", a), kw.get("n", 16), kw.get("am", a),
                                               kw.get("s", a), None)
    assert su(n=0) == 2 and su(n=1025) == 2
    assert su(h=0) == 1 and su(s=0) == 1
    assert su(am=a + 2) == 4


def test_layer_workspace_layout(lib):
    """The stage offsets lie inside the workspace, 256-byte aligned, in carve order,
    and the stages a configuration lacks are reported absent."""
    import mixture_experts_transformer_amd as M
    for args, has_latent, has_c in [((8192, 6144, 3072, 384, 8, 3072, 2, 3072), True, True),
                                    ((8192, 2048, 0, 64, 4, 1024, 1, 2048), False, True),
                                    ((100, 256, 0, 16, 2, 128, 0, 128), False, False)]:
        desc = M.layer_desc(*args, "bf16")
        lay = M.moe_layer_workspace_layout(desc)
        assert lay["total"] == M.moe_layer_workspace_size(desc)
        assert (lay["z_pre"] is not None) == has_latent and (lay["z_e"] is not None) == has_latent
        assert (lay["c"] is not None) == has_c
        T, D, L, E, k, H, ns, Hs = args
        de = L if L else D
        order = [("row_src", T * k * 4), ("h", T * k * H * 2), ("Y", T * k * de * 2)]
        for (a, na), (b, _) in zip(order, order[1:]):
            assert lay[a] % 256 == 0 and lay[a] + na <= lay[b]
        assert lay["Y"] + T * k * de * 2 <= lay["total"]
    # a rejected desc is an error, not a layout
    bad = M.layer_desc(8, 64, 0, 0, 1, 64, 0, 64, "bf16")
    with pytest.raises(M.MoeError):
        M.moe_layer_workspace_layout(bad)
