"""Python face of the CPU oracle (moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use this module; the GPU library never imports it, and this
module imports nothing from the GPU library.  Arrays are numpy; bfloat16 data is
passed as its raw uint16 bits, float32 as float32.  Every function is a thin
ctypes call into the C oracle, whose header comment cites the passages each step
follows.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
import threading

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_oracle.c")
LIB = os.path.join(HERE, "libmoe_oracle.so")

DT_F32 = 0
DT_BF16 = 1

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, OpenMP over tokens, no FMA contraction)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
               "-fPIC", "-shared", "-Wall", "-o", tmp, SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


class Dims(C.Structure):
    _fields_ = [("T", C.c_int64), ("D", C.c_int64), ("L", C.c_int64), ("E", C.c_int32),
                ("k", C.c_int32), ("H", C.c_int64), ("n_shared", C.c_int32), ("Hs", C.c_int64),
                ("dtype", C.c_int32), ("eps", C.c_double)]


class Weights(C.Structure):
    _fields_ = [("W_dn", C.c_void_p), ("norm_g", C.c_void_p), ("W_r", C.c_void_p),
                ("b_r", C.c_void_p), ("W_gu_e", C.c_void_p), ("W_d_e", C.c_void_p),
                ("W_up", C.c_void_p), ("W_gu_s", C.c_void_p), ("W_d_s", C.c_void_p)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = C.CDLL(LIB)
            vp, i32, i64, f64 = C.c_void_p, C.c_int32, C.c_int64, C.c_double
            L.moe_ref_set_threads.argtypes = [C.c_int]
            L.moe_ref_max_threads.restype = C.c_int
            L.moe_ref_to_bf16.restype = C.c_uint16
            L.moe_ref_to_bf16.argtypes = [f64]
            L.moe_ref_rmsnorm_row.argtypes = [vp, i64, vp, f64, vp]
            L.moe_ref_topk.argtypes = [vp, i64, i32, i32, vp, vp]
            L.moe_ref_capacity.restype = i64
            L.moe_ref_capacity.argtypes = [i64, i64, i64, i64]
            L.moe_ref_permute.restype = C.c_int
            L.moe_ref_permute.argtypes = [vp, i64, i32, i64, vp, vp, vp, vp, i64, vp]
            L.moe_ref_expert_rows.argtypes = [vp, C.c_int, i64, i64, i64, vp, vp, vp, vp, vp]
            L.moe_ref_combine.argtypes = [vp, C.c_int, vp, vp, i64, i32, i64, vp]
            L.moe_ref_e4m3_value.restype = f64
            L.moe_ref_e4m3_value.argtypes = [C.c_uint8]
            L.moe_ref_to_e4m3.restype = C.c_uint8
            L.moe_ref_to_e4m3.argtypes = [f64]
            L.moe_ref_quantize_e4m3.argtypes = [vp, C.c_int, i64, C.c_float, vp, vp]
            L.moe_ref_fp8_scale_update.argtypes = [vp, i32, C.c_float, vp]
            L.moe_ref_swiglu_quantize_e4m3.argtypes = [vp, C.c_int, i64, i64, C.c_float, vp, vp,
                                                       vp]
            L.moe_ref_ragged_dot_e4m3.argtypes = [vp, vp, vp, i32, i64, i64, f64, vp]
            L.moe_ref_ragged_dot.argtypes = [vp, vp, C.c_int, vp, i32, i64, i64, vp]
            L.moe_ref_ragged_dlhs.argtypes = [vp, vp, C.c_int, vp, i32, i64, i64, vp]
            L.moe_ref_ragged_drhs.argtypes = [vp, vp, C.c_int, vp, i32, i64, i64, vp]
            L.moe_ref_expert_rows_bwd.argtypes = [vp, vp, C.c_int, vp, i32, i64, i64, vp, vp,
                                                  vp, vp, vp]
            L.moe_ref_route_tokens.argtypes = [C.POINTER(Dims), C.POINTER(Weights), vp, vp, i64,
                                               vp, vp, vp, vp, vp]
            L.moe_ref_output_tokens.argtypes = [C.POINTER(Dims), C.POINTER(Weights), vp, vp, i64,
                                                vp, vp, vp, vp, vp]
            _lib = L
    return _lib


def set_threads(n: int) -> int:
    """Threads the oracle's parallel loops use from now on; returns the previous
    count.  Timing plumbing only: no result depends on it."""
    prev = int(lib().moe_ref_max_threads())
    lib().moe_ref_set_threads(int(n))
    return prev


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _dt_of(a) -> int:
    if a.dtype == np.uint16:
        return DT_BF16
    if a.dtype == np.float32:
        return DT_F32
    raise TypeError(f"oracle takes float32 or bfloat16-as-uint16 arrays, got {a.dtype}")


# ----------------------------------------------------------------- storage --

def to_bf16(x) -> np.ndarray:
    """Round doubles to bfloat16 (ties to even, straight from double); uint16 bits."""
    x = np.asarray(x, dtype=np.float64)
    f = lib().moe_ref_to_bf16
    return np.array([f(float(v)) for v in x.ravel()], dtype=np.uint16).reshape(x.shape)


def bf16_to_f64(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rmsnorm_row(v, g=None, eps=1e-5) -> np.ndarray:
    v = _c(v, np.float64)
    gg = None if g is None else _c(g, np.float32)
    z = np.empty_like(v)
    lib().moe_ref_rmsnorm_row(_p(v), v.size, _p(gg), eps, _p(z))
    return z


# ----------------------------------------------------------------- routing --

def topk(logits, k: int):
    """logits [T, E] float32 -> (ids [T, k] int32, w [T, k] float32)."""
    lg = _c(logits, np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    lib().moe_ref_topk(_p(lg), T, E, k, _p(ids), _p(w))
    return ids, w


def capacity(cf_num: int, cf_den: int, n_assign: int, E: int) -> int:
    return int(lib().moe_ref_capacity(cf_num, cf_den, n_assign, E))


def permute(ids, E: int, capacity: int = -1, R_phys: int | None = None) -> dict:
    """ids [n] int32 (negative = padding) -> grouping maps (see moe_oracle.c)."""
    ids = _c(ids, np.int32).ravel()
    n = ids.size
    if R_phys is None:
        R_phys = n
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    slot_row = np.empty(n, np.int32)
    row_src = np.empty(max(R_phys, 1), np.int32)
    nd = np.zeros(1, np.int64)
    rc = lib().moe_ref_permute(_p(ids), n, E, capacity, _p(counts), _p(offsets), _p(slot_row),
                               _p(row_src), R_phys, _p(nd))
    if rc != 0:
        raise ValueError("oracle permute: expert id out of range or too few rows")
    return dict(counts=counts, offsets=offsets, slot_row=slot_row, row_src=row_src[:R_phys],
                n_dropped=int(nd[0]))


# ----------------------------------------------------------------- experts --

def expert_rows(X, expert, W_gu_e, W_d_e, H: int, want_h: bool = False):
    """X [n, d] (float32 or bf16 bits), expert [n] -> Y [n, d] float64 (unrounded).

    W_gu_e / W_d_e: sequences indexed by expert id of arrays [2H, d] / [d, H]
    (entries for unused experts may be None)."""
    X = np.ascontiguousarray(X)
    dt = _dt_of(X)
    n, d = X.shape
    expert = _c(expert, np.int32)
    keep = []
    gu_ptrs = (C.c_void_p * len(W_gu_e))()
    d_ptrs = (C.c_void_p * len(W_d_e))()
    for e, (a, b) in enumerate(zip(W_gu_e, W_d_e)):
        if a is None:
            continue
        a = np.ascontiguousarray(a)
        b = np.ascontiguousarray(b)
        assert a.dtype == X.dtype and b.dtype == X.dtype
        assert a.shape == (2 * H, d) and b.shape == (d, H)
        keep += [a, b]
        gu_ptrs[e] = a.ctypes.data
        d_ptrs[e] = b.ctypes.data
    Y = np.empty((n, d), np.float64)
    h = np.empty((n, H), np.float64) if want_h else None
    lib().moe_ref_expert_rows(_p(X), dt, n, d, H, _p(expert), C.cast(gu_ptrs, C.c_void_p),
                              C.cast(d_ptrs, C.c_void_p), _p(Y), _p(h))
    return (Y, h) if want_h else Y


def e4m3_value(code: int) -> float:
    """Value of an OCP E4M3 code (NaN for S.1111.111)."""
    return lib().moe_ref_e4m3_value(int(code))


def to_e4m3(x: float) -> int:
    """Nearest E4M3 code, ties to even mantissa, saturating at +-448."""
    return int(lib().moe_ref_to_e4m3(float(x)))


def quantize_e4m3(x, inv_scale: float):
    """x (float32 or bf16 bits) -> (E4M3 codes uint8 of x's shape, amax float)."""
    x = np.ascontiguousarray(x)
    q = np.empty(x.shape, np.uint8)
    amax = C.c_float()
    lib().moe_ref_quantize_e4m3(_p(x), _dt_of(x), x.size, inv_scale, _p(q), C.byref(amax))
    return q, amax.value


def fp8_scale_update(history, amax: float):
    """Delayed scaling's update: returns (new history [len] float32, scale, 1/scale)."""
    h = np.array(history, dtype=np.float32)
    sc = np.zeros(2, np.float32)
    lib().moe_ref_fp8_scale_update(_p(h), h.size, float(amax), _p(sc))
    return h, float(sc[0]), float(sc[1])


def ragged_dot_e4m3(X, W, offsets, scale: float):
    """Z[r] = scale * W[e] X[r] on E4M3 codes: X [R, K] uint8, W [E, N, K] uint8 -> Z [R, N]
    float64 (rows >= offsets[E] NaN)."""
    X, W = np.ascontiguousarray(X, np.uint8), np.ascontiguousarray(W, np.uint8)
    E, N, K = W.shape
    off = _c(offsets, np.int32)
    assert X.shape[1] == K and off.shape == (E + 1,) and off[-1] <= X.shape[0]
    Z = np.full((X.shape[0], N), np.nan)
    lib().moe_ref_ragged_dot_e4m3(_p(X), _p(W), _p(off), E, N, K, float(scale), _p(Z))
    return Z


def swiglu_quantize_e4m3(gu, inv_scale: float, want_h: bool = False):
    """gu [n, 2H] (float32 or bf16 bits, gate half first) -> (q [n, H] E4M3 codes of
    float32(silu(g) u) * inv_scale, amax = max |float32(silu(g) u)| [, h in double])."""
    gu = np.ascontiguousarray(gu)
    n, twoH = gu.shape
    H = twoH // 2
    q = np.empty((n, H), np.uint8)
    h = np.empty((n, H), np.float64) if want_h else None
    amax = C.c_float()
    lib().moe_ref_swiglu_quantize_e4m3(_p(gu), _dt_of(gu), n, H, float(inv_scale), _p(q),
                                       C.byref(amax), _p(h))
    return (q, amax.value, h) if want_h else (q, amax.value)


def expert_mlp_e4m3(Xq, W_gu_q, W_d_q, offsets, scale_gu: float, inv_scale_h: float,
                    scale_d: float) -> dict:
    """The gated expert MLP on E4M3 codes, as moe_grouped_ffn_e4m3 defines it: [g | u]
    = scale_gu W_gu_q[e] Xq[r] stored in bf16, h's codes from swiglu_quantize_e4m3, Y =
    scale_d W_d_q[e] hq[r] in double.  Rows are those below offsets[E]."""
    off = _c(offsets, np.int32)
    R = int(off[-1])
    gu = to_bf16(ragged_dot_e4m3(Xq[:R], W_gu_q, off, scale_gu)[:R])
    hq, amax, h = swiglu_quantize_e4m3(gu, inv_scale_h, want_h=True)
    Y = ragged_dot_e4m3(hq, W_d_q, off, scale_d)
    return {"gu": gu, "h": h, "hq": hq, "amax_h": amax, "Y": Y}


def ragged_dot(X, W, offsets):
    """Z[r] = W[e] X[r] in double: X [R, K], W [E, N, K] (float32 or bf16 bits) -> [R, N]."""
    X, W = np.ascontiguousarray(X), np.ascontiguousarray(W)
    assert X.dtype == W.dtype
    E, N, K = W.shape
    off = _c(offsets, np.int32)
    Z = np.full((X.shape[0], N), np.nan)
    lib().moe_ref_ragged_dot(_p(X), _p(W), _dt_of(X), _p(off), E, N, K, _p(Z))
    return Z


def ragged_dlhs(dZ, W, offsets):
    """Input gradient of the grouped matmul Z[r] = W[e(r)] X[r]: dZ [R, N], W [E, N, K]
    (float32 or bf16 bits) -> dX [R, K] float64; rows >= offsets[E] are NaN (unwritten)."""
    dZ, W = np.ascontiguousarray(dZ), np.ascontiguousarray(W)
    dt = _dt_of(dZ)
    assert W.dtype == dZ.dtype
    E, N, K = W.shape
    off = _c(offsets, np.int32)
    assert off.shape == (E + 1,) and dZ.shape[1] == N and off[-1] <= dZ.shape[0]
    dX = np.full((dZ.shape[0], K), np.nan)
    lib().moe_ref_ragged_dlhs(_p(dZ), _p(W), dt, _p(off), E, N, K, _p(dX))
    return dX


def ragged_drhs(X, dZ, offsets):
    """Weight gradient of the grouped matmul: X [R, K], dZ [R, N] -> dW [E, N, K] float64."""
    X, dZ = np.ascontiguousarray(X), np.ascontiguousarray(dZ)
    dt = _dt_of(X)
    assert dZ.dtype == X.dtype
    off = _c(offsets, np.int32)
    E = off.size - 1
    N, K = dZ.shape[1], X.shape[1]
    assert off[-1] <= min(X.shape[0], dZ.shape[0])
    dW = np.empty((E, N, K))
    lib().moe_ref_ragged_drhs(_p(X), _p(dZ), dt, _p(off), E, N, K, _p(dW))
    return dW


def expert_rows_bwd(X, dY, offsets, W_gu, W_d):
    """Backward of the gated expert MLP over row groups.  X, dY [R, d]; W_gu [E, 2H, d];
    W_d [E, d, H] (float32 or bf16 bits) -> (dX [R, d], dW_gu [E, 2H, d], dW_d [E, d, H])
    float64; dX rows >= offsets[E] are NaN (unwritten)."""
    X, dY = np.ascontiguousarray(X), np.ascontiguousarray(dY)
    W_gu, W_d = np.ascontiguousarray(W_gu), np.ascontiguousarray(W_d)
    dt = _dt_of(X)
    assert dY.dtype == X.dtype == W_gu.dtype == W_d.dtype
    off = _c(offsets, np.int32)
    E = off.size - 1
    d = X.shape[1]
    H = W_d.shape[2]
    assert W_gu.shape == (E, 2 * H, d) and W_d.shape == (E, d, H) and dY.shape[1] == d
    dX = np.full((X.shape[0], d), np.nan)
    dWgu = np.empty((E, 2 * H, d))
    dWd = np.empty((E, d, H))
    lib().moe_ref_expert_rows_bwd(_p(X), _p(dY), dt, _p(off), E, d, H, _p(W_gu), _p(W_d),
                                  _p(dX), _p(dWgu), _p(dWd))
    return dX, dWgu, dWd


def combine(Y, slot_row, w, T: int, k: int):
    """Ordered weighted gather; Y [*, d] (float32 or bf16 bits) -> c [T, d] float64."""
    Y = np.ascontiguousarray(Y)
    dt = _dt_of(Y)
    d = Y.shape[1]
    sr = _c(slot_row, np.int32)
    ww = None if w is None else _c(w, np.float32)
    c = np.empty((T, d), np.float64)
    lib().moe_ref_combine(_p(Y), dt, _p(sr), _p(ww), T, k, d, _p(c))
    return c


# -------------------------------------------------------------- full layer --

class LayerWeights:
    """Host copies of one layer's weights in the oracle's layout.

    W_gu_e / W_d_e are per-expert lists so that only the experts a test touches
    need to be on the host."""

    def __init__(self, W_dn, norm_g, W_r, b_r, W_gu_e, W_d_e, W_up, W_gu_s, W_d_s):
        c = np.ascontiguousarray
        self.W_dn = None if W_dn is None else c(W_dn)
        self.norm_g = None if norm_g is None else c(norm_g, dtype=np.float32)
        self.W_r = c(W_r, dtype=np.float32)
        self.b_r = None if b_r is None else c(b_r, dtype=np.float32)
        self.W_gu_e = [None if a is None else c(a) for a in W_gu_e]
        self.W_d_e = [None if a is None else c(a) for a in W_d_e]
        self.W_up = None if W_up is None else c(W_up)
        self.W_gu_s = None if W_gu_s is None else c(W_gu_s)
        self.W_d_s = None if W_d_s is None else c(W_d_s)
        E = len(self.W_gu_e)
        self._gu = (C.c_void_p * E)(*[None if a is None else a.ctypes.data for a in self.W_gu_e])
        self._d = (C.c_void_p * E)(*[None if a is None else a.ctypes.data for a in self.W_d_e])

    def cstruct(self) -> Weights:
        return Weights(_p(self.W_dn), _p(self.norm_g), _p(self.W_r), _p(self.b_r),
                       C.cast(self._gu, C.c_void_p), C.cast(self._d, C.c_void_p),
                       _p(self.W_up), _p(self.W_gu_s), _p(self.W_d_s))


def dims(T, D, L, E, k, H, n_shared, Hs, dtype: int, eps: float = 1e-5) -> Dims:
    return Dims(T, D, L, E, k, H, n_shared, Hs, dtype, eps)


def route_tokens(dm: Dims, W: LayerWeights, x, tok):
    """Router part for tokens `tok`: returns dict(z, logits32, logits64, ids, w)."""
    x = np.ascontiguousarray(x)
    tok = _c(tok, np.int32)
    n = tok.size
    d_r = dm.L if dm.L > 0 else dm.D
    z = np.empty((n, d_r), np.float64)
    l32 = np.empty((n, dm.E), np.float32)
    l64 = np.empty((n, dm.E), np.float64)
    ids = np.empty((n, dm.k), np.int32)
    w = np.empty((n, dm.k), np.float32)
    ws = W.cstruct()
    lib().moe_ref_route_tokens(C.byref(dm), C.byref(ws), _p(x), _p(tok), n, _p(z), _p(l32),
                               _p(l64), _p(ids), _p(w))
    return dict(z=z, logits32=l32, logits64=l64, ids=ids, w=w)


def output_tokens(dm: Dims, W: LayerWeights, x, tok, ids, w, keep=None, want_c=False):
    """Output part for tokens `tok` given their routing: y [n, D] float64 (unrounded)."""
    x = np.ascontiguousarray(x)
    tok = _c(tok, np.int32)
    n = tok.size
    ids = _c(ids, np.int32)
    w = _c(w, np.float32)
    kp = None if keep is None else _c(keep, np.int32)
    d_e = dm.L if dm.L > 0 else dm.D
    y = np.empty((n, dm.D), np.float64)
    c = np.empty((n, d_e), np.float64) if want_c else None
    ws = W.cstruct()
    lib().moe_ref_output_tokens(C.byref(dm), C.byref(ws), _p(x), _p(tok), n, _p(ids), _p(w),
                                _p(kp), _p(y), _p(c))
    return (y, c) if want_c else y
