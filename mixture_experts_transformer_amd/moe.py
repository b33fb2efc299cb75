"""Thin Python binding of libmoe's C ABI (include/moe.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libmoe.so.  torch supplies device memory and the current HIP stream.  If the
library is not built this module fails to import -- there is no fallback.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run `python mixture_experts_transformer_amd/build.py`"
                      " (or __graft_entry__.build()); there is no non-HIP fallback")
_lib = C.CDLL(LIB_PATH)

MOE_OK, MOE_EINVAL, MOE_ESHAPE, MOE_EDTYPE, MOE_EALIGN, MOE_EWORKSPACE, MOE_ELAUNCH = range(7)
MOE_F32, MOE_BF16 = 0, 1
MOE_COMBINE_KEEP_UNROUTED = 1
EV_NAMES = ["start", "downproj", "route", "permute", "gemm1", "gemm2", "combine", "shared",
            "output"]
MOE_EV_COUNT = len(EV_NAMES)

_vp, _i32, _i64, _f32, _sz = C.c_void_p, C.c_int32, C.c_int64, C.c_float, C.c_size_t


class LayerDesc(C.Structure):
    _fields_ = [("T", _i64), ("D", _i64), ("L", _i64), ("E", _i32), ("k", _i32), ("H", _i64),
                ("n_shared", _i32), ("Hs", _i64), ("dtype", C.c_int), ("eps", _f32),
                ("capacity", _i64)]


class LayerWeights(C.Structure):
    _fields_ = [(n, _vp) for n in ["W_dn", "norm_g", "W_r", "b_r", "W_gu", "W_d", "W_up",
                                   "W_gu_s", "W_d_s"]]


class LayerAux(C.Structure):
    _fields_ = [("logits", _vp), ("ids", _vp), ("w", _vp), ("counts", _vp), ("offsets", _vp),
                ("n_dropped", _vp), ("slot_row", _vp), ("events", _vp)]


_lib.moe_abi_version.restype = C.c_int
_lib.moe_status_str.restype = C.c_char_p
_lib.moe_status_str.argtypes = [C.c_int]
_lib.moe_route.restype = C.c_int
_lib.moe_route.argtypes = [_vp, C.c_int, _i64, _i64, _vp, _f32, _i32, _vp, _vp, _i32, _i32, _vp,
                           C.c_int, _vp, _vp, _vp, _vp]
_lib.moe_permute.restype = C.c_int
_lib.moe_permute.argtypes = [_vp, _i64, _i32, _i64, _vp, C.c_int, _i64, _i32, _vp, _i64, _vp, _vp,
                             _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_permute_workspace_size.restype = _sz
_lib.moe_permute_workspace_size.argtypes = [_i64, _i32]
_lib.moe_permute_noalloc.restype = C.c_int
_lib.moe_permute_noalloc.argtypes = [_vp, _i64, _i32, _i64, _vp, C.c_int, _i64, _i32, _vp, _i64,
                                     _vp, _vp, _vp, _vp, _vp, _vp]
MOE_PERMUTE_NOALLOC_SCRATCH_BYTES = 16 << 20
_lib.moe_grouped_ffn.restype = C.c_int
_lib.moe_grouped_ffn.argtypes = [_vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64, C.c_int, _vp, _vp,
                                 _sz, _vp]
_lib.moe_grouped_ffn_workspace_size.restype = _sz
_lib.moe_grouped_ffn_workspace_size.argtypes = [_i32, _i64, _i64, C.c_int]
_lib.moe_ragged_dot.restype = C.c_int
_lib.moe_ragged_dot.argtypes = [_vp, _vp, _i32, _i64, _vp, _i64, _i64, C.c_int, _vp, C.c_int, _vp,
                                _sz, _vp]
_lib.moe_ragged_dot_workspace_size.restype = _sz
_lib.moe_ragged_dot_workspace_size.argtypes = [_i32]
_lib.moe_ragged_dot_e4m3.restype = C.c_int
_lib.moe_ragged_dot_e4m3.argtypes = [_vp, _vp, _i32, _i64, _vp, _i64, _i64, _vp, _vp, _vp,
                                     C.c_int, _vp, _sz, _vp]
_lib.moe_quantize_e4m3.restype = C.c_int
_lib.moe_quantize_e4m3.argtypes = [_vp, C.c_int, _i64, _vp, _vp, _vp, _vp]
_lib.moe_swiglu_quantize_e4m3.restype = C.c_int
_lib.moe_swiglu_quantize_e4m3.argtypes = [_vp, C.c_int, _vp, _i32, _i64, _i64, _vp, _vp, _vp,
                                          _vp]
_lib.moe_grouped_ffn_e4m3.restype = C.c_int
_lib.moe_grouped_ffn_e4m3.argtypes = [_vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64, _vp, _vp, _vp,
                                      _vp, _vp, C.c_int, _vp, _vp, _sz, _vp]
_lib.moe_permute_e4m3.restype = C.c_int
_lib.moe_permute_e4m3.argtypes = [_vp, _i64, _i32, _i64, _vp, C.c_int, _i64, _i32, _vp, _i64, _vp,
                                  _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_dispatch_pack.restype = C.c_int
_lib.moe_dispatch_pack.argtypes = [_vp, _i64, _i32, _i32, _i32, _i64, _vp, C.c_int, _i64, _vp, _vp,
                                   _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]
_lib.moe_dispatch_pack_e4m3.restype = C.c_int
_lib.moe_dispatch_pack_e4m3.argtypes = [_vp, _i64, _i32, _i32, _i32, _i64, _vp, C.c_int, _i64, _vp,
                                        _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                                        _vp]
_lib.moe_dispatch_pack_workspace_size.restype = _sz
_lib.moe_dispatch_pack_workspace_size.argtypes = [_i64, _i32]
_lib.moe_fp8_scale_update.restype = C.c_int
_lib.moe_fp8_scale_update.argtypes = [_vp, _i32, _vp, _vp, _vp]
_lib.moe_grouped_ffn_e4m3_workspace_size.restype = _sz
_lib.moe_grouped_ffn_e4m3_workspace_size.argtypes = [_i32, _i64, _i64]
_lib.moe_ragged_dot_dlhs.restype = C.c_int
_lib.moe_ragged_dot_dlhs.argtypes = [_vp, _vp, _i32, _i64, _vp, _i64, _i64, C.c_int, _vp, _vp, _sz,
                                     _vp]
_lib.moe_ragged_dot_dlhs_workspace_size.restype = _sz
_lib.moe_ragged_dot_dlhs_workspace_size.argtypes = [_i32]
_lib.moe_ragged_dot_drhs.restype = C.c_int
_lib.moe_ragged_dot_drhs.argtypes = [_vp, _vp, _vp, _i32, _i64, _i64, _i64, C.c_int, _vp, C.c_int,
                                     _vp, _sz, _vp]
_lib.moe_ragged_dot_drhs_workspace_size.restype = _sz
_lib.moe_ragged_dot_drhs_workspace_size.argtypes = [_i32]
_lib.moe_grouped_ffn_bwd.restype = C.c_int
_lib.moe_grouped_ffn_bwd.argtypes = [_vp, _vp, _vp, _i32, _i64, _vp, _vp, _i64, _i64, C.c_int, _vp,
                                     _vp, _vp, C.c_int, _vp, _sz, _vp]
_lib.moe_grouped_ffn_bwd_workspace_size.restype = _sz
_lib.moe_grouped_ffn_bwd_workspace_size.argtypes = [_i32, _i64, _i64, C.c_int]
_lib.moe_combine.restype = C.c_int
_lib.moe_combine.argtypes = [_vp, C.c_int, _vp, _vp, _i64, _i32, _i64, _vp, _i32, _vp]
_lib.moe_layer_fwd.restype = C.c_int
_lib.moe_layer_fwd.argtypes = [C.POINTER(LayerDesc), C.POINTER(LayerWeights), _vp, _vp,
                               C.POINTER(LayerAux), _vp, _sz, _vp]
_lib.moe_layer_workspace_size.restype = _sz
_lib.moe_layer_workspace_size.argtypes = [C.POINTER(LayerDesc)]


class LayerWsLayout(C.Structure):
    _fields_ = [(n, _sz) for n in ["z_pre", "z_e", "row_src", "h", "Y", "c", "h_s", "total"]]


_lib.moe_layer_workspace_layout.restype = C.c_int
_lib.moe_layer_workspace_layout.argtypes = [C.POINTER(LayerDesc), C.POINTER(LayerWsLayout)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_lib.moe_status_str(status).decode()} (status {status})")


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _dt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MOE_F32
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    raise TypeError(f"libmoe takes float32 or bfloat16 tensors, got {t.dtype}")


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("libmoe takes device tensors")
    if not t.is_contiguous():
        raise ValueError("libmoe takes contiguous tensors")
    return t.data_ptr()


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes: int, device, ws):
    if ws is not None:
        return ws
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _check_group_out(out: dict, n: int, R_phys: int, G: int, where: str):
    """Caller-supplied grouping outputs: sizes and dtypes the kernels will write."""
    need = dict(slot_row=(n, torch.int32), row_src=(max(R_phys, 1), torch.int32),
                counts=(G, torch.int32), offsets=(G + 1, torch.int32),
                n_dropped=(1, torch.int64))
    for key, (size, dtype) in need.items():
        t = out.get(key)
        if t is None or t.numel() < size or t.dtype != dtype:
            raise ValueError(f"{where}: out[{key!r}] must hold at least {size} {dtype}")


def _check_rows(t, rows: int, width: int, dtype, where: str, what: str):
    """A destination matrix of at least `rows` rows of `width` elements of dtype."""
    if t.dtype != dtype or t.dim() != 2 or t.shape[0] < rows or t.shape[1] != width:
        raise ValueError(f"{where}: {what} must be [>= {rows}, {width}] {dtype}, "
                         f"got {tuple(t.shape)} {t.dtype}")


def abi_version() -> int:
    return _lib.moe_abi_version()


def status_str(s: int) -> str:
    return _lib.moe_status_str(s).decode()


# --------------------------------------------------------------------- route --
def moe_route(h, W_r, k, b_r=None, norm_g=None, eps=1e-5, apply_norm=False, r_out=None,
              logits_out=None, topk_ids=None, topk_w=None):
    """Router on h [T, d_r].  Returns (topk_ids [T,k] int32, topk_w [T,k] float32)."""
    T, d = h.shape
    E = W_r.shape[0]
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=h.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=h.device)
    r_dt = _dt(r_out) if r_out is not None else MOE_F32
    _check(_lib.moe_route(_ptr(h), _dt(h), T, d, _ptr(norm_g), eps, int(bool(apply_norm)),
                          _ptr(W_r), _ptr(b_r), E, k, _ptr(r_out), r_dt, _ptr(logits_out),
                          _ptr(topk_ids), _ptr(topk_w), _stream()), "moe_route")
    return topk_ids, topk_w


# ------------------------------------------------------------------- permute --
def moe_permute_workspace_size(n_assign: int, E: int) -> int:
    return int(_lib.moe_permute_workspace_size(n_assign, E))


def moe_permute(ids, E, capacity=-1, src=None, src_div=1, dst=None, R_phys=None, ws=None,
                out=None):
    """Group assignments by expert.  Returns dict(slot_row, row_src, counts, offsets,
    n_dropped) of device tensors (and fills dst if given).  `out` may supply those
    tensors (row_src with at least max(R_phys, 1) entries)."""
    ids = ids.reshape(-1)
    n = ids.numel()
    R_phys = n if R_phys is None else R_phys
    dev = ids.device
    if out is None:
        out = dict(slot_row=torch.empty(n, dtype=torch.int32, device=dev),
                   row_src=torch.empty(max(R_phys, 1), dtype=torch.int32, device=dev),
                   counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
    else:
        out = dict(out)
        _check_group_out(out, n, R_phys, E, "moe_permute")
    if src is not None:
        if dst is None:
            raise ValueError("moe_permute: a row copy needs dst")
        _check_rows(dst, R_phys, src.shape[-1], src.dtype, "moe_permute", "dst")
    need = moe_permute_workspace_size(n, E)
    ws = _ws(need, dev, ws)
    width = src.shape[-1] if src is not None else 0
    dt = _dt(src) if src is not None else MOE_F32
    _check(_lib.moe_permute(_ptr(ids), n, E, capacity, _ptr(src), dt, width, src_div, _ptr(dst),
                            R_phys, _ptr(out["slot_row"]), _ptr(out["row_src"]),
                            _ptr(out["counts"]), _ptr(out["offsets"]), _ptr(out["n_dropped"]),
                            _ptr(ws), ws.numel(), _stream()), "moe_permute")
    out["row_src"] = out["row_src"][:R_phys]
    return out


def moe_permute_noalloc(ids, E, out, capacity=-1, src=None, src_div=1, dst=None, R_phys=None):
    """moe_permute without a workspace, for callers that cannot allocate: the library's
    own device scratch (MOE_PERMUTE_NOALLOC_SCRATCH_BYTES) serves the grouping passes.
    Nothing is allocated here either: `out` supplies slot_row [>= n], row_src
    [>= max(R_phys, 1)], counts [>= E], offsets [>= E + 1] (int32) and n_dropped
    (int64 [>= 1]).  Calls that overlap on one device race on that scratch."""
    ids = ids.reshape(-1)
    n = ids.numel()
    R_phys = n if R_phys is None else R_phys
    _check_group_out(out, n, R_phys, E, "moe_permute_noalloc")
    if src is not None:
        if dst is None:
            raise ValueError("moe_permute_noalloc: a row copy needs dst")
        _check_rows(dst, R_phys, src.shape[-1], src.dtype, "moe_permute_noalloc", "dst")
    width = src.shape[-1] if src is not None else 0
    dt = _dt(src) if src is not None else MOE_F32
    _check(_lib.moe_permute_noalloc(_ptr(ids), n, E, capacity, _ptr(src), dt, width, src_div,
                                    _ptr(dst), R_phys, _ptr(out["slot_row"]), _ptr(out["row_src"]),
                                    _ptr(out["counts"]), _ptr(out["offsets"]),
                                    _ptr(out["n_dropped"]), _stream()), "moe_permute_noalloc")
    return out


def moe_permute_e4m3(ids, E, src, dst, capacity=-1, src_div=1, R_phys=None, scale=None,
                     amax=None, ws=None, out=None):
    """moe_permute whose row copy writes E4M3 codes of src / scale[0] into dst (uint8
    [R_phys, width]); amax (float32 [1]) receives max |x| over the rows read."""
    ids = ids.reshape(-1)
    n = ids.numel()
    R_phys = n if R_phys is None else R_phys
    dev = ids.device
    if out is None:
        out = dict(slot_row=torch.empty(n, dtype=torch.int32, device=dev),
                   row_src=torch.empty(max(R_phys, 1), dtype=torch.int32, device=dev),
                   counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
    else:
        out = dict(out)
        _check_group_out(out, n, R_phys, E, "moe_permute_e4m3")
    _check_rows(dst, R_phys, src.shape[-1], torch.uint8, "moe_permute_e4m3", "dst")
    ws = _ws(moe_permute_workspace_size(n, E), dev, ws)
    _check(_lib.moe_permute_e4m3(_ptr(ids), n, E, capacity, _ptr(src), _dt(src), src.shape[-1],
                                 src_div, _ptr(dst), R_phys, _ptr(out["slot_row"]),
                                 _ptr(out["row_src"]), _ptr(out["counts"]), _ptr(out["offsets"]),
                                 _ptr(out["n_dropped"]), _scale(scale), _ptr(amax), _ptr(ws),
                                 ws.numel(), _stream()), "moe_permute_e4m3")
    out["row_src"] = out["row_src"][:R_phys]
    return out


def moe_dispatch_pack_workspace_size(n_assign: int, n_peers: int) -> int:
    return int(_lib.moe_dispatch_pack_workspace_size(n_assign, n_peers))


def moe_dispatch_pack(expert_ids, E, n_peers, x, capacity=-1, R_phys=None, send_rows=None,
                      send_expert=None, ws=None, out=None):
    """The sender's half of an expert-parallel dispatch: the assignments expert_ids [T, k]
    grouped by destination peer (experts in contiguous blocks of E / n_peers), each kept
    row of x copied into send_rows and its local expert id into send_expert.  Returns
    dict(send_rows, send_expert, slot_row, row_src, counts, offsets, n_dropped)."""
    T, k = expert_ids.shape
    n = T * k
    R_phys = n if R_phys is None else R_phys
    dev = expert_ids.device
    if out is None:
        out = dict(slot_row=torch.empty(n, dtype=torch.int32, device=dev),
                   row_src=torch.empty(max(R_phys, 1), dtype=torch.int32, device=dev),
                   counts=torch.empty(n_peers, dtype=torch.int32, device=dev),
                   offsets=torch.empty(n_peers + 1, dtype=torch.int32, device=dev),
                   n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
    else:
        out = dict(out)
        _check_group_out(out, n, R_phys, n_peers, "moe_dispatch_pack")
    if send_rows is None:
        send_rows = torch.empty((R_phys, x.shape[-1]), dtype=x.dtype, device=dev)
    _check_rows(send_rows, R_phys, x.shape[-1], x.dtype, "moe_dispatch_pack", "send_rows")
    if send_expert is None:
        send_expert = torch.empty(max(R_phys, 1), dtype=torch.int32, device=dev)
    if send_expert.dtype != torch.int32 or send_expert.numel() < max(R_phys, 1):
        raise ValueError(f"moe_dispatch_pack: send_expert must hold at least {max(R_phys, 1)} int32")
    ws = _ws(moe_dispatch_pack_workspace_size(n, n_peers), dev, ws)
    _check(_lib.moe_dispatch_pack(_ptr(expert_ids), T, k, E, n_peers, capacity, _ptr(x), _dt(x),
                                  x.shape[-1], _ptr(send_rows), _ptr(send_expert), R_phys,
                                  _ptr(out["slot_row"]), _ptr(out["row_src"]), _ptr(out["counts"]),
                                  _ptr(out["offsets"]), _ptr(out["n_dropped"]), _ptr(ws),
                                  ws.numel(), _stream()), "moe_dispatch_pack")
    out.update(send_rows=send_rows, send_expert=send_expert[:R_phys],
               row_src=out["row_src"][:R_phys])
    return out


def moe_dispatch_pack_e4m3(expert_ids, E, n_peers, x, capacity=-1, R_phys=None, scale=None,
                           amax=None, send_rows=None, send_expert=None, ws=None):
    """moe_dispatch_pack sending E4M3 codes of x / scale[0] (uint8 send_rows)."""
    T, k = expert_ids.shape
    n = T * k
    R_phys = n if R_phys is None else R_phys
    dev = expert_ids.device
    out = dict(slot_row=torch.empty(n, dtype=torch.int32, device=dev),
               row_src=torch.empty(max(R_phys, 1), dtype=torch.int32, device=dev),
               counts=torch.empty(n_peers, dtype=torch.int32, device=dev),
               offsets=torch.empty(n_peers + 1, dtype=torch.int32, device=dev),
               n_dropped=torch.empty(1, dtype=torch.int64, device=dev))
    if send_rows is None:
        send_rows = torch.empty((R_phys, x.shape[-1]), dtype=torch.uint8, device=dev)
    _check_rows(send_rows, R_phys, x.shape[-1], torch.uint8, "moe_dispatch_pack_e4m3",
                "send_rows")
    if send_expert is None:
        send_expert = torch.empty(max(R_phys, 1), dtype=torch.int32, device=dev)
    if send_expert.dtype != torch.int32 or send_expert.numel() < max(R_phys, 1):
        raise ValueError("moe_dispatch_pack_e4m3: send_expert must hold at least "
                         f"{max(R_phys, 1)} int32")
    ws = _ws(moe_dispatch_pack_workspace_size(n, n_peers), dev, ws)
    _check(_lib.moe_dispatch_pack_e4m3(_ptr(expert_ids), T, k, E, n_peers, capacity, _ptr(x),
                                       _dt(x), x.shape[-1], _ptr(send_rows), _ptr(send_expert),
                                       R_phys, _ptr(out["slot_row"]), _ptr(out["row_src"]),
                                       _ptr(out["counts"]), _ptr(out["offsets"]),
                                       _ptr(out["n_dropped"]), _scale(scale), _ptr(amax),
                                       _ptr(ws), ws.numel(), _stream()), "moe_dispatch_pack_e4m3")
    out.update(send_rows=send_rows, send_expert=send_expert[:R_phys],
               row_src=out["row_src"][:R_phys])
    return out


# --------------------------------------------------------------- grouped FFN --
def moe_grouped_ffn_workspace_size(E: int, R_phys: int, H: int, dtype: torch.dtype) -> int:
    return int(_lib.moe_grouped_ffn_workspace_size(E, R_phys, H, _dt(torch.empty(0, dtype=dtype))))


def moe_grouped_ffn(X, offsets, W_gu, W_d, Y=None, ws=None):
    """Y[rows of e] = W_d[e] SwiGLU(W_gu[e] X[rows of e]) for row groups `offsets`."""
    R, d = X.shape
    E, twoH, d2 = W_gu.shape
    H = twoH // 2
    if Y is None:
        Y = torch.empty_like(X)
    ws = _ws(moe_grouped_ffn_workspace_size(E, R, H, X.dtype), X.device, ws)
    _check(_lib.moe_grouped_ffn(_ptr(X), _ptr(offsets), E, R, _ptr(W_gu), _ptr(W_d), d, H, _dt(X),
                                _ptr(Y), _ptr(ws), ws.numel(), _stream()), "moe_grouped_ffn")
    return Y


# ----------------------------------------------------- ragged dot forward --
MOE_E4M3 = 2


def moe_ragged_dot(X, offsets, W, Z=None, z_dtype=None, ws=None):
    """Z[r] = W[e] X[r] for the rows of each group e (W [E, N, K], X [R, K])."""
    R, K = X.shape
    E, N, _ = W.shape
    if Z is None:
        Z = torch.empty((R, N), dtype=z_dtype or X.dtype, device=X.device)
    ws = _ws(int(_lib.moe_ragged_dot_workspace_size(E)), X.device, ws)
    _check(_lib.moe_ragged_dot(_ptr(X), _ptr(offsets), E, R, _ptr(W), N, K, _dt(X), _ptr(Z),
                               _dt(Z), _ptr(ws), ws.numel(), _stream()), "moe_ragged_dot")
    return Z


def _scale(t):
    """Device pointer of a per-tensor scale (a float32 tensor of at least one element)
    or None (scale 1)."""
    if t is None:
        return None
    if t.dtype != torch.float32 or t.numel() < 1:
        raise ValueError("a scale is a float32 tensor of at least one element")
    return _ptr(t)


def moe_quantize_e4m3(x, scale=None, q=None, amax=None):
    """E4M3 codes (uint8 tensor of x's shape) of x / scale[0]; amax (float32 [1]) optional.
    scale: the dequantisation scale, a float32 device tensor, or None for 1."""
    if q is None:
        q = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    _check(_lib.moe_quantize_e4m3(_ptr(x), _dt(x), x.numel(), _scale(scale), _ptr(q), _ptr(amax),
                                  _stream()), "moe_quantize_e4m3")
    return q


def moe_ragged_dot_e4m3(Xq, offsets, Wq, scale_x=None, scale_w=None, Z=None,
                        z_dtype=torch.bfloat16, ws=None):
    """Z[r] = scale_x[0] scale_w[0] W[e] X[r] on E4M3 codes (uint8 Xq [R, K], Wq [E, N, K])."""
    R, K = Xq.shape
    E, N, _ = Wq.shape
    if Z is None:
        Z = torch.empty((R, N), dtype=z_dtype, device=Xq.device)
    ws = _ws(int(_lib.moe_ragged_dot_workspace_size(E)), Xq.device, ws)
    _check(_lib.moe_ragged_dot_e4m3(_ptr(Xq), _ptr(offsets), E, R, _ptr(Wq), N, K, _scale(scale_x),
                                    _scale(scale_w), _ptr(Z), _dt(Z), _ptr(ws), ws.numel(),
                                    _stream()), "moe_ragged_dot_e4m3")
    return Z


def moe_swiglu_quantize_e4m3(gu, offsets, scale=None, hq=None, amax=None):
    """E4M3 codes of silu(g) u / scale[0] for the rows < offsets[E] of gu = [g | u]
    ([R, 2H], float32 or bf16); amax (float32 [1]) optional."""
    R, twoH = gu.shape
    H = twoH // 2
    E = offsets.numel() - 1
    if hq is None:
        hq = torch.empty((R, H), dtype=torch.uint8, device=gu.device)
    _check(_lib.moe_swiglu_quantize_e4m3(_ptr(gu), _dt(gu), _ptr(offsets), E, R, H, _scale(scale),
                                         _ptr(hq), _ptr(amax), _stream()),
           "moe_swiglu_quantize_e4m3")
    return hq


def moe_grouped_ffn_e4m3_workspace_size(E: int, R_phys: int, H: int) -> int:
    return int(_lib.moe_grouped_ffn_e4m3_workspace_size(E, R_phys, H))


def moe_grouped_ffn_e4m3(Xq, offsets, W_gu_q, W_d_q, scale_x=None, scale_gu=None, scale_h=None,
                         scale_d=None, Y=None, y_dtype=torch.bfloat16, amax_h=None, ws=None):
    """The gated expert MLP on E4M3 codes (Xq [R, d], W_gu_q [E, 2H, d], W_d_q [E, d, H]):
    [g | u] = s_x s_gu W_gu_q[e] Xq[r] (bf16), h's codes = E4M3(silu(g) u / s_h),
    Y[r] = s_h s_d W_d_q[e] hq[r].  Scales are float32 device tensors (None = 1).  The
    workspace holds [g | u] then h's codes."""
    R, d = Xq.shape
    E, twoH, _ = W_gu_q.shape
    H = twoH // 2
    if Y is None:
        Y = torch.empty((R, d), dtype=y_dtype, device=Xq.device)
    ws = _ws(moe_grouped_ffn_e4m3_workspace_size(E, R, H), Xq.device, ws)
    _check(_lib.moe_grouped_ffn_e4m3(_ptr(Xq), _ptr(offsets), E, R, _ptr(W_gu_q), _ptr(W_d_q), d,
                                     H, _scale(scale_x), _scale(scale_gu), _scale(scale_h),
                                     _scale(scale_d), _ptr(Y), _dt(Y), _ptr(amax_h), _ptr(ws),
                                     ws.numel(), _stream()), "moe_grouped_ffn_e4m3")
    return Y


def moe_fp8_scale_update(history, amax, scale):
    """Delayed scaling: history (float32 [len], newest first) <- [amax, history[:-1]];
    scale[0] <- largest finite entry / 448 (1 if none is positive).  All on the device."""
    _check(_lib.moe_fp8_scale_update(_ptr(history), history.numel(), _scale(amax), _scale(scale),
                                     _stream()), "moe_fp8_scale_update")
    return scale


# --------------------------------------------------------- ragged dot VJP --
def moe_ragged_dot_dlhs(dZ, offsets, W, dX=None, ws=None):
    """dX[r] = W[e]^T dZ[r] for the rows of each group e (W [E, N, K], dZ [R, N])."""
    R, N = dZ.shape
    E, N2, K = W.shape
    if dX is None:
        dX = torch.empty((R, K), dtype=dZ.dtype, device=dZ.device)
    ws = _ws(int(_lib.moe_ragged_dot_dlhs_workspace_size(E)), dZ.device, ws)
    _check(_lib.moe_ragged_dot_dlhs(_ptr(dZ), _ptr(offsets), E, R, _ptr(W), N, K, _dt(dZ),
                                    _ptr(dX), _ptr(ws), ws.numel(), _stream()),
           "moe_ragged_dot_dlhs")
    return dX


def moe_ragged_dot_drhs(X, dZ, offsets, dW=None, dw_dtype=None, ws=None):
    """dW[e] = sum over the rows r of group e of dZ[r] X[r]^T -> [E, N, K]."""
    R, K = X.shape
    N = dZ.shape[1]
    E = offsets.numel() - 1
    if dW is None:
        dW = torch.empty((E, N, K), dtype=dw_dtype or X.dtype, device=X.device)
    ws = _ws(int(_lib.moe_ragged_dot_drhs_workspace_size(E)), X.device, ws)
    _check(_lib.moe_ragged_dot_drhs(_ptr(X), _ptr(dZ), _ptr(offsets), E, R, N, K, _dt(X), _ptr(dW),
                                    _dt(dW), _ptr(ws), ws.numel(), _stream()),
           "moe_ragged_dot_drhs")
    return dW


def moe_grouped_ffn_bwd_workspace_size(E: int, R_phys: int, H: int, dtype: torch.dtype) -> int:
    return int(_lib.moe_grouped_ffn_bwd_workspace_size(E, R_phys, H,
                                                        _dt(torch.empty(0, dtype=dtype))))


def moe_grouped_ffn_bwd(X, dY, offsets, W_gu, W_d, dX=None, dW_gu=None, dW_d=None,
                        dw_dtype=None, ws=None):
    """Backward of moe_grouped_ffn: returns (dX, dW_gu, dW_d)."""
    R, d = X.shape
    E, twoH, _ = W_gu.shape
    H = twoH // 2
    wdt = dw_dtype or X.dtype
    if dX is None:
        dX = torch.empty_like(X)
    if dW_gu is None:
        dW_gu = torch.empty(W_gu.shape, dtype=wdt, device=X.device)
    if dW_d is None:
        dW_d = torch.empty(W_d.shape, dtype=wdt, device=X.device)
    ws = _ws(moe_grouped_ffn_bwd_workspace_size(E, R, H, X.dtype), X.device, ws)
    _check(_lib.moe_grouped_ffn_bwd(_ptr(X), _ptr(dY), _ptr(offsets), E, R, _ptr(W_gu), _ptr(W_d),
                                    d, H, _dt(X), _ptr(dX), _ptr(dW_gu), _ptr(dW_d), _dt(dW_gu),
                                    _ptr(ws), ws.numel(), _stream()), "moe_grouped_ffn_bwd")
    return dX, dW_gu, dW_d


# ------------------------------------------------------------------- combine --
def moe_combine(Y, slot_row, w, T, k, out=None, flags=0):
    width = Y.shape[1]
    if out is None:
        out = torch.empty((T, width), dtype=Y.dtype, device=Y.device)
    _check(_lib.moe_combine(_ptr(Y), _dt(Y), _ptr(slot_row), _ptr(w), T, k, width, _ptr(out),
                            flags, _stream()), "moe_combine")
    return out


# ---------------------------------------------------------------- full layer --
def layer_desc(T, D, L, E, k, H, n_shared, Hs, dtype, eps=1e-5, capacity=-1) -> LayerDesc:
    dt = MOE_BF16 if dtype in (torch.bfloat16, "bf16") else MOE_F32
    return LayerDesc(T, D, L, E, k, H, n_shared, Hs, dt, eps, capacity)


def moe_layer_workspace_size(desc: LayerDesc) -> int:
    return int(_lib.moe_layer_workspace_size(C.byref(desc)))


def moe_layer_workspace_layout(desc: LayerDesc) -> dict:
    """Byte offsets of the layer's intermediate stages inside its workspace (None where
    the configuration has no such stage), and the workspace's total size."""
    lay = LayerWsLayout()
    _check(_lib.moe_layer_workspace_layout(C.byref(desc), C.byref(lay)),
           "moe_layer_workspace_layout")
    none = (1 << (8 * C.sizeof(_sz))) - 1
    return {n: (None if getattr(lay, n) == none else int(getattr(lay, n)))
            for n, _ in LayerWsLayout._fields_}


def moe_grouped_ffn_hidden_offset(E: int) -> int:
    """Byte offset of the hidden h inside moe_grouped_ffn's workspace (after the
    row-tile prefix of E + 1 int32, padded to 256 bytes)."""
    return ((E + 1) * 4 + 255) // 256 * 256


def moe_layer_fwd(desc: LayerDesc, W: dict, x, y=None, aux: dict | None = None, ws=None,
                  events=None):
    """Whole layer forward.  W holds device tensors named as moe_layer_weights;
    aux (optional) maps logits/ids/w/counts/offsets/n_dropped/slot_row to output
    tensors; events (optional) is a list of MOE_EV_COUNT raw hipEvent_t handles."""
    if y is None:
        y = torch.empty_like(x)
    ws = _ws(moe_layer_workspace_size(desc), x.device, ws)
    wts = LayerWeights(*[_ptr(W.get(n)) for n, _ in LayerWeights._fields_])
    ev_arr = None
    auxs = None
    if aux is not None or events is not None:
        aux = aux or {}
        if events is not None:
            ev_arr = (C.c_void_p * MOE_EV_COUNT)(*events)
        auxs = LayerAux(*[_ptr(aux.get(n)) for n, _ in LayerAux._fields_[:-1]],
                        C.cast(ev_arr, C.c_void_p) if ev_arr is not None else None)
    _check(_lib.moe_layer_fwd(C.byref(desc), C.byref(wts), _ptr(x), _ptr(y),
                              C.byref(auxs) if auxs is not None else None, _ptr(ws), ws.numel(),
                              _stream()), "moe_layer_fwd")
    return y
