"""ctypes binding of ``libmoe.so`` (declared in ``include/moe.h``).

Argument marshalling only: each function has the C name, takes torch tensors
(or raw integer addresses, or None for NULL) and ints, passes their device
addresses to the library and raises :class:`MoeError` on a non-zero status.
Every step of the layer runs in the library's HIP kernels; if the library is
missing this module raises on import instead of computing anything itself.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_LIB", os.path.join(PKG, "libmoe.so"))

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python -m routing_permute_grouped_moe_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTER_WG_SPLIT = 1          # moe_router_logits_bwd: reuse the forward's split of wg
MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = range(5)

_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        detail = _lib.moe_last_error().decode()
        super().__init__(f"{fn}: {_lib.moe_status_string(status).decode()} ({detail})")
        self.status = status


class SharedExpert(ctypes.Structure):
    """``moe_shared_expert``: the always-on shared expert run as one more group."""
    _fields_ = [("T", _I), ("x", _P), ("w13", _P), ("w2", _P), ("h13", _P), ("act", _P),
                ("y", _P), ("dy", _P), ("dh13", _P), ("dx", _P), ("dw13", _P), ("dw2", _P)]


_SIGS = {
    "moe_status_string": (ctypes.c_char_p, [_I]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (_I, []),
    "moe_router_workspace_bytes": (_SZ, [_I, _I, _I, _I]),
    "moe_router_logits": (_I, [_P, _I, _P, _P, _I, _I, _I, _P, _P, _SZ, _P]),
    "moe_router_logits_bwd": (_I, [_P, _P, _I, _P, _I, _I, _I, _P, _P, _P, _I, _P, _SZ, _P]),
    "moe_route": (_I, [_P, _I, _I, _I, _P, _P, _P]),
    "moe_route_bwd": (_I, [_P, _P, _P, _I, _I, _I, _P, _P]),
    "moe_permute_workspace_bytes": (_SZ, [_I, _I, _I]),
    "moe_permute": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_permute_noalloc_max_scratch_bytes": (_SZ, []),
    "moe_permute_noalloc": (_I, [_P, _I, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P]),
    "moe_load_stats": (_I, [_P, _I, _I, _P, _P, _P, _P]),
    "moe_permute_capacity": (_I, [_P, _I, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P, _SZ,
                                  _P]),
    "moe_clear_empty_rows": (_I, [_P, _I, _I, _I, _P, _P]),
    "moe_permute_bwd": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P]),
    "moe_unpermute_combine": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P]),
    "moe_unpermute_combine_bwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _P]),
    "moe_gmm_workspace_bytes": (_SZ, []),
    "moe_grouped_gemm_fwd": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                  ctypes.POINTER(SharedExpert), _P, _SZ, _P]),
    "moe_grouped_gemm_bwd_dx": (_I, [_P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P,
                                     ctypes.POINTER(SharedExpert), _P, _SZ, _P]),
    "moe_grouped_gemm_bwd_dw": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P,
                                     ctypes.POINTER(SharedExpert), _P, _SZ, _P]),
    "moe_grouped_gemm_bwd": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _P,
                                  _P, ctypes.POINTER(SharedExpert), _P, _SZ, _P]),
    "moe_grouped_gemm_fwd_gather": (_I, [_P, _P, _I, _P, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                                         _P, ctypes.POINTER(SharedExpert), _P, _SZ, _P]),
    "moe_grouped_gemm_bwd_dw_recompute": (_I, [_P, _P, _I, _P, _P, _P, _P, _P, _I, _I, _I, _I,
                                               _I, _I, _P, _P, ctypes.POINTER(SharedExpert), _P,
                                               _SZ, _P]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def addr(t) -> Optional[int]:
    """Device address of a tensor (or an int address, or None for NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    st = getattr(_lib, name)(*args)
    if st != MOE_OK:
        raise MoeError(name, st)


def dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return MOE_BF16
    if t.dtype == torch.float32:
        return MOE_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_last_error() -> str:
    return _lib.moe_last_error().decode()


def moe_abi_version() -> int:
    return _lib.moe_abi_version()


def moe_router_workspace_bytes(T, H, E, dt) -> int:
    return _lib.moe_router_workspace_bytes(T, H, E, dt)


def moe_router_logits(x, dt, wg, bias, T, H, E, logits, ws=None, ws_bytes=0, stream=None):
    _call("moe_router_logits", addr(x), dt, addr(wg), addr(bias), T, H, E, addr(logits),
          addr(ws), ws_bytes, _stream(stream))


def moe_router_logits_bwd(dlogits, x, dt, wg, T, H, E, dx, dwg, dbias=None, ws=None, ws_bytes=0,
                          stream=None, flags=0):
    _call("moe_router_logits_bwd", addr(dlogits), addr(x), dt, addr(wg), T, H, E, addr(dx),
          addr(dwg), addr(dbias), flags, addr(ws), ws_bytes, _stream(stream))


def moe_route(logits, T, E, k, idx, gate, stream=None):
    _call("moe_route", addr(logits), T, E, k, addr(idx), addr(gate), _stream(stream))


def moe_route_bwd(logits, idx, dgate, T, E, k, dlogits, stream=None):
    _call("moe_route_bwd", addr(logits), addr(idx), addr(dgate), T, E, k, addr(dlogits),
          _stream(stream))


def moe_permute_workspace_bytes(T, E, k) -> int:
    return _lib.moe_permute_workspace_bytes(T, E, k)


def moe_permute(x, dt, idx, T, H, E, k, xp, counts, offsets, row_id_map, src_token, ws,
                ws_bytes, stream=None):
    _call("moe_permute", addr(x), dt, addr(idx), T, H, E, k, addr(xp), addr(counts),
          addr(offsets), addr(row_id_map), addr(src_token), addr(ws), ws_bytes, _stream(stream))


def moe_permute_noalloc_max_scratch_bytes() -> int:
    return _lib.moe_permute_noalloc_max_scratch_bytes()


def moe_permute_noalloc(x, dt, idx, T, H, E, k, xp, counts, offsets, row_id_map, src_token,
                        stream=None):
    _call("moe_permute_noalloc", addr(x), dt, addr(idx), T, H, E, k, addr(xp), addr(counts),
          addr(offsets), addr(row_id_map), addr(src_token), _stream(stream))


def moe_load_stats(counts, E, experts_per_group, load, cv, group_counts, stream=None):
    _call("moe_load_stats", addr(counts), E, experts_per_group, addr(load), addr(cv),
          addr(group_counts), _stream(stream))


def moe_permute_capacity(x, dt, idx, T, H, E, k, C, xp, counts, offsets, row_id_map,
                         src_token, ws, ws_bytes, stream=None):
    _call("moe_permute_capacity", addr(x), dt, addr(idx), T, H, E, k, C, addr(xp), addr(counts),
          addr(offsets), addr(row_id_map), addr(src_token), addr(ws), ws_bytes, _stream(stream))


def moe_clear_empty_rows(src_token, R, dt, H, buf, stream=None):
    _call("moe_clear_empty_rows", addr(src_token), R, dt, H, addr(buf), _stream(stream))


def moe_permute_bwd(dxp, row_id_map, dt, T, H, k, R, add0, add1, dx, stream=None):
    _call("moe_permute_bwd", addr(dxp), addr(row_id_map), dt, T, H, k, R, addr(add0), addr(add1),
          addr(dx), _stream(stream))


def moe_unpermute_combine(yp, row_id_map, gate, y_shared, dt, T, H, k, R, y, stream=None):
    _call("moe_unpermute_combine", addr(yp), addr(row_id_map), addr(gate), addr(y_shared), dt,
          T, H, k, R, addr(y), _stream(stream))


def moe_unpermute_combine_bwd(dy, yp, row_id_map, gate, dt, T, H, k, R, dyp, dgate, stream=None):
    _call("moe_unpermute_combine_bwd", addr(dy), addr(yp), addr(row_id_map), addr(gate), dt, T,
          H, k, R, addr(dyp), addr(dgate), _stream(stream))


def shared_expert(T=0, **tensors) -> SharedExpert:
    s = SharedExpert()
    s.T = T
    for k, v in tensors.items():
        setattr(s, k, addr(v))
    return s


def _sh(sh):
    return ctypes.byref(sh) if sh is not None else None


def moe_gmm_workspace_bytes() -> int:
    return _lib.moe_gmm_workspace_bytes()


def moe_grouped_gemm_fwd(xp, offsets, g0, G, R, dt, H, I, w13, w2, h13, act, yp, shared=None,
                         ws=None, ws_bytes=0, stream=None):
    _call("moe_grouped_gemm_fwd", addr(xp), addr(offsets), g0, G, R, dt, H, I, addr(w13),
          addr(w2), addr(h13), addr(act), addr(yp), _sh(shared), addr(ws), ws_bytes,
          _stream(stream))


def moe_grouped_gemm_bwd_dx(dyp, offsets, g0, G, R, dt, H, I, w13, w2, h13, dh13, dxp,
                            shared=None, ws=None, ws_bytes=0, stream=None):
    _call("moe_grouped_gemm_bwd_dx", addr(dyp), addr(offsets), g0, G, R, dt, H, I, addr(w13),
          addr(w2), addr(h13), addr(dh13), addr(dxp), _sh(shared), addr(ws), ws_bytes,
          _stream(stream))


def moe_grouped_gemm_bwd_dw(xp, act, dyp, dh13, offsets, g0, G, R, dt, H, I, dw13, dw2,
                            shared=None, ws=None, ws_bytes=0, stream=None):
    _call("moe_grouped_gemm_bwd_dw", addr(xp), addr(act), addr(dyp), addr(dh13), addr(offsets),
          g0, G, R, dt, H, I, addr(dw13), addr(dw2), _sh(shared), addr(ws), ws_bytes,
          _stream(stream))


def moe_grouped_gemm_bwd(xp, act, dyp, offsets, g0, G, R, dt, H, I, w13, w2, h13, dh13, dxp,
                         dw13, dw2, shared=None, ws=None, ws_bytes=0, stream=None):
    _call("moe_grouped_gemm_bwd", addr(xp), addr(act), addr(dyp), addr(offsets), g0, G, R, dt, H,
          I, addr(w13), addr(w2), addr(h13), addr(dh13), addr(dxp), addr(dw13), addr(dw2),
          _sh(shared), addr(ws), ws_bytes, _stream(stream))


def moe_grouped_gemm_fwd_gather(x, src_token, T, offsets, g0, G, R, dt, H, I, w13, w2, h13, act,
                                yp, shared=None, ws=None, ws_bytes=0, stream=None):
    _call("moe_grouped_gemm_fwd_gather", addr(x), addr(src_token), T, addr(offsets), g0, G, R,
          dt, H, I, addr(w13), addr(w2), addr(h13), addr(act), addr(yp), _sh(shared), addr(ws),
          ws_bytes, _stream(stream))


def moe_grouped_gemm_bwd_dw_recompute(x, src_token, T, h13, act, dyp, dh13, offsets, g0, G, R,
                                      dt, H, I, dw13, dw2, shared=None, ws=None, ws_bytes=0,
                                      stream=None):
    _call("moe_grouped_gemm_bwd_dw_recompute", addr(x), addr(src_token), T, addr(h13),
          addr(act), addr(dyp), addr(dh13), addr(offsets), g0, G, R, dt, H, I, addr(dw13),
          addr(dw2), _sh(shared), addr(ws), ws_bytes, _stream(stream))
