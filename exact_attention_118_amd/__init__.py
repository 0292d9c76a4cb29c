"""MI355X (gfx950) fused scaled-dot-product attention: Python binding of libfa.

The binding only marshals arguments: every step of the computation runs in the
HIP kernels of ``libfa.so`` (built in-tree from ``csrc/`` by ``build.py``).
torch is used for device memory and the current stream.  There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "FAError", "load_library", "lib_path", "fa_fwd", "fa_bwd", "fa_fwd_bias", "fa_bwd_bias",
    "fa_fwd_ex", "fa_bwd_ex", "fa_bias_tile_map", "fa_bwd_noalloc", "bwd_noalloc_max_rows",
    "forward", "backward",
    "fwd_workspace_size", "bwd_workspace_size", "bwd_stores_ds", "fwd_num_splits",
    "status_string", "version",
    "FA_OK", "FA_ERR_NULL", "FA_ERR_SHAPE", "FA_ERR_UNSUPPORTED", "FA_ERR_ALIGN",
    "FA_ERR_WORKSPACE", "FA_ERR_HIP", "FA_BF16", "FA_FP32", "FA_FP16", "EXPORTED_SYMBOLS",
    "FA_BWD_PREPROCESS", "FA_BWD_DKDV", "FA_BWD_DQ", "FA_BWD_ALL",
]

FA_OK, FA_ERR_NULL, FA_ERR_SHAPE, FA_ERR_UNSUPPORTED, FA_ERR_ALIGN, FA_ERR_WORKSPACE, FA_ERR_HIP = range(7)
FA_BF16, FA_FP32, FA_FP16 = 0, 1, 2

FA_BWD_PREPROCESS, FA_BWD_DKDV, FA_BWD_DQ, FA_BWD_ALL = 1, 2, 4, 7

EXPORTED_SYMBOLS = ("fa_fwd", "fa_bwd", "fa_bwd_stages", "fa_fwd_bias", "fa_bwd_bias",
                    "fa_fwd_ex", "fa_bwd_ex", "fa_bias_tile_map", "fa_bias_tile_map_size",
                    "fa_fwd_workspace_size", "fa_bwd_workspace_size", "fa_bwd_stores_ds",
                    "fa_fwd_num_splits",
                    "fa_status_string", "fa_version", "fa_bwd_noalloc", "fa_bwd_noalloc_max_rows")

_LIB = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")


def load_library():
    """Load libfa.so (built by ``build.py``) and declare its C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with exact_attention_118_amd.build.build()")
    lib = ctypes.CDLL(path)
    vp, sz, i, f = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp, sz, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_stages.argtypes = lib.fa_bwd.argtypes + [i]
    lib.fa_bwd_stages.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc_max_rows.argtypes = []
    lib.fa_bwd_noalloc_max_rows.restype = sz
    ll = ctypes.c_longlong
    lib.fa_fwd_bias.argtypes = [vp, vp, vp, vp, ll, ll, ll, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_bias.restype = i
    lib.fa_bwd_bias.argtypes = [vp, vp, vp, vp, ll, ll, ll, vp, vp, vp, vp, vp, vp, i, i, i, i, i,
                                f, i, i, vp, sz, vp]
    lib.fa_bwd_bias.restype = i
    ull, u = ctypes.c_ulonglong, ctypes.c_uint
    lib.fa_fwd_ex.argtypes = [vp, vp, vp, vp, ll, ll, ll, vp, sz, f, ull, u, vp, vp, i, i, i, i, i,
                              f, i, i, vp]
    lib.fa_fwd_ex.restype = i
    lib.fa_bwd_ex.argtypes = [vp, vp, vp, vp, ll, ll, ll, vp, sz, f, ull, u, vp, vp, vp, vp, vp, vp,
                              i, i, i, i, i, f, i, i, vp, sz, vp]
    lib.fa_bwd_ex.restype = i
    lib.fa_bias_tile_map_size.argtypes = [ll, ll, i, i, i, i]
    lib.fa_bias_tile_map_size.restype = sz
    lib.fa_bias_tile_map.argtypes = [vp, ll, ll, ll, i, i, i, i, i, vp, sz, vp]
    lib.fa_bias_tile_map.restype = i
    lib.fa_fwd_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_fwd_workspace_size.restype = sz
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd_stores_ds.argtypes = [i, i, i, i, i, i, i]
    lib.fa_bwd_stores_ds.restype = i
    lib.fa_fwd_num_splits.argtypes = [i, i, i, i, i, i, i]
    lib.fa_fwd_num_splits.restype = i
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def version() -> int:
    return load_library().fa_version()


# --------------------------------------------------------------------------- torch helpers

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_FP16
    if t.dtype == torch.float32:
        return FA_FP32
    raise TypeError(f"unsupported dtype {t.dtype}; libfa takes bfloat16, float16 or float32")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    """The torch stream a call is enqueued on: `stream`, else the current one."""
    return stream if stream is not None else _torch().cuda.current_stream(device)


def _stream_handle(device, stream):
    return ctypes.c_void_p(_stream(device, stream).cuda_stream)


def _check_tensor(name, t, shape, dtype, device):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd_workspace_size(B, H, Nq, Nk, d, dtype_code, num_splits=0) -> int:
    return load_library().fa_fwd_workspace_size(B, H, Nq, Nk, d, dtype_code, num_splits)


def bwd_workspace_size(B, H, Nq, Nk, d, dtype_code) -> int:
    return load_library().fa_bwd_workspace_size(B, H, Nq, Nk, d, dtype_code)


def bwd_stores_ds(B, H, Nq, Nk, d, causal, dtype_code) -> bool:
    """Whether fa_bwd with these arguments stores dS and forms dQ from it."""
    return bool(load_library().fa_bwd_stores_ds(B, H, Nq, Nk, d, int(bool(causal)), dtype_code))


def fwd_num_splits(B, H, Nq, Nk, d, dtype_code, num_splits=0) -> int:
    return load_library().fa_fwd_num_splits(B, H, Nq, Nk, d, dtype_code, num_splits)


def _alloc_workspace(nbytes, device, stream):
    """A workspace for a call enqueued on `stream` (None: the current stream).

    The block is allocated on that stream, so torch's caching allocator hands
    it to no other stream's allocation after it is freed here, while the
    call's kernels may still be using it."""
    torch = _torch()
    if nbytes == 0:
        return None
    with torch.cuda.stream(_stream(device, stream)):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _tile_map_arg(lib, tile_map, bias, sb, sh, B, H, Nq, Nk, device):
    """(pointer, bytes) of a tile map after the checks that keep the kernels
    inside it: a contiguous uint8 GPU tensor on the inputs' device holding at
    least fa_bias_tile_map_size() bytes for this bias geometry."""
    if tile_map is None:
        return None, 0
    torch = _torch()
    if bias is None:
        raise ValueError("tile_map needs the bias it was built from")
    if not tile_map.is_cuda or tile_map.device != device:
        raise ValueError(f"tile_map must be a GPU tensor on {device}")
    if tile_map.dtype != torch.uint8:
        raise ValueError(f"tile_map has dtype {tile_map.dtype}, expected torch.uint8")
    if not tile_map.is_contiguous():
        raise ValueError("tile_map must be contiguous")
    need = lib.fa_bias_tile_map_size(sb, sh, B, H, Nq, Nk)
    if tile_map.numel() < need:
        raise ValueError(f"tile_map holds {tile_map.numel()} bytes; this bias needs {need}")
    return _ptr(tile_map), tile_map.numel()


def fa_fwd(Q, K, V, O, L, scale, causal, num_splits=0, workspace=None, stream=None):
    """Call ``fa_fwd`` on existing tensors (O and L are written in place)."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    _check_tensor("Q", Q, (B, H, Nq, d), Q.dtype, dev)
    _check_tensor("K", K, (B, H, Nk, d), Q.dtype, dev)
    _check_tensor("V", V, (B, H, Nk, d), Q.dtype, dev)
    _check_tensor("O", O, (B, H, Nq, d), Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    code = _dtype_code(Q)
    need = lib.fa_fwd_workspace_size(B, H, Nq, Nk, d, code, num_splits)
    if workspace is None:
        workspace = _alloc_workspace(need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fa_fwd(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), B, H, Nq, Nk, d, float(scale),
                    int(bool(causal)), code, int(num_splits), _ptr(workspace), ws_bytes,
                    _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return O, L


def fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, scale, causal, workspace=None, stream=None,
           stages=FA_BWD_ALL):
    """Call ``fa_bwd`` (or ``fa_bwd_stages`` for a partial stage mask) on
    existing tensors (dQ, dK, dV are overwritten)."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    for name, t, shp in (("Q", Q, (B, H, Nq, d)), ("K", K, (B, H, Nk, d)), ("V", V, (B, H, Nk, d)),
                         ("O", O, (B, H, Nq, d)), ("dO", dO, (B, H, Nq, d)),
                         ("dQ", dQ, (B, H, Nq, d)), ("dK", dK, (B, H, Nk, d)),
                         ("dV", dV, (B, H, Nk, d))):
        _check_tensor(name, t, shp, Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    code = _dtype_code(Q)
    need = lib.fa_bwd_workspace_size(B, H, Nq, Nk, d, code)
    if workspace is None:
        workspace = _alloc_workspace(need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV),
            B, H, Nq, Nk, d, float(scale), int(bool(causal)), code, _ptr(workspace), ws_bytes,
            _stream_handle(dev, stream))
    if stages == FA_BWD_ALL:
        st = lib.fa_bwd(*args)
    else:
        st = lib.fa_bwd_stages(*args, int(stages))
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dQ, dK, dV


def bwd_noalloc_max_rows() -> int:
    return load_library().fa_bwd_noalloc_max_rows()


def fa_bwd_noalloc(Q, K, V, O, L, dO, dQ, dK, dV, scale, causal, stream=None):
    """Call ``fa_bwd_noalloc``: ``fa_bwd`` with the library's own scratch
    array instead of a workspace (nothing is allocated; calls that overlap on
    one GPU race)."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    for name, t, shp in (("Q", Q, (B, H, Nq, d)), ("K", K, (B, H, Nk, d)), ("V", V, (B, H, Nk, d)),
                         ("O", O, (B, H, Nq, d)), ("dO", dO, (B, H, Nq, d)),
                         ("dQ", dQ, (B, H, Nq, d)), ("dK", dK, (B, H, Nk, d)),
                         ("dV", dV, (B, H, Nk, d))):
        _check_tensor(name, t, shp, Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    st = lib.fa_bwd_noalloc(_ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(L), _ptr(dO), _ptr(dQ),
                            _ptr(dK), _ptr(dV), B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                            _dtype_code(Q), _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_noalloc")
    return dQ, dK, dV


def _bias_strides(bias, B, H, Nq, Nk, dtype, device):
    """Element strides (sb, sh, sq) of a bias viewable as [B or 1, H or 1, Nq, Nk]
    whose last dim is contiguous; broadcast dims (size 1) get stride 0."""
    if not bias.is_cuda or bias.device != device:
        raise ValueError(f"bias must be a GPU tensor on {device}")
    if bias.dtype != dtype:
        raise ValueError(f"bias has dtype {bias.dtype}, expected {dtype}")
    if bias.dim() != 4 or tuple(bias.shape[2:]) != (Nq, Nk) or bias.shape[0] not in (1, B) \
            or bias.shape[1] not in (1, H):
        raise ValueError(f"bias has shape {tuple(bias.shape)}, expected [B or 1, H or 1, {Nq}, {Nk}]")
    if bias.stride(3) != 1:
        raise ValueError("bias must be contiguous along keys")
    sb = 0 if bias.shape[0] == 1 else bias.stride(0)
    sh = 0 if bias.shape[1] == 1 else bias.stride(1)
    return sb, sh, bias.stride(2)


def fa_fwd_bias(Q, K, V, bias, O, L, scale, causal, stream=None):
    """Call ``fa_fwd_bias``: attention with an additive bias [B or 1, H or 1, Nq, Nk]."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    _check_tensor("Q", Q, (B, H, Nq, d), Q.dtype, dev)
    _check_tensor("K", K, (B, H, Nk, d), Q.dtype, dev)
    _check_tensor("V", V, (B, H, Nk, d), Q.dtype, dev)
    _check_tensor("O", O, (B, H, Nq, d), Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    sb, sh, sq = _bias_strides(bias, B, H, Nq, Nk, Q.dtype, dev)
    st = lib.fa_fwd_bias(_ptr(Q), _ptr(K), _ptr(V), _ptr(bias), sb, sh, sq, _ptr(O), _ptr(L), B, H,
                         Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(Q),
                         _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_bias")
    return O, L


def fa_bwd_bias(Q, K, V, bias, O, L, dO, dQ, dK, dV, scale, causal, workspace=None, stream=None):
    """Call ``fa_bwd_bias`` (dQ, dK, dV overwritten; no gradient for the bias)."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    for name, t, shp in (("Q", Q, (B, H, Nq, d)), ("K", K, (B, H, Nk, d)), ("V", V, (B, H, Nk, d)),
                         ("O", O, (B, H, Nq, d)), ("dO", dO, (B, H, Nq, d)),
                         ("dQ", dQ, (B, H, Nq, d)), ("dK", dK, (B, H, Nk, d)),
                         ("dV", dV, (B, H, Nk, d))):
        _check_tensor(name, t, shp, Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    sb, sh, sq = _bias_strides(bias, B, H, Nq, Nk, Q.dtype, dev)
    code = _dtype_code(Q)
    need = lib.fa_bwd_workspace_size(B, H, Nq, Nk, d, code)
    if workspace is None:
        workspace = _alloc_workspace(need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fa_bwd_bias(_ptr(Q), _ptr(K), _ptr(V), _ptr(bias), sb, sh, sq, _ptr(O), _ptr(L),
                         _ptr(dO), _ptr(dQ), _ptr(dK), _ptr(dV), B, H, Nq, Nk, d, float(scale),
                         int(bool(causal)), code, _ptr(workspace), ws_bytes,
                         _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_bias")
    return dQ, dK, dV


def _check_dropout(dropout_p, seed, offset):
    if not (0.0 <= float(dropout_p) < 1.0):
        raise ValueError(f"dropout_p must lie in [0, 1), got {dropout_p}")
    if not (0 <= int(seed) < 2**64) or not (0 <= int(offset) < 2**32):
        raise ValueError("seed must fit 64 bits and offset 32 bits")


def fa_bias_tile_map(bias, B, H, Nq, Nk, tile_map=None, stream=None):
    """Call ``fa_bias_tile_map``: the uint8 map of the bias's 128 x 64 tiles
    that hold an entry above -inf (allocated when not given)."""
    lib = load_library()
    torch = _torch()
    dev = bias.device
    if bias.dtype not in (torch.bfloat16, torch.float16):
        raise ValueError("tile maps are built for bf16 or fp16 biases")
    sb, sh, sq = _bias_strides(bias, B, H, Nq, Nk, bias.dtype, dev)
    n = lib.fa_bias_tile_map_size(sb, sh, B, H, Nq, Nk)
    if tile_map is None:
        with torch.cuda.stream(_stream(dev, stream)):
            tile_map = torch.empty(max(n, 1), dtype=torch.uint8, device=dev)
    elif (not tile_map.is_cuda or tile_map.device != dev or tile_map.dtype != torch.uint8
          or not tile_map.is_contiguous()):
        raise ValueError(f"tile_map must be a contiguous uint8 GPU tensor on {dev}")
    st = lib.fa_bias_tile_map(_ptr(bias), sb, sh, sq, B, H, Nq, Nk, _dtype_code(bias),
                              _ptr(tile_map), tile_map.numel(), _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_bias_tile_map")
    return tile_map


def fa_fwd_ex(Q, K, V, O, L, scale, causal, bias=None, dropout_p=0.0, seed=0, offset=0,
              stream=None, tile_map=None):
    """Call ``fa_fwd_ex``: optional additive bias and optional dropout on P."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    _check_tensor("Q", Q, (B, H, Nq, d), Q.dtype, dev)
    _check_tensor("K", K, (B, H, Nk, d), Q.dtype, dev)
    _check_tensor("V", V, (B, H, Nk, d), Q.dtype, dev)
    _check_tensor("O", O, (B, H, Nq, d), Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    _check_dropout(dropout_p, seed, offset)
    sb, sh, sq = (0, 0, 0) if bias is None else _bias_strides(bias, B, H, Nq, Nk, Q.dtype, dev)
    map_ptr, map_bytes = _tile_map_arg(lib, tile_map, bias, sb, sh, B, H, Nq, Nk, dev)
    st = lib.fa_fwd_ex(_ptr(Q), _ptr(K), _ptr(V), None if bias is None else _ptr(bias), sb, sh, sq,
                       map_ptr, map_bytes, float(dropout_p), int(seed), int(offset), _ptr(O), _ptr(L), B, H, Nq, Nk, d,
                       float(scale), int(bool(causal)), _dtype_code(Q), _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_fwd_ex")
    return O, L


def fa_bwd_ex(Q, K, V, O, L, dO, dQ, dK, dV, scale, causal, bias=None, dropout_p=0.0, seed=0,
              offset=0, workspace=None, stream=None, tile_map=None):
    """Call ``fa_bwd_ex`` with the bias and dropout arguments the forward pass used."""
    lib = load_library()
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dev = Q.device
    for name, t, shp in (("Q", Q, (B, H, Nq, d)), ("K", K, (B, H, Nk, d)), ("V", V, (B, H, Nk, d)),
                         ("O", O, (B, H, Nq, d)), ("dO", dO, (B, H, Nq, d)),
                         ("dQ", dQ, (B, H, Nq, d)), ("dK", dK, (B, H, Nk, d)),
                         ("dV", dV, (B, H, Nk, d))):
        _check_tensor(name, t, shp, Q.dtype, dev)
    _check_tensor("L", L, (B, H, Nq), _torch().float32, dev)
    _check_dropout(dropout_p, seed, offset)
    sb, sh, sq = (0, 0, 0) if bias is None else _bias_strides(bias, B, H, Nq, Nk, Q.dtype, dev)
    map_ptr, map_bytes = _tile_map_arg(lib, tile_map, bias, sb, sh, B, H, Nq, Nk, dev)
    code = _dtype_code(Q)
    need = lib.fa_bwd_workspace_size(B, H, Nq, Nk, d, code)
    if workspace is None:
        workspace = _alloc_workspace(need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.fa_bwd_ex(_ptr(Q), _ptr(K), _ptr(V), None if bias is None else _ptr(bias), sb, sh, sq,
                       map_ptr, map_bytes, float(dropout_p), int(seed), int(offset), _ptr(O), _ptr(L), _ptr(dO),
                       _ptr(dQ), _ptr(dK), _ptr(dV), B, H, Nq, Nk, d, float(scale),
                       int(bool(causal)), code, _ptr(workspace), ws_bytes,
                       _stream_handle(dev, stream))
    if st != FA_OK:
        raise FAError(st, "fa_bwd_ex")
    return dQ, dK, dV


def forward(Q, K, V, scale=None, causal=False, num_splits=0, stream=None, bias=None,
            dropout_p=0.0, seed=0, offset=0, tile_map=None):
    """Allocate O, L and run ``fa_fwd`` (``fa_fwd_bias`` with a bias, ``fa_fwd_ex``
    with dropout).  Returns (O, L)."""
    torch = _torch()
    B, H, Nq, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    O = torch.empty_like(Q)
    L = torch.empty((B, H, Nq), dtype=torch.float32, device=Q.device)
    if dropout_p or tile_map is not None:
        return fa_fwd_ex(Q, K, V, O, L, scale, causal, bias=bias, dropout_p=dropout_p, seed=seed,
                         offset=offset, stream=stream, tile_map=tile_map)
    if bias is not None:
        return fa_fwd_bias(Q, K, V, bias, O, L, scale, causal, stream=stream)
    return fa_fwd(Q, K, V, O, L, scale, causal, num_splits=num_splits, stream=stream)


def backward(Q, K, V, O, L, dO, scale=None, causal=False, stream=None, bias=None, dropout_p=0.0,
             seed=0, offset=0, tile_map=None):
    """Allocate dQ, dK, dV and run ``fa_bwd`` (or the bias / dropout entry point
    matching the forward call).  Returns (dQ, dK, dV)."""
    torch = _torch()
    d = Q.shape[-1]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dQ = torch.empty_like(Q)
    dK = torch.empty_like(K)
    dV = torch.empty_like(V)
    if dropout_p or tile_map is not None:
        return fa_bwd_ex(Q, K, V, O, L, dO, dQ, dK, dV, scale, causal, bias=bias,
                         dropout_p=dropout_p, seed=seed, offset=offset, stream=stream,
                         tile_map=tile_map)
    if bias is not None:
        return fa_bwd_bias(Q, K, V, bias, O, L, dO, dQ, dK, dV, scale, causal, stream=stream)
    return fa_bwd(Q, K, V, O, L, dO, dQ, dK, dV, scale, causal, stream=stream)
