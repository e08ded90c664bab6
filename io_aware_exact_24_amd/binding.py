"""ctypes binding of libfa.so with the C ABI's entry-point names.

Argument marshalling only: torch tensors are checked for shape, dtype, device
and layout, then passed as raw device pointers (and, for the strided entry
points, their element strides) together with the HIP stream handle of torch's
current stream.  All compute happens in the library's kernels.  If libfa.so
is missing the first call raises; there is no fallback.
"""

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_NAME = "libfa.so"

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
FA_F32, FA_BF16, FA_F16 = 0, 1, 2

EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_status_string", "fa_bwd_preprocess",
           "fa_bwd_dkdv", "fa_bwd_dq", "fa_fwd_split", "fa_fwd_split_workspace_size",
           "fa_bwd_noalloc", "fa_fwd_strided", "fa_bwd_strided", "fa_fwd_varlen", "fa_bwd_varlen",
           "fa_bwd_varlen_workspace_size", "fa_bwd_split", "fa_bwd_split_workspace_size",
           "fa_fwd_varlen_device", "fa_bwd_varlen_device", "fa_bwd_varlen_device_workspace_size")
FA_MAX_SPLITS = 64
FA_NOALLOC_SCRATCH_BYTES = 32 << 20

_lib = None


class FaStrides(ctypes.Structure):
    """fa_strides: element strides (batch, head, row) of a [B, H, N, d] tensor."""
    _fields_ = [("batch", ctypes.c_int64), ("head", ctypes.c_int64), ("row", ctypes.c_int64)]


class FaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {fa_status_string(status)} (status {status})")


def library_path():
    return os.path.join(PKG, LIB_NAME)


def load_library():
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise OSError(f"{path} is missing; build it with `python -m io_aware_exact_24_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, f, u64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_uint64, ctypes.c_size_t
    lib.fa_fwd.restype = i
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f, u64, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f, u64,
                           vp, sz, vp]
    lib.fa_fwd_split.restype = i
    lib.fa_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f, u64, i, vp, sz, vp]
    lib.fa_fwd_split_workspace_size.restype = sz
    lib.fa_fwd_split_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_split.restype = i
    lib.fa_bwd_split.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f,
                                 u64, i, vp, sz, vp]
    lib.fa_bwd_split_workspace_size.restype = sz
    lib.fa_bwd_split_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_bwd_workspace_size.argtypes = [i, i, i, i, i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_status_string.argtypes = [i]
    lib.fa_bwd_preprocess.restype = i
    lib.fa_bwd_preprocess.argtypes = [vp, vp, vp, i, i, i, i, i, vp, sz, vp]
    lib.fa_bwd_dkdv.restype = i
    lib.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f, u64, vp, sz, vp]
    lib.fa_bwd_dq.restype = i
    lib.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f, u64, vp, sz,
                              vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp, f,
                                   u64, vp]
    sp = ctypes.POINTER(FaStrides)
    lib.fa_fwd_strided.restype = i
    lib.fa_fwd_strided.argtypes = [vp, vp, vp, vp, vp, sp, i, i, i, i, i, f, i, vp, f, u64, vp]
    ip = ctypes.POINTER(ctypes.c_int32)
    lib.fa_fwd_varlen.restype = i
    lib.fa_fwd_varlen.argtypes = [vp, vp, vp, vp, vp, sp, ip, i, i, i, i, f, i, f, u64, vp]
    lib.fa_bwd_varlen_workspace_size.restype = sz
    lib.fa_bwd_varlen_workspace_size.argtypes = [ip, i, i, i, i]
    lib.fa_bwd_varlen.restype = i
    lib.fa_bwd_varlen.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sp, ip, i, i, i, i, f, i, f, u64,
                                  vp, sz, vp]
    lib.fa_bwd_strided.restype = i
    lib.fa_bwd_strided.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sp, i, i, i, i, i, f, i, vp,
                                   f, u64, vp, sz, vp]
    lib.fa_fwd_varlen_device.restype = i
    lib.fa_fwd_varlen_device.argtypes = [vp, vp, vp, vp, vp, sp, vp, i, i, i, i, i, i, f, i, f, u64,
                                         vp]
    lib.fa_bwd_varlen_device_workspace_size.restype = sz
    lib.fa_bwd_varlen_device_workspace_size.argtypes = [i, i, i, i]
    lib.fa_bwd_varlen_device.restype = i
    lib.fa_bwd_varlen_device.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, sp, vp, i, i, i, i, i,
                                         i, f, i, f, u64, vp, sz, vp]
    _lib = lib
    return lib


def fa_status_string(status):
    return load_library().fa_status_string(int(status)).decode()


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t, shape, dtype, device, name):
    if t.shape != shape or t.dtype != dtype or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name}: expected contiguous {tuple(shape)} {dtype} on {device}, got "
                         f"{tuple(t.shape)} {t.dtype} on {t.device} (contiguous={t.is_contiguous()})")


def _check_view(t, shape, dtype, device, name):
    """A [B, H, N, d] tensor of any strides whose last dimension is contiguous
    (the library checks the strides themselves)."""
    if t.shape != shape or t.dtype != dtype or t.device != device or (t.shape[-1] > 1 and
                                                                         t.stride(-1) != 1):
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype} on {device} with a contiguous "
                         f"last dimension, got {tuple(t.shape)} {t.dtype} on {t.device} strides "
                         f"{t.stride()}")


def _strides(tensors):
    arr = (FaStrides * len(tensors))()
    for a, t in zip(arr, tensors):
        a.batch, a.head, a.row = t.stride(0), t.stride(1), t.stride(2)
    return arr


def kernel_layout_ok(t):
    """True when the strided entry points can read or write t in place: last
    dimension contiguous, 16-byte aligned base and strides, rows at least d
    elements apart (fa_strides in include/fa.h)."""
    if t.dim() != 4 or t.stride(-1) != 1 or t.data_ptr() % 16 != 0:
        return False
    unit = 16 // t.element_size()
    d = t.shape[-1]
    return all(s >= 0 and s % unit == 0 for s in t.stride()[:3]) and t.stride(2) >= d


def _stream(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _key_lens(key_lens, B, device):
    import torch

    if key_lens is None:
        return None
    _check(key_lens, (B,), torch.int32, device, "key_lens")
    return key_lens


def fa_fwd(q, k, v, o, lse, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
           stream=None):
    """Enqueue the forward pass; o and lse are written.  See include/fa.h."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check(t, q.shape, q.dtype, q.device, name)
    _check(q, q.shape, q.dtype, q.device, "q")
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    st = lib.fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _dtype_code(q),
                    float(scale), int(bool(causal)), _ptr(kl), float(dropout_p), int(seed),
                    _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")


def fa_fwd_strided(q, k, v, o, lse, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
                   stream=None):
    """fa_fwd on [B, H, N, d] views of any strides (last dimension
    contiguous): each tensor's batch, head and row strides go to the library,
    nothing is copied."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_view(t, q.shape, q.dtype, q.device, name)
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    st = lib.fa_fwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _strides((q, k, v, o)),
                            B, H, N, d, _dtype_code(q), float(scale), int(bool(causal)), _ptr(kl),
                            float(dropout_p), int(seed), _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_strided")


def fa_fwd_split_workspace_size(B, H, N, d, num_splits, dtype_code=FA_BF16):
    return int(load_library().fa_fwd_split_workspace_size(B, H, N, d, dtype_code, num_splits))


def fa_fwd_split(q, k, v, o, lse, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
                 num_splits=2, workspace=None, stream=None):
    """Enqueue the split-KV forward (bf16); o and lse are written.  workspace: a
    uint8 device tensor of at least fa_fwd_split_workspace_size() bytes."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o)):
        _check(t, q.shape, q.dtype, q.device, name)
    _check(q, q.shape, q.dtype, q.device, "q")
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    if workspace is None:
        raise ValueError("fa_fwd_split needs a workspace tensor (see fa_fwd_split_workspace_size)")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.fa_fwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, _dtype_code(q),
                          float(scale), int(bool(causal)), _ptr(kl), float(dropout_p), int(seed),
                          int(num_splits), _ptr(workspace), ws_bytes, _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_split")


def forward_split(q, k, v, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0, num_splits=2,
                  stream=None):
    """Allocate O, LSE and the workspace with torch and call fa_fwd_split."""
    import torch

    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    nbytes = fa_fwd_split_workspace_size(B, H, N, d, num_splits, _dtype_code(q))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    fa_fwd_split(q, k, v, o, lse, scale, causal, key_lens, dropout_p, seed, num_splits, ws, stream)
    return o, lse


def fa_bwd_workspace_size(B, H, N, d, dtype_code=FA_BF16):
    return int(load_library().fa_bwd_workspace_size(B, H, N, d, dtype_code))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, scale, causal=False, key_lens=None,
           dropout_p=0.0, seed=0, workspace=None, stream=None):
    """Enqueue the backward pass; dq, dk, dv are written.  workspace: a uint8
    device tensor of at least fa_bwd_workspace_size() bytes."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, q.shape, q.dtype, q.device, name)
    _check(q, q.shape, q.dtype, q.device, "q")
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    if workspace is None:
        raise ValueError("fa_bwd needs a workspace tensor (see fa_bwd_workspace_size)")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                    _ptr(dv), B, H, N, d, _dtype_code(q), float(scale), int(bool(causal)), _ptr(kl),
                    float(dropout_p), int(seed), _ptr(workspace), ws_bytes,
                    _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")


def fa_bwd_split_workspace_size(B, H, N, d, num_splits, dtype_code=FA_BF16):
    return int(load_library().fa_bwd_split_workspace_size(B, H, N, d, dtype_code, num_splits))


def fa_bwd_split(q, k, v, o, dout, lse, dq, dk, dv, scale, causal=False, key_lens=None,
                 dropout_p=0.0, seed=0, num_splits=2, workspace=None, stream=None):
    """Enqueue the split backward (16-bit, contiguous); dq, dk, dv are written.
    workspace: a uint8 device tensor of at least fa_bwd_split_workspace_size()
    bytes."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, q.shape, q.dtype, q.device, name)
    _check(q, q.shape, q.dtype, q.device, "q")
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    if workspace is None:
        raise ValueError("fa_bwd_split needs a workspace tensor (see fa_bwd_split_workspace_size)")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.fa_bwd_split(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                          _ptr(dk), _ptr(dv), B, H, N, d, _dtype_code(q), float(scale),
                          int(bool(causal)), _ptr(kl), float(dropout_p), int(seed),
                          int(num_splits), _ptr(workspace), ws_bytes, _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_split")


def backward_split(q, k, v, o, dout, lse, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
                   num_splits=2, stream=None):
    """Allocate dQ, dK, dV and the workspace with torch and call fa_bwd_split."""
    import torch

    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa_bwd_split_workspace_size(B, H, N, d, num_splits, _dtype_code(q))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    fa_bwd_split(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, key_lens, dropout_p, seed,
                 num_splits, ws, stream)
    return dq, dk, dv


def fa_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, scale, causal=False, key_lens=None,
                   dropout_p=0.0, seed=0, workspace=None, stream=None):
    """fa_bwd on [B, H, N, d] views of any strides (last dimension
    contiguous); nothing is copied."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    ts = (q, k, v, o, dout, dq, dk, dv)
    for name, t in zip(("q", "k", "v", "o", "dout", "dq", "dk", "dv"), ts):
        _check_view(t, q.shape, q.dtype, q.device, name)
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    if workspace is None:
        raise ValueError("fa_bwd_strided needs a workspace tensor (see fa_bwd_workspace_size)")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.fa_bwd_strided(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), _strides(ts), B, H, N, d, _dtype_code(q),
                            float(scale), int(bool(causal)), _ptr(kl), float(dropout_p), int(seed),
                            _ptr(workspace), ws_bytes, _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_strided")


def _cu(cu_seqlens):
    """Host int32 array of the sequence offsets (a list, numpy array or CPU tensor)."""
    vals = [int(x) for x in (cu_seqlens.tolist() if hasattr(cu_seqlens, "tolist") else cu_seqlens)]
    return (ctypes.c_int32 * len(vals))(*vals), len(vals) - 1


def _packed_strides(tensors):
    arr = (FaStrides * len(tensors))()
    for a, t in zip(arr, tensors):
        a.batch, a.head, a.row = 0, t.stride(1), t.stride(0)
    return arr


def _check_packed(t, shape, dtype, device, name):
    if t.shape != shape or t.dtype != dtype or t.device != device or t.stride(-1) != 1:
        raise ValueError(f"{name}: expected {tuple(shape)} {dtype} on {device} with a contiguous "
                         f"last dimension, got {tuple(t.shape)} {t.dtype} on {t.device} strides "
                         f"{t.stride()}")


def fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, scale, causal=False, dropout_p=0.0, seed=0,
                  stream=None):
    """fa_fwd_varlen: packed [T, H, d] tensors (any token and head strides),
    sequence b = tokens [cu_seqlens[b], cu_seqlens[b+1]) (host offsets); lse:
    fp32 with H * T elements (sequence b's [H, len] block at H * cu_seqlens[b])."""
    import torch

    lib = load_library()
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_packed(t, q.shape, q.dtype, q.device, name)
    if lse.dtype != torch.float32 or lse.numel() != H * T or not lse.is_contiguous():
        raise ValueError("lse: expected a contiguous fp32 tensor of H * T elements")
    cu, n = _cu(cu_seqlens)
    if n < 1 or cu[n] != T:
        raise ValueError(f"cu_seqlens must end at T = {T}")
    st = lib.fa_fwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                           _packed_strides((q, k, v, o)), cu, n, H, d, _dtype_code(q), float(scale),
                           int(bool(causal)), float(dropout_p), int(seed), _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_varlen")


def fa_bwd_varlen_workspace_size(cu_seqlens, H, d, dtype_code=FA_BF16):
    cu, n = _cu(cu_seqlens)
    return int(load_library().fa_bwd_varlen_workspace_size(cu, n, H, d, dtype_code))


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, scale, causal=False, dropout_p=0.0,
                  seed=0, workspace=None, stream=None):
    """fa_bwd_varlen on packed [T, H, d] tensors (see fa_fwd_varlen)."""
    import torch

    lib = load_library()
    T, H, d = q.shape
    ts = (q, k, v, o, dout, dq, dk, dv)
    for name, t in zip(("q", "k", "v", "o", "dout", "dq", "dk", "dv"), ts):
        _check_packed(t, q.shape, q.dtype, q.device, name)
    if lse.dtype != torch.float32 or lse.numel() != H * T or not lse.is_contiguous():
        raise ValueError("lse: expected a contiguous fp32 tensor of H * T elements")
    cu, n = _cu(cu_seqlens)
    if n < 1 or cu[n] != T:
        raise ValueError(f"cu_seqlens must end at T = {T}")
    if workspace is None:
        raise ValueError("fa_bwd_varlen needs a workspace tensor (see fa_bwd_varlen_workspace_size)")
    ws_bytes = workspace.numel() * workspace.element_size()
    st = lib.fa_bwd_varlen(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                           _ptr(dk), _ptr(dv), _packed_strides(ts), cu, n, H, d, _dtype_code(q),
                           float(scale), int(bool(causal)), float(dropout_p), int(seed),
                           _ptr(workspace), ws_bytes, _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_varlen")


def forward_varlen(q, k, v, cu_seqlens, scale, causal=False, dropout_p=0.0, seed=0, stream=None):
    """Allocate O (in q's layout) and LSE and call fa_fwd_varlen."""
    import torch

    T, H, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(H * T, dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_seqlens, scale, causal, dropout_p, seed, stream)
    return o, lse


def backward_varlen(q, k, v, o, dout, lse, cu_seqlens, scale, causal=False, dropout_p=0.0, seed=0,
                    stream=None):
    """Allocate dQ, dK, dV and the workspace and call fa_bwd_varlen."""
    import torch

    T, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa_bwd_varlen_workspace_size(cu_seqlens, H, d, _dtype_code(q))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, scale, causal, dropout_p, seed, ws,
                  stream)
    return dq, dk, dv


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale, causal=False, key_lens=None,
                   dropout_p=0.0, seed=0, stream=None):
    """Enqueue the backward pass with the library's fixed device scratch instead
    of a workspace (no allocation anywhere); dq, dk, dv are written.  Calls
    that may overlap on one GPU race on that scratch."""
    import torch

    lib = load_library()
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(t, q.shape, q.dtype, q.device, name)
    _check(q, q.shape, q.dtype, q.device, "q")
    _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    st = lib.fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                            _ptr(dk), _ptr(dv), B, H, N, d, _dtype_code(q), float(scale),
                            int(bool(causal)), _ptr(kl), float(dropout_p), int(seed),
                            _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_noalloc")


def _bwd_common(q, tensors, lse, key_lens, workspace):
    import torch

    B, H, N, d = q.shape
    for name, t in tensors:
        _check(t, q.shape, q.dtype, q.device, name)
    if lse is not None:
        _check(lse, (B, H, N), torch.float32, q.device, "lse")
    kl = _key_lens(key_lens, B, q.device)
    if workspace is None:
        raise ValueError("the backward stages need a workspace tensor (see fa_bwd_workspace_size)")
    return B, H, N, d, kl, workspace.numel() * workspace.element_size()


def fa_bwd_preprocess(o, dout, lse, workspace, stream=None):
    """Enqueue the backward preprocessing (per-row D and LSE*log2e into the workspace)."""
    B, H, N, d, _, ws_bytes = _bwd_common(o, (("dout", dout),), lse, None, workspace)
    st = load_library().fa_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(lse), B, H, N, d,
                                          _dtype_code(o), _ptr(workspace), ws_bytes,
                                          _stream(stream, o.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_preprocess")


def fa_bwd_dkdv(q, k, v, dout, dk, dv, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
                workspace=None, stream=None):
    """Enqueue the dK/dV stage (after fa_bwd_dq or fa_bwd_preprocess filled the workspace)."""
    B, H, N, d, kl, ws_bytes = _bwd_common(
        q, (("k", k), ("v", v), ("dout", dout), ("dk", dk), ("dv", dv)), None, key_lens, workspace)
    st = load_library().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dk), _ptr(dv), B, H,
                                    N, d, _dtype_code(q), float(scale), int(bool(causal)), _ptr(kl),
                                    float(dropout_p), int(seed), _ptr(workspace), ws_bytes,
                                    _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dkdv")


def fa_bwd_dq(q, k, v, o, dout, lse, dq, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
              workspace=None, stream=None):
    """Enqueue the dQ stage; it also writes the per-row terms (D, LSE*log2e)
    into the workspace for fa_bwd_dkdv."""
    B, H, N, d, kl, ws_bytes = _bwd_common(
        q, (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq)), lse, key_lens, workspace)
    st = load_library().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                  _ptr(dq), B, H, N, d, _dtype_code(q), float(scale),
                                  int(bool(causal)), _ptr(kl), float(dropout_p), int(seed),
                                  _ptr(workspace), ws_bytes, _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_dq")


def forward(q, k, v, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0, stream=None):
    """Allocate O (in q's memory layout) and LSE with torch and call fa_fwd, or
    fa_fwd_strided when a tensor is not contiguous [B, H, N, d]."""
    import torch

    B, H, N, d = q.shape
    o = torch.empty_like(q)  # keeps q's strides for a dense q
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if all(t.is_contiguous() for t in (q, k, v, o)):
        fa_fwd(q, k, v, o, lse, scale, causal, key_lens, dropout_p, seed, stream)
    else:
        fa_fwd_strided(q, k, v, o, lse, scale, causal, key_lens, dropout_p, seed, stream)
    return o, lse


def backward(q, k, v, o, dout, lse, scale, causal=False, key_lens=None, dropout_p=0.0, seed=0,
             stream=None, workspace=None):
    """Allocate dQ, dK, dV (each in its input's memory layout; the workspace
    unless given) and call fa_bwd, or fa_bwd_strided when a tensor is not
    contiguous [B, H, N, d]."""
    import torch

    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if workspace is None:
        nbytes = fa_bwd_workspace_size(B, H, N, d, _dtype_code(q))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if all(t.is_contiguous() for t in (q, k, v, o, dout, dq, dk, dv)):
        fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, key_lens, dropout_p, seed,
               workspace, stream)
    else:
        fa_bwd_strided(q, k, v, o, dout, lse, dq, dk, dv, scale, causal, key_lens, dropout_p, seed,
                       workspace, stream)
    return dq, dk, dv


def _cu_device(cu_seqlens, device):
    """Device int32 offsets (a CUDA tensor is used as it is) and the sequence count."""
    import torch

    if isinstance(cu_seqlens, torch.Tensor) and cu_seqlens.is_cuda:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens: expected a contiguous int32 tensor")
        return cu_seqlens, cu_seqlens.numel() - 1
    t = torch.as_tensor(cu_seqlens, dtype=torch.int32).to(device)
    return t, t.numel() - 1


def fa_fwd_varlen_device(q, k, v, o, lse, cu_seqlens, max_len, scale, causal=False, dropout_p=0.0,
                         seed=0, stream=None):
    """fa_fwd_varlen_device: fa_fwd_varlen with the offsets on the device (one
    launch for every sequence); max_len >= the longest sequence."""
    import torch

    lib = load_library()
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_packed(t, q.shape, q.dtype, q.device, name)
    if lse.dtype != torch.float32 or lse.numel() != H * T or not lse.is_contiguous():
        raise ValueError("lse: expected a contiguous fp32 tensor of H * T elements")
    cu, n = _cu_device(cu_seqlens, q.device)
    st = lib.fa_fwd_varlen_device(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                  _packed_strides((q, k, v, o)), _ptr(cu), n, int(max_len), T, H, d,
                                  _dtype_code(q), float(scale), int(bool(causal)), float(dropout_p),
                                  int(seed), _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_varlen_device")


def fa_bwd_varlen_device_workspace_size(total_tokens, H, d, dtype_code=FA_BF16):
    return int(load_library().fa_bwd_varlen_device_workspace_size(total_tokens, H, d, dtype_code))


def fa_bwd_varlen_device(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, max_len, scale,
                         causal=False, dropout_p=0.0, seed=0, workspace=None, stream=None):
    """fa_bwd_varlen_device: fa_bwd_varlen with the offsets on the device."""
    lib = load_library()
    T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check_packed(t, q.shape, q.dtype, q.device, name)
    if workspace is None:
        raise ValueError("fa_bwd_varlen_device needs a workspace tensor")
    cu, n = _cu_device(cu_seqlens, q.device)
    st = lib.fa_bwd_varlen_device(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
                                  _ptr(dq), _ptr(dk), _ptr(dv),
                                  _packed_strides((q, k, v, o, dout, dq, dk, dv)), _ptr(cu), n,
                                  int(max_len), T, H, d, _dtype_code(q), float(scale),
                                  int(bool(causal)), float(dropout_p), int(seed), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(),
                                  _stream(stream, q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd_varlen_device")


def forward_varlen_device(q, k, v, cu_seqlens, max_len, scale, causal=False, dropout_p=0.0, seed=0,
                          stream=None):
    """Allocate O (in q's layout) and LSE and call fa_fwd_varlen_device."""
    import torch

    T, H, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty(H * T, dtype=torch.float32, device=q.device)
    fa_fwd_varlen_device(q, k, v, o, lse, cu_seqlens, max_len, scale, causal, dropout_p, seed,
                         stream)
    return o, lse


def backward_varlen_device(q, k, v, o, dout, lse, cu_seqlens, max_len, scale, causal=False,
                           dropout_p=0.0, seed=0, stream=None):
    """Allocate dQ, dK, dV and the workspace and call fa_bwd_varlen_device."""
    import torch

    T, H, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    nbytes = fa_bwd_varlen_device_workspace_size(T, H, d, _dtype_code(q))
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    fa_bwd_varlen_device(q, k, v, o, dout, lse, dq, dk, dv, cu_seqlens, max_len, scale, causal,
                         dropout_p, seed, ws, stream)
    return dq, dk, dv
