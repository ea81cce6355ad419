"""ctypes binding of libfa.so — argument marshalling only.

Each function has the name of the C entry point it calls (include/fa.h) and
takes torch tensors that already live on the GPU; torch supplies device
memory and the current stream, every step of the computation runs in the
HIP kernels. There is no fallback: if the library is missing the import of
the first call raises.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F32, FA_BF16 = 0, 1
MASK_CODES = {None: 0, "none": 0, "causal": 1, "local": 2}
STATUS_NAMES = {0: "FA_OK", 1: "FA_ERR_NULL", 2: "FA_ERR_SHAPE", 3: "FA_ERR_DTYPE",
                4: "FA_ERR_HEADDIM", 5: "FA_ERR_MASK", 6: "FA_ERR_SCALE", 7: "FA_ERR_ALIGN",
                8: "FA_ERR_WORKSPACE", 9: "FA_ERR_LAUNCH", 10: "FA_ERR_ALIAS",
                11: "FA_ERR_CONFIG"}
I32_MAX = 2 ** 31 - 1
EXPORTS = ("fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string")

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {fa_status_string(status)}")


def ensure_built():
    """Compile libfa.so (hipcc, gfx950) if it is not there yet; an existing
    library is used as it is. For the test suite, the smoke check and the
    bench; load() itself never builds and fails when the library is missing."""
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()


def load():
    """Load libfa.so (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise OSError(f"{LIB_PATH} is missing: build it with "
                      "`python -m exact_tiled_attention_fwd_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd.restype = i
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                           i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_fwd_tuned.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_tuned.restype = i
    lib.fa_bwd_tuned.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                 i, i, i, i, i, f, i, i, i, vp]
    lib.fa_bwd_tuned.restype = i
    lib.fa_bwd_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_status_string.argtypes = [i]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_fwd_standard_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_fwd_standard_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_standard.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                    i, i, i, i, i, f, i, i, vp]
    lib.fa_fwd_standard.restype = i
    lib.fa_bwd_standard_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_bwd_standard_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_bwd_standard.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp, vp, vp, vp,
                                    ctypes.c_size_t, i, i, i, i, i, f, vp]
    lib.fa_bwd_standard.restype = i
    lib.fa_fwd_keymajor_workspace_bytes.argtypes = [i, i, i, i, i]
    lib.fa_fwd_keymajor_workspace_bytes.restype = ctypes.c_size_t
    lib.fa_fwd_keymajor.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                    i, i, i, i, i, f, i, i, i, vp]
    lib.fa_fwd_keymajor.restype = i
    dp = ctypes.POINTER(ctypes.c_double)
    lib.fa_probe_mfma_bf16.argtypes = [i, vp, dp]
    lib.fa_probe_mfma_bf16.restype = i
    lib.fa_probe_copy.argtypes = [vp, vp, ctypes.c_size_t, i, vp, dp]
    lib.fa_probe_copy.restype = i
    _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float32:
        return FA_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _mask_code(mask) -> int:
    if mask not in MASK_CODES:
        raise ValueError(f"mask must be None, 'none', 'causal' or 'local', not {mask!r}")
    return MASK_CODES[mask]


def _window(window) -> int:
    """The band radius as the C int the library takes: radii past 2^31 - 1
    allow the same pairs as 2^31 - 1 (every |i - j| is below N), negative ones
    stay negative (the library rejects them under the band mask), so no value
    wraps around."""
    w = int(window)
    if w > I32_MAX:
        return I32_MAX
    return max(w, -1)


def _check(name, t, ref=None, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ref is not None and t.device != ref.device:
        raise ValueError(f"{name} is on {t.device}, expected {ref.device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(t, stream):
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _fwd_args(q, k, v, o, lse):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check("q", q)
    for n, t in (("k", k), ("v", v), ("o", o)):
        _check(n, t, q, q.dtype, q.shape)
    _check("lse", lse, q, torch.float32, (B, H, N))
    return B, H, N, d


def fa_fwd(q, k, v, o, lse, scale, mask=None, window=0, stream=None):
    """Call fa_fwd on [B, H, N, d] tensors q, k, v -> o (same dtype) and
    lse [B, H, N] float32, enqueued on `stream` (default: torch's current)."""
    B, H, N, d = _fwd_args(q, k, v, o, lse)
    st = load().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       B, H, N, d, _dtype_code(q), float(scale), _mask_code(mask),
                       _window(window), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_fwd")


def fa_fwd_tuned(q, k, v, o, lse, scale, mask=None, window=0, cfg=0, stream=None):
    """Call fa_fwd_tuned (include/fa_tuning.h): fa_fwd with the alternative
    kernel shape `cfg` (0 = the default shape)."""
    B, H, N, d = _fwd_args(q, k, v, o, lse)
    st = load().fa_fwd_tuned(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, H, N, d, _dtype_code(q), float(scale),
                             _mask_code(mask), _window(window), int(cfg), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_fwd_tuned")


def fa_fwd_standard_workspace_bytes(B, H, N, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().fa_fwd_standard_workspace_bytes(int(B), int(H), int(N), int(d), code))


def fa_fwd_standard(q, k, v, o, lse, workspace, scale, mask=None, window=0, stream=None):
    """Call fa_fwd_standard (unfused S -> P -> O through device memory) on
    bf16 [B, H, N, d] tensors; `workspace` is a uint8 GPU tensor of at least
    fa_fwd_standard_workspace_bytes(...) bytes."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check("q", q)
    for n, t in (("k", k), ("v", v), ("o", o)):
        _check(n, t, q, q.dtype, q.shape)
    _check("lse", lse, q, torch.float32, (B, H, N))
    _check("workspace", workspace, q)
    wbytes = workspace.numel() * workspace.element_size()
    st = load().fa_fwd_standard(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), workspace.data_ptr(), wbytes, B, H, N, d,
                                _dtype_code(q), float(scale), _mask_code(mask), _window(window),
                                _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_fwd_standard")


def fa_bwd_standard_workspace_bytes(B, H, N, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().fa_bwd_standard_workspace_bytes(int(B), int(H), int(N), int(d), code))


def fa_bwd_standard(q, k, v, dout, fwd_workspace, dq, dk, dv, workspace, scale, stream=None):
    """Call fa_bwd_standard: the unfused backward reading the P that
    fa_fwd_standard left in `fwd_workspace`; `workspace` (uint8 GPU tensor of
    at least fa_bwd_standard_workspace_bytes(...) bytes) holds dP and dS."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check("q", q)
    for n, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(n, t, q, q.dtype, q.shape)
    _check("fwd_workspace", fwd_workspace, q)
    _check("workspace", workspace, q)
    fb = fwd_workspace.numel() * fwd_workspace.element_size()
    wb = workspace.numel() * workspace.element_size()
    st = load().fa_bwd_standard(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                fwd_workspace.data_ptr(), fb, dq.data_ptr(), dk.data_ptr(),
                                dv.data_ptr(), workspace.data_ptr(), wb, B, H, N, d,
                                _dtype_code(q), float(scale), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_bwd_standard")


def fa_fwd_keymajor_workspace_bytes(B, H, N, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().fa_fwd_keymajor_workspace_bytes(int(B), int(H), int(N), int(d), code))


def fa_fwd_keymajor(q, k, v, o, lse, workspace, scale, mask=None, window=0, block_keys=64,
                    stream=None):
    """Call fa_fwd_keymajor (outer loop over key blocks of `block_keys`, the
    running state in `workspace`, a uint8 GPU tensor of at least
    fa_fwd_keymajor_workspace_bytes(...) bytes) on bf16 [B, H, N, d] tensors."""
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check("q", q)
    for n, t in (("k", k), ("v", v), ("o", o)):
        _check(n, t, q, q.dtype, q.shape)
    _check("lse", lse, q, torch.float32, (B, H, N))
    _check("workspace", workspace, q)
    wbytes = workspace.numel() * workspace.element_size()
    st = load().fa_fwd_keymajor(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr(), workspace.data_ptr(), wbytes, B, H, N, d,
                                _dtype_code(q), float(scale), _mask_code(mask), _window(window),
                                int(block_keys), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_fwd_keymajor")


def fa_bwd_workspace_bytes(B, H, N, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(torch.empty(0, dtype=dtype))
    return int(load().fa_bwd_workspace_bytes(int(B), int(H), int(N), int(d), code))


def _bwd_args(q, k, v, o, dout, lse, dq, dk, dv):
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    _check("q", q)
    for n, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(n, t, q, q.dtype, q.shape)
    _check("lse", lse, q, torch.float32, (B, H, N))
    return B, H, N, d


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, mask=None, window=0,
           stream=None):
    """Call fa_bwd: gradients dq, dk, dv (same dtype/shape as q) from
    q, k, v, o, dout and lse; `workspace` is a uint8 GPU tensor of at least
    fa_bwd_workspace_bytes(...) bytes."""
    B, H, N, d = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv)
    _check("workspace", workspace, q)
    wbytes = workspace.numel() * workspace.element_size()
    st = load().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       workspace.data_ptr(), wbytes, B, H, N, d, _dtype_code(q), float(scale),
                       _mask_code(mask), _window(window), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_bwd")


FA_BWD_NOALLOC_MAX_ROWS = 1 << 24


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale, mask=None, window=0, stream=None):
    """Call fa_bwd_noalloc: fa_bwd without a workspace (the library's static
    device array holds D; B*H*N <= FA_BWD_NOALLOC_MAX_ROWS). Calls that can
    overlap on one GPU race."""
    B, H, N, d = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv)
    st = load().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                               dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                               dv.data_ptr(), B, H, N, d, _dtype_code(q), float(scale),
                               _mask_code(mask), _window(window), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_bwd_noalloc")


def fa_bwd_tuned(q, k, v, o, dout, lse, dq, dk, dv, workspace, scale, mask=None, window=0,
                 cfg=0, stream=None):
    """Call fa_bwd_tuned (include/fa_tuning.h): fa_bwd with the alternative
    kernel shape `cfg` (0 = the default shape)."""
    B, H, N, d = _bwd_args(q, k, v, o, dout, lse, dq, dk, dv)
    _check("workspace", workspace, q)
    wbytes = workspace.numel() * workspace.element_size()
    st = load().fa_bwd_tuned(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                             dv.data_ptr(), workspace.data_ptr(), wbytes, B, H, N, d,
                             _dtype_code(q), float(scale), _mask_code(mask), _window(window),
                             int(cfg), _stream(q, stream))
    if st != 0:
        raise FAError(st, "fa_bwd_tuned")


def fa_probe_mfma_bf16(iters, stream=None) -> float:
    """Call fa_probe_mfma_bf16 (waits for the device): sustained bf16 MFMA
    TFLOP/s of a full-device grid of register-operand MFMAs."""
    out = ctypes.c_double(0.0)
    st = load().fa_probe_mfma_bf16(int(iters), _stream_handle(stream), ctypes.byref(out))
    if st != 0:
        raise FAError(st, "fa_probe_mfma_bf16")
    return out.value


def fa_probe_copy(src, dst, reps, stream=None) -> float:
    """Call fa_probe_copy (waits for the device) on two equally sized uint8
    GPU tensors: GB/s of bytes read plus bytes written."""
    _check("src", src)
    _check("dst", dst, src, src.dtype, src.shape)
    nbytes = src.numel() * src.element_size()
    out = ctypes.c_double(0.0)
    st = load().fa_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, int(reps),
                              _stream(src, stream), ctypes.byref(out))
    if st != 0:
        raise FAError(st, "fa_probe_copy")
    return out.value
