"""dense_attention_amd: fused dense attention forward on AMD MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (declared in
``include/attn.h``).  It only marshals arguments: every step of the attention
forward runs in the library's HIP kernels.  PyTorch supplies device memory and
streams.  There is no fallback: if the library is missing, every call raises.
"""

from __future__ import annotations

import ctypes
import math
import os
import threading

__all__ = [
    "ATTN_F16", "ATTN_BF16", "ATTN_F32", "AttnError", "attn_fwd", "attn_fwd_ex",
    "attn_fwd_strided", "attn_fwd_partial", "attn_merge", "attn_fwd_split",
    "attn_fwd_split_workspace_size", "attn_fwd_split_noalloc", "NOALLOC_SCRATCH_BYTES",
    "attn_get_config", "attn_variants", "attn_strerror",
    "library_path", "load_library",
]

ATTN_F16 = 0
ATTN_BF16 = 1
ATTN_F32 = 2

STATUS = {
    0: "ATTN_OK", -1: "ATTN_ERR_NULL", -2: "ATTN_ERR_DTYPE", -3: "ATTN_ERR_SHAPE",
    -4: "ATTN_ERR_ALIGN", -5: "ATTN_ERR_SCALE", -6: "ATTN_ERR_DEVICE", -7: "ATTN_ERR_LAUNCH",
    -8: "ATTN_ERR_ARG", -9: "ATTN_ERR_SCRATCH",
}

# Size of the static device scratch behind attn_fwd_split_noalloc (attn.h).
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None
_lock = threading.Lock()


def library_path() -> str:
    return os.path.join(_HERE, "libattn.so")


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str = ""):
        self.status = status
        name = STATUS.get(status, str(status))
        super().__init__(f"{name}: {detail}" if detail else name)


class attn_fwd_options(ctypes.Structure):
    _fields_ = [("rescale_threshold", ctypes.c_float), ("variant", ctypes.c_int),
                ("grid", ctypes.c_int), ("causal", ctypes.c_int), ("causal_offset", ctypes.c_int),
                ("reserved", ctypes.c_int * 2)]


class attn_layout(ctypes.Structure):
    _fields_ = [("batch_stride", ctypes.c_int64), ("head_stride", ctypes.c_int64),
                ("seq_stride", ctypes.c_int64)]


class attn_config(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int), ("block_m", ctypes.c_int), ("block_n", ctypes.c_int),
                ("waves", ctypes.c_int), ("stages", ctypes.c_int), ("lds_bytes", ctypes.c_int),
                ("work_items", ctypes.c_int), ("grid", ctypes.c_int),
                ("workgroups_per_cu", ctypes.c_int), ("num_cus", ctypes.c_int)]


def load_library(path: str | None = None):
    """Loads libattn.so (once).  Raises if it has not been built."""
    global _lib
    # torch ships its own HIP runtime (libamdhip64.so.7).  Loaded first, it
    # satisfies libattn.so's dependency of the same soname, so the library and
    # torch share one runtime: the device, the streams and the pointers torch
    # hands over are then the library's too.  Loaded after libattn.so, torch
    # would map a second runtime next to ROCm's and the two would not see each
    # other's device state.
    import torch  # noqa: F401
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or library_path()
        if not os.path.exists(p):
            raise ImportError(f"{p} is missing: build it with `python -m dense_attention_amd.build`")
        lib = ctypes.CDLL(p)
        vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
        lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp]
        lib.attn_fwd.restype = i
        lib.attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp,
                                    ctypes.POINTER(attn_fwd_options)]
        lib.attn_fwd_ex.restype = i
        lib.attn_get_config.argtypes = [i, i, i, i, i, ctypes.POINTER(attn_fwd_options),
                                        ctypes.POINTER(attn_config)]
        lib.attn_get_config.restype = i
        lib.attn_variant_count.argtypes = []
        lib.attn_variant_count.restype = i
        ip = ctypes.POINTER(ctypes.c_int)
        lib.attn_variant_info.argtypes = [i, ip, ip, ip, ip, ip, ip, ip, ip, ip]
        lib.attn_variant_info.restype = i
        lp = ctypes.POINTER(attn_layout)
        op = ctypes.POINTER(attn_fwd_options)
        lib.attn_fwd_strided.argtypes = [vp, lp, vp, lp, vp, lp, vp, lp, vp, i, i, i, i, i, f, i,
                                         vp, op]
        lib.attn_fwd_strided.restype = i
        lib.attn_fwd_partial.argtypes = [vp, lp, vp, lp, vp, lp, vp, vp, i, i, i, i, i, f, i, vp,
                                         op]
        lib.attn_fwd_partial.restype = i
        lib.attn_merge.argtypes = [vp, vp, i, vp, lp, vp, i, i, i, i, i, vp]
        lib.attn_merge.restype = i
        lib.attn_fwd_split_workspace_size.argtypes = [i, i, i, i, i]
        lib.attn_fwd_split_workspace_size.restype = ctypes.c_size_t
        lib.attn_fwd_split.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp,
                                       ctypes.c_size_t, op]
        lib.attn_fwd_split.restype = i
        lib.attn_fwd_split_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, op]
        lib.attn_fwd_split_noalloc.restype = i
        lib.attn_strerror.argtypes = [i]
        lib.attn_strerror.restype = ctypes.c_char_p
        lib.attn_last_error.argtypes = []
        lib.attn_last_error.restype = ctypes.c_char_p
        if path is None:
            _lib = lib
        return lib


def attn_strerror(status: int) -> str:
    return load_library().attn_strerror(status).decode()


def _check(lib, status: int):
    if status != 0:
        raise AttnError(status, lib.attn_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return ATTN_F16
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float16 or bfloat16")


def _options(rescale_threshold, variant, grid, causal=False):
    """causal: False (no mask), True (last query row sees every key) or an int
    offset (query row i sees keys j <= i + offset)."""
    opts = attn_fwd_options()
    opts.rescale_threshold = -1.0 if rescale_threshold is None else float(rescale_threshold)
    opts.variant = int(variant)
    opts.grid = int(grid)
    if causal is True:
        opts.causal = 1
    elif causal is not False and causal is not None:
        opts.causal = 2
        opts.causal_offset = int(causal)
    return opts


def attn_fwd_ex(q, k, v, o=None, lse=None, scale=None, *, stream=None, return_lse=True,
                rescale_threshold=None, variant=0, grid=0, causal=False):
    """O = softmax(scale·Q·Kᵀ)·V (and the fp32 LSE) for contiguous [B, H, S, D] tensors.

    ``o`` and ``lse`` are allocated with torch when not given.  ``stream`` is a
    ``torch.cuda.Stream`` (default: the current stream).  Returns (o, lse);
    lse is None when ``return_lse`` is false and no buffer was passed.
    """
    import torch

    lib = load_library()
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, S, D = q.shape
    for name, t in (("k", k), ("v", v)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [B, H, S, D]")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    dt = _dtype_code(q)
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous tensor like q")
    if lse is None and return_lse:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if lse is not None and (lse.shape != (B, H, S) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    opts = _options(rescale_threshold, variant, grid, causal)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr() if lse is not None else None, B, H, S, D,
                             float(scale), dt, stream.cuda_stream, ctypes.byref(opts))
    _check(lib, st)
    return o, lse


def attn_fwd(q, k, v, o=None, lse=None, scale=None, *, stream=None, return_lse=True,
             causal=False):
    """The library's default attention forward; see attn_fwd_ex."""
    return attn_fwd_ex(q, k, v, o, lse, scale, stream=stream, return_lse=return_lse,
                       causal=causal)


def attn_get_config(B, H, S, D, dtype, *, rescale_threshold=None, variant=0, grid=0,
                    causal=False) -> dict:
    """Launch configuration for the current device (needs a gfx950 GPU)."""
    lib = load_library()
    code = dtype if isinstance(dtype, int) else _dtype_code_from_torch(dtype)
    out = attn_config()
    opts = _options(rescale_threshold, variant, grid, causal)
    _check(lib, lib.attn_get_config(B, H, S, D, code, ctypes.byref(opts), ctypes.byref(out)))
    return {name: getattr(out, name) for name, _ in attn_config._fields_}


def _dtype_code_from_torch(dtype) -> int:
    import torch
    return {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}[dtype]


def attn_variants() -> list:
    """All tile variants compiled into the library (host only)."""
    lib = load_library()
    out = []
    for idx in range(lib.attn_variant_count()):
        vals = [ctypes.c_int() for _ in range(9)]
        _check(lib, lib.attn_variant_info(idx, *[ctypes.byref(x) for x in vals]))
        keys = ["id", "head_dim", "dtype", "block_m", "block_n", "waves", "stages", "key_split",
                "soft_exp"]
        out.append({kk: x.value for kk, x in zip(keys, vals)})
    return out


def _layout(t):
    """attn_layout of a [B, H, S, D] view whose last dimension is contiguous."""
    if t.dim() != 4 or (t.shape[3] > 1 and t.stride(3) != 1):
        raise ValueError("tensors must be [B, H, S, D] views with a contiguous last dimension")
    return attn_layout(t.stride(0), t.stride(1), t.stride(2))


def _check_inputs(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    B, H, Sq, D = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError("k and v must be [B, H, Skv, D] with q's B, H and D")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype and device")
    if q.device.type != "cuda":
        raise ValueError("tensors must be on a HIP device")
    return B, H, Sq, k.shape[2], D


def _lse_buffer(lse, shape, device, required=False):
    import torch
    if lse is None:
        return torch.empty(shape, dtype=torch.float32, device=device)
    if tuple(lse.shape) != tuple(shape) or lse.dtype != torch.float32 or not lse.is_contiguous() \
            or lse.device != device:
        raise ValueError(f"lse must be a contiguous float32 {tuple(shape)} tensor")
    return lse


def attn_fwd_strided(q, k, v, o=None, lse=None, scale=None, *, stream=None, return_lse=True,
                     rescale_threshold=None, variant=0, grid=0, causal=False):
    """Attention over strided [B, H, S, D] views (e.g. BSHD storage seen through
    ``x.transpose(1, 2)``); k and v may have their own length Skv.

    ``o`` may be any [B, H, Sq, D] view with a contiguous last dimension
    (default: contiguous).  Returns (o, lse).
    """
    import torch

    lib = load_library()
    B, H, Sq, Skv, D = _check_inputs(q, k, v)
    if o is None:
        o = torch.empty((B, H, Sq, D), dtype=q.dtype, device=q.device)
    elif tuple(o.shape) != (B, H, Sq, D) or o.dtype != q.dtype or o.device != q.device:
        raise ValueError("o must be a [B, H, Sq, D] tensor of q's dtype")
    if return_lse or lse is not None:
        lse = _lse_buffer(lse, (B, H, Sq), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    opts = _options(rescale_threshold, variant, grid, causal)
    ql, kl, vl, ol = _layout(q), _layout(k), _layout(v), _layout(o)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_strided(q.data_ptr(), ctypes.byref(ql), k.data_ptr(), ctypes.byref(kl),
                                  v.data_ptr(), ctypes.byref(vl), o.data_ptr(), ctypes.byref(ol),
                                  lse.data_ptr() if lse is not None else None, B, H, Sq, Skv, D,
                                  float(scale), _dtype_code(q), stream.cuda_stream,
                                  ctypes.byref(opts))
    _check(lib, st)
    return o, lse


def attn_fwd_partial(q, k, v, o_part=None, lse_part=None, scale=None, *, stream=None,
                     rescale_threshold=None, variant=0, grid=0, causal=False):
    """Attention of q over the keys k, v of one range, as fp32 (o_part, lse_part):
    o_part normalised within the range, lse_part = ln Σ_range exp(scale·q·k).
    Inputs may be strided views (a key slice ``k[:, :, a:b]`` is one)."""
    import torch

    lib = load_library()
    B, H, Sq, Skv, D = _check_inputs(q, k, v)
    if o_part is None:
        o_part = torch.empty((B, H, Sq, D), dtype=torch.float32, device=q.device)
    elif tuple(o_part.shape) != (B, H, Sq, D) or o_part.dtype != torch.float32 \
            or not o_part.is_contiguous() or o_part.device != q.device:
        raise ValueError("o_part must be a contiguous float32 [B, H, Sq, D] tensor")
    lse_part = _lse_buffer(lse_part, (B, H, Sq), q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    opts = _options(rescale_threshold, variant, grid, causal)
    ql, kl, vl = _layout(q), _layout(k), _layout(v)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_partial(q.data_ptr(), ctypes.byref(ql), k.data_ptr(), ctypes.byref(kl),
                                  v.data_ptr(), ctypes.byref(vl), o_part.data_ptr(),
                                  lse_part.data_ptr(), B, H, Sq, Skv, D, float(scale),
                                  _dtype_code(q), stream.cuda_stream, ctypes.byref(opts))
    _check(lib, st)
    return o_part, lse_part


def attn_merge(o_parts, lse_parts, o=None, lse=None, *, out_dtype=None, stream=None,
               return_lse=True):
    """Merges partials over disjoint key ranges: o_parts [n, B, H, S, D] fp32 and
    lse_parts [n, B, H, S] fp32 (contiguous).  ``out_dtype`` is torch.float16,
    torch.bfloat16 or torch.float32 (default float32 unless ``o`` is given)."""
    import torch

    lib = load_library()
    if o_parts.dim() != 5 or o_parts.dtype != torch.float32 or not o_parts.is_contiguous():
        raise ValueError("o_parts must be a contiguous float32 [n, B, H, S, D] tensor")
    n, B, H, S, D = o_parts.shape
    if tuple(lse_parts.shape) != (n, B, H, S) or lse_parts.dtype != torch.float32 \
            or not lse_parts.is_contiguous():
        raise ValueError("lse_parts must be a contiguous float32 [n, B, H, S] tensor")
    if o is None:
        o = torch.empty((B, H, S, D), dtype=out_dtype or torch.float32, device=o_parts.device)
    elif tuple(o.shape) != (B, H, S, D):
        raise ValueError("o must be [B, H, S, D]")
    code = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}[o.dtype]
    if return_lse or lse is not None:
        lse = _lse_buffer(lse, (B, H, S), o_parts.device)
    if stream is None:
        stream = torch.cuda.current_stream(o_parts.device)
    ol = _layout(o)
    with torch.cuda.device(o_parts.device):
        st = lib.attn_merge(o_parts.data_ptr(), lse_parts.data_ptr(), n, o.data_ptr(),
                            ctypes.byref(ol), lse.data_ptr() if lse is not None else None,
                            B, H, S, D, code, stream.cuda_stream)
    _check(lib, st)
    return o, lse


def attn_fwd_split_workspace_size(B, H, S, D, kv_splits=0) -> int:
    return int(load_library().attn_fwd_split_workspace_size(B, H, S, D, kv_splits))


def attn_fwd_split(q, k, v, o=None, lse=None, scale=None, *, kv_splits=0, workspace=None,
                   stream=None, return_lse=True, rescale_threshold=None, variant=0, grid=0,
                   causal=False):
    """attn_fwd with the keys of each item split into kv_splits ranges (0 = the
    library's choice) and merged; contiguous [B, H, S, D] tensors.  The fp32
    workspace is allocated with torch when not given."""
    import torch

    lib = load_library()
    B, H, S, Skv, D = _check_inputs(q, k, v)
    if Skv != S or not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, S, D] tensors of one shape")
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous tensor like q")
    if return_lse or lse is not None:
        lse = _lse_buffer(lse, (B, H, S), q.device)
    need = attn_fwd_split_workspace_size(B, H, S, D, kv_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    opts = _options(rescale_threshold, variant, grid, causal)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                lse.data_ptr() if lse is not None else None, B, H, S, D,
                                float(scale), _dtype_code(q), stream.cuda_stream, int(kv_splits),
                                workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                ctypes.byref(opts))
    _check(lib, st)
    return o, lse


def attn_fwd_split_noalloc(q, k, v, o, lse=None, scale=None, *, kv_splits=0, stream=None,
                           rescale_threshold=None, variant=0, grid=0, causal=False):
    """attn_fwd_split whose key-range partials live in the library's static device
    scratch (NOALLOC_SCRATCH_BYTES per device): the library call allocates
    nothing.  ``o`` (and ``lse``, if wanted) must be given, so that this
    wrapper allocates nothing either.  Calls that may overlap on one device
    share the scratch and must be ordered by the caller."""
    import torch

    lib = load_library()
    B, H, S, Skv, D = _check_inputs(q, k, v)
    if Skv != S or not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous [B, H, S, D] tensors of one shape")
    if o is None or o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() \
            or o.device != q.device:
        raise ValueError("o must be given: a contiguous tensor like q")
    if lse is not None and (tuple(lse.shape) != (B, H, S) or lse.dtype != torch.float32
                            or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous float32 [B, H, S] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    opts = _options(rescale_threshold, variant, grid, causal)
    with torch.cuda.device(q.device):
        st = lib.attn_fwd_split_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        lse.data_ptr() if lse is not None else None, B, H, S, D,
                                        float(scale), _dtype_code(q), stream.cuda_stream,
                                        int(kv_splits), ctypes.byref(opts))
    _check(lib, st)
    return o, lse
