"""Python binding of libflashsampling.so: the C entry points under the same names.

Argument marshalling only.  Tensors are PyTorch tensors on the library's GPU
(PyTorch supplies device memory and streams); every computation happens in the
HIP kernels behind the C ABI declared in include/flashsampling.h.  If the
library has not been built, importing this module raises: there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflashsampling.so")

FS_OK = 0
FS_ERR_INVALID_ARG = -1
FS_ERR_UNSUPPORTED = -2
FS_ERR_CAPACITY = -3
FS_ERR_HIP = -4

FS_COMBINE_GUMBEL = 0
FS_COMBINE_MAX = 1

FS_PATH_AUTO = 0
FS_PATH_DOT = 1
FS_PATH_MFMA = 2

# exported symbols and their C signatures
_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_F = ctypes.c_float
SIGNATURES = {
    "fs_create": (_I, [ctypes.POINTER(_P), _I, _I, _I64, _I]),
    "fs_destroy": (None, [_P]),
    "fs_last_error": (ctypes.c_char_p, []),
    "fs_fmms_tiling": (_I, [_P, _I, _I, _I64, _I, ctypes.POINTER(_I64), _P]),
    "fs_fmms_sample": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _F, _U64, _U64, _P, _I64, _I, _P, _P, _P, _I]),
    "fs_fmms_sample_top_p": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _F, _U64, _U64, _P, _I64, _I, _F, _P, _I]),
    "fs_fmms_sample_multi": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _F, _U64, _U64, _P, _I64, _I, _P, _I]),
    "fs_unfused_sample": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _F, _U64, _U64, _P, _I64, _I, _P, _P, _I64,
                               _I]),
    "fs_softmax_sample": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _F, _U64, _U64, _P, _I64, _P, _P, _I64, _I]),
    "fs_group_summary": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _I64, _F, _U64, _U64, _P, _I64, _P, _I]),
    "fs_group_summaries": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _I64, _I, _F, _U64, _U64, _P, _I64, _P,
                                _I]),
    "fs_group_summaries_online": (_I, [_P, _P, _P, _I64, _P, _I64, _I, _I, _I64, _I64, _I, _F, _U64, _U64, _P, _I64,
                                       _P, ctypes.c_uint32, ctypes.c_uint32, _P, _P, _I]),
    "fs_group_combine": (_I, [_P, _P, _P, _I, _I, _U64, _U64, _I, _P]),
    "fs_fmms_sample_noalloc": (_I, [_P, _P, _I64, _P, _I64, _I, _I, _I64, _F, _U64, _U64, _P, _I64, _P]),
    "fs_profile_next_launch": (_I, [_P, _P, _P]),
    "fs_debug_philox": (_I, [_P, _P, _U64, _U64, _I, _I64, _I64, _P, _P]),
    "fs_debug_gumbel_bits": (_I, [_P, _P, _U64, _I64, _P]),
    "fs_debug_gumbel_scan": (_I, [_P, _P, _P]),
}


class FSError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"flashsampling error {code}: {message}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is missing: build the HIP library first (python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = load_library()


def _check(rc: int) -> None:
    if rc != FS_OK:
        raise FSError(rc, _lib.fs_last_error().decode())


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _dptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _matrix(t: torch.Tensor, name: str) -> tuple[int, int, int]:
    if t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16 (got {t.dtype})")
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D row-major tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    return t.shape[0], t.shape[1], t.stride(0)


def _mask_args(mask, B: int, V: int):
    """Pointer and row stride of a packed [B, >= ceil(V/32)] mask (None: no mask)."""
    if mask is None:
        return None, 0
    if mask.dtype not in (torch.int32, torch.uint32) or mask.dim() != 2 or mask.stride(1) != 1:
        raise TypeError("mask must be a 2-D row-major int32/uint32 tensor of packed words")
    if not mask.is_cuda:
        raise ValueError("mask must live on the GPU")
    if mask.shape[0] < B or mask.shape[1] < (V + 31) // 32:
        raise ValueError(f"mask must be at least [{B}, {(V + 31) // 32}] words (got {tuple(mask.shape)})")
    return mask.data_ptr(), mask.stride(0)


def _device_buffer(t: torch.Tensor, dtype, numel: int, name: str) -> None:
    """A contiguous GPU tensor of `dtype` with room for `numel` elements."""
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, {numel} needed")


def _logits_ws(t: torch.Tensor, B: int, V: int) -> None:
    if t.dtype != torch.float32 or t.dim() != 2 or t.stride(1) != 1:
        raise TypeError("logits_ws must be a 2-D row-major float32 tensor")
    if not t.is_cuda:
        raise ValueError("logits_ws must live on the GPU")
    if t.shape[0] < B or t.shape[1] < V:
        raise ValueError(f"logits_ws must be at least [{B}, {V}] (got {tuple(t.shape)})")


# --- context ---------------------------------------------------------------

def fs_create(device: int = 0, max_B: int = 256, max_V: int = 262144, max_top_k: int = 64) -> int:
    h = _P()
    _check(_lib.fs_create(ctypes.byref(h), device, max_B, max_V, max_top_k))
    return h.value


def fs_destroy(ctx: int) -> None:
    _lib.fs_destroy(ctx)


def fs_last_error() -> str:
    return _lib.fs_last_error().decode()


def fs_fmms_tiling(ctx: int, B: int, d: int, V: int, path: int = FS_PATH_AUTO):
    """(n_tiles, bounds) with bounds a list of n_tiles + 1 vocab ids."""
    n = _I64()
    _check(_lib.fs_fmms_tiling(ctx, B, d, V, path, ctypes.byref(n), None))
    bounds = (_I64 * (n.value + 1))()
    _check(_lib.fs_fmms_tiling(ctx, B, d, V, path, ctypes.byref(n), bounds))
    return n.value, list(bounds)


# --- sampling ---------------------------------------------------------------

def fs_fmms_sample(ctx: int, H: torch.Tensor, W: torch.Tensor, temperature: float, seed: int, step: int,
                   mask: torch.Tensor | None = None, top_k: int = 0, out: torch.Tensor | None = None,
                   tile_max: torch.Tensor | None = None, tile_arg: torch.Tensor | None = None,
                   path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B, "out")
    if (tile_max is None) != (tile_arg is None):
        raise ValueError("tile_max and tile_arg go together")
    if tile_max is not None:
        nt, _ = fs_fmms_tiling(ctx, B, d, V, path)
        _device_buffer(tile_max, torch.float32, B * nt, "tile_max")
        _device_buffer(tile_arg, torch.int32, B * nt, "tile_arg")
    mptr, ldm = _mask_args(mask, B, V)
    _check(_lib.fs_fmms_sample(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, V,
                               float(temperature), seed, step, mptr, ldm, top_k, out.data_ptr(), _dptr(tile_max),
                               _dptr(tile_arg), path))
    return out


def fs_fmms_sample_top_p(ctx: int, H: torch.Tensor, W: torch.Tensor, temperature: float, seed: int, step: int,
                         top_k: int, top_p: float, mask: torch.Tensor | None = None, out: torch.Tensor | None = None,
                         path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    """Top-k, then the nucleus holding top_p of the kept mass; returns out [B] int32."""
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B, "out")
    mptr, ldm = _mask_args(mask, B, V)
    _check(_lib.fs_fmms_sample_top_p(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, V,
                                     float(temperature), seed, step, mptr, ldm, top_k, float(top_p), out.data_ptr(),
                                     path))
    return out


def fs_fmms_sample_multi(ctx: int, H: torch.Tensor, W: torch.Tensor, temperature: float, seed: int, step: int,
                         num_samples: int, mask: torch.Tensor | None = None, out: torch.Tensor | None = None,
                         path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    """Returns out: [B, num_samples] int32; out[b, s] is the sample of row b at step `step + s`."""
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if out is None:
        out = torch.empty((B, num_samples), dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B * num_samples, "out")
    mptr, ldm = _mask_args(mask, B, V)
    _check(_lib.fs_fmms_sample_multi(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, V,
                                     float(temperature), seed, step, mptr, ldm, num_samples, out.data_ptr(), path))
    return out


def fs_fmms_sample_noalloc(H: torch.Tensor, W: torch.Tensor, temperature: float, seed: int, step: int,
                           mask: torch.Tensor | None = None, out: torch.Tensor | None = None,
                           stream=None) -> torch.Tensor:
    """fs_fmms_sample without a context (no top-k, tile maxima or path choice), on H's device."""
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B, "out")
    mptr, ldm = _mask_args(mask, B, V)
    with torch.cuda.device(H.device):
        _check(_lib.fs_fmms_sample_noalloc(_stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, V,
                                           float(temperature), seed, step, mptr, ldm, out.data_ptr()))
    return out


def fs_unfused_sample(ctx: int, H: torch.Tensor, W: torch.Tensor, temperature: float, seed: int, step: int,
                      mask: torch.Tensor | None = None, top_k: int = 0, out: torch.Tensor | None = None,
                      logits_ws: torch.Tensor | None = None, path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B, "out")
    if logits_ws is None:
        logits_ws = torch.empty((B, (V + 3) // 4 * 4), dtype=torch.float32, device=H.device)
    _logits_ws(logits_ws, B, V)
    mptr, ldm = _mask_args(mask, B, V)
    _check(_lib.fs_unfused_sample(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, V,
                                  float(temperature), seed, step, mptr, ldm, top_k, out.data_ptr(),
                                  logits_ws.data_ptr(), logits_ws.stride(0), path))
    return out


def fs_softmax_sample(ctx: int, H: torch.Tensor, W: torch.Tensor, temperature: float, seed: int, step: int,
                      mask: torch.Tensor | None = None, out: torch.Tensor | None = None,
                      logits_ws: torch.Tensor | None = None, path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    """Conventional comparator (softmax, prefix sum, inverse CDF); logits_ws holds the probabilities after."""
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B, "out")
    if logits_ws is None:
        logits_ws = torch.empty((B, (V + 3) // 4 * 4), dtype=torch.float32, device=H.device)
    _logits_ws(logits_ws, B, V)
    mptr, ldm = _mask_args(mask, B, V)
    _check(_lib.fs_softmax_sample(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, V,
                                  float(temperature), seed, step, mptr, ldm, out.data_ptr(), logits_ws.data_ptr(),
                                  logits_ws.stride(0), path))
    return out


def summary_views(s: torch.Tensor):
    """(lse, pmax, arg) views of a [..., 3] int32 tensor holding fs_group_summary_t records."""
    return s[..., 0].view(torch.float32), s[..., 1].view(torch.float32), s[..., 2]


def fs_group_summary(ctx: int, H: torch.Tensor, W_group: torch.Tensor, vocab_offset: int, temperature: float,
                     seed: int, step: int, mask: torch.Tensor | None = None, out: torch.Tensor | None = None,
                     path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    """Returns out: [B, 3] int32 records (lse f32, pmax f32, arg i32); see summary_views."""
    B, d, ldh = _matrix(H, "H")
    G, d2, ldw = _matrix(W_group, "W_group")
    if d2 != d:
        raise ValueError("H and W_group disagree on d")
    if out is None:
        out = torch.empty((B, 3), dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, B * 3, "out")
    mptr, ldm = _mask_args(mask, B, vocab_offset + G)
    _check(_lib.fs_group_summary(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W_group.data_ptr(), ldw, B, d,
                                 vocab_offset, G, float(temperature), seed, step, mptr, ldm, out.data_ptr(), path))
    return out


def fs_group_summaries(ctx: int, H: torch.Tensor, W: torch.Tensor, vocab_offset: int, group_size: int,
                       temperature: float, seed: int, step: int, mask: torch.Tensor | None = None,
                       out: torch.Tensor | None = None, path: int = FS_PATH_AUTO, stream=None) -> torch.Tensor:
    """Summaries of the W.shape[0] // group_size consecutive groups of W: [n_groups, B, 3] int32 records."""
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if group_size < 1 or V % group_size != 0:
        raise ValueError("W's rows must be a whole number of groups")
    n_groups = V // group_size
    if out is None:
        out = torch.empty((n_groups, B, 3), dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, n_groups * B * 3, "out")
    mptr, ldm = _mask_args(mask, B, vocab_offset + V)
    _check(_lib.fs_group_summaries(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d, vocab_offset,
                                   group_size, n_groups, float(temperature), seed, step, mptr, ldm, out.data_ptr(),
                                   path))
    return out


def fs_group_summaries_online(ctx: int, H: torch.Tensor, W: torch.Tensor, vocab_offset: int, group_size: int,
                              temperature: float, seed: int, step: int, ready: torch.Tensor, epoch: int,
                              status: torch.Tensor, max_wait_us: int = 1_000_000, mask: torch.Tensor | None = None,
                              out: torch.Tensor | None = None, path: int = FS_PATH_AUTO,
                              stream=None) -> torch.Tensor:
    """fs_group_summaries whose group k starts once ready[k] == epoch.  ready: [n_groups] int32 on the GPU or in
    pinned host memory; status: one int32 on the GPU, set to 1 if a group's wait ran out."""
    B, d, ldh = _matrix(H, "H")
    V, d2, ldw = _matrix(W, "W")
    if d2 != d:
        raise ValueError("H and W disagree on d")
    if group_size < 1 or V % group_size != 0:
        raise ValueError("W's rows must be a whole number of groups")
    n_groups = V // group_size
    if ready.dtype != torch.int32 or not ready.is_contiguous() or ready.numel() < n_groups:
        raise TypeError(f"ready must be a contiguous int32 tensor of at least {n_groups} flags")
    if not (ready.is_cuda or ready.is_pinned()):
        raise ValueError("ready must live on the GPU or in pinned host memory")
    _device_buffer(status, torch.int32, 1, "status")
    if out is None:
        out = torch.empty((n_groups, B, 3), dtype=torch.int32, device=H.device)
    _device_buffer(out, torch.int32, n_groups * B * 3, "out")
    mptr, ldm = _mask_args(mask, B, vocab_offset + V)
    _check(_lib.fs_group_summaries_online(ctx, _stream_ptr(stream), H.data_ptr(), ldh, W.data_ptr(), ldw, B, d,
                                          vocab_offset, group_size, n_groups, float(temperature), seed, step, mptr, ldm,
                                          ready.data_ptr(), epoch & 0xFFFFFFFF, max_wait_us, status.data_ptr(),
                                          out.data_ptr(), path))
    return out


def fs_group_combine(ctx: int, summaries: torch.Tensor, seed: int, step: int, mode: int = FS_COMBINE_GUMBEL,
                     out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """summaries: [n_groups, B, 3] int32 records (contiguous)."""
    if summaries.dtype != torch.int32 or summaries.dim() != 3 or summaries.shape[2] != 3 or not summaries.is_contiguous():
        raise TypeError("summaries must be a contiguous [n_groups, B, 3] int32 tensor")
    n_groups, B, _ = summaries.shape
    if not summaries.is_cuda:
        raise ValueError("summaries must live on the GPU")
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=summaries.device)
    _device_buffer(out, torch.int32, B, "out")
    _check(_lib.fs_group_combine(ctx, _stream_ptr(stream), summaries.data_ptr(), n_groups, B, seed, step, mode,
                                 out.data_ptr()))
    return out


# --- measurement -------------------------------------------------------------

def fs_profile_next_launch(ctx: int, before=None, after=None) -> None:
    """Arm the next streaming call to record torch.cuda.Event `before` / `after` around its
    streaming kernel (both None disarms).  Events must have been recorded once already,
    so that they exist as HIP events."""
    b = None if before is None else before.cuda_event
    a = None if after is None else after.cuda_event
    _check(_lib.fs_profile_next_launch(ctx, b, a))


# --- test exports -------------------------------------------------------------

def fs_debug_philox(ctx: int, seed: int, step: int, row: int, v0: int, n: int, device="cuda", stream=None):
    r = torch.empty(n, dtype=torch.int32, device=device)
    g = torch.empty(n, dtype=torch.float32, device=device)
    _check(_lib.fs_debug_philox(ctx, _stream_ptr(stream), seed, step, row, v0, n, r.data_ptr(), g.data_ptr()))
    return r, g


def fs_debug_gumbel_bits(ctx: int, r0: int, n: int, device="cuda", stream=None) -> torch.Tensor:
    g = torch.empty(n, dtype=torch.float32, device=device)
    _check(_lib.fs_debug_gumbel_bits(ctx, _stream_ptr(stream), r0, n, g.data_ptr()))
    return g


def fs_debug_gumbel_scan(ctx: int, device="cuda", stream=None) -> torch.Tensor:
    stats = torch.zeros(4, dtype=torch.int64, device=device)
    _check(_lib.fs_debug_gumbel_scan(ctx, _stream_ptr(stream), stats.data_ptr()))
    return stats
