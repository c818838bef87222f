"""Device side of the input generator: fills torch CUDA tensors through gen/libgcgen.so.

Same bits as gen.host for the same (key, index); see the package docstring.
"""

import ctypes
import os

import torch

from .host import normal_scale

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgcgen.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run python collective_communication_reduction_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        u64, vp, dbl = ctypes.c_uint64, ctypes.c_void_p, ctypes.c_double
        for name, args in (("gcgen_uniform_f32", [vp, u64, u64, u64, vp]),
                           ("gcgen_normal_bf16", [vp, u64, u64, u64, dbl, vp]),
                           ("gcgen_normal_f32", [vp, u64, u64, u64, dbl, vp]),
                           ("gcgen_int32", [vp, u64, u64, u64, vp]),
                           ("gcgen_normal_bf16_rows", [vp, vp, u64, u64, u64, dbl, vp])):
            f = getattr(lib, name)
            f.restype = ctypes.c_int
            f.argtypes = args
        _lib = lib
    return _lib


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ok(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with HIP error {rc}")


def fill_uniform_f32(t, key, base=0):
    assert t.dtype == torch.float32 and t.is_contiguous()
    _ok(_load().gcgen_uniform_f32(t.data_ptr(), t.numel(), key, base, _stream(t)), "gcgen_uniform_f32")
    return t


def fill_normal_bf16(t, key, sigma, base=0):
    assert t.dtype == torch.bfloat16 and t.is_contiguous()
    _ok(_load().gcgen_normal_bf16(t.data_ptr(), t.numel(), key, base, normal_scale(sigma), _stream(t)),
        "gcgen_normal_bf16")
    return t


def fill_normal_f32(t, key, sigma, base=0):
    assert t.dtype == torch.float32 and t.is_contiguous()
    _ok(_load().gcgen_normal_f32(t.data_ptr(), t.numel(), key, base, normal_scale(sigma), _stream(t)),
        "gcgen_normal_f32")
    return t


def fill_int32(t, key, base=0):
    assert t.dtype == torch.int32 and t.is_contiguous()
    _ok(_load().gcgen_int32(t.data_ptr(), t.numel(), key, base, _stream(t)), "gcgen_int32")
    return t


def fill_normal_bf16_rows(t, tokens, hidden, key, sigma):
    """t: [nrows * hidden] bf16; tokens: int32 CUDA tensor [nrows]; row r = token tokens[r]'s vector."""
    assert t.dtype == torch.bfloat16 and tokens.dtype == torch.int32 and t.numel() == tokens.numel() * hidden
    _ok(_load().gcgen_normal_bf16_rows(t.data_ptr(), tokens.data_ptr(), tokens.numel(), hidden, key,
                                       normal_scale(sigma), _stream(t)), "gcgen_normal_bf16_rows")
    return t
