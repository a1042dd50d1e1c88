"""Python binding of libzero_probe.so (include/zero_probe.h): the
achievable-bandwidth probes reported beside the shard step.

Argument marshalling only; the kernels are HIP (csrc/stream_probe.hip).
Importing this module fails loudly when the library has not been built.

  step_pattern(grads, p, m, v, p_out, m_out, v_out, slot, reps)  -> mean ms
  copy(src, dst, reps)                                           -> mean ms
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_probe.so")

_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "zero_probe_step_pattern": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _P, _P, _I64, _I32, _P, _P]),
    "zero_probe_copy": (ctypes.c_int, [_P, _P, _I64, _I32, _P, _P]),
    "zero_probe_last_error": (ctypes.c_char_p, []),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sharded_zero_partition_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _check(rc: int):
    if rc != 0:
        raise RuntimeError(f"probe status {rc}: {lib.zero_probe_last_error().decode(errors='replace')}")


def _ptr(t: torch.Tensor) -> int:
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("probe buffers must be contiguous device tensors")
    return t.data_ptr()


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def step_pattern(grads, p, m, v, p_out, m_out, v_out, slot, reps: int = 10, stream=None) -> float:
    """zero_probe_step_pattern over p.numel() elements; returns the mean kernel ms."""
    n = p.numel()
    for t in (*grads, m, v, p_out, m_out, v_out, slot):
        if t.numel() != n:
            raise ValueError("every probe array must hold the same number of elements")
    ptrs = (ctypes.c_void_p * len(grads))(*[_ptr(g) for g in grads])
    ms = ctypes.c_float()
    _check(lib.zero_probe_step_pattern(ptrs, len(grads), _ptr(p), _ptr(m), _ptr(v), _ptr(p_out),
                                       _ptr(m_out), _ptr(v_out), _ptr(slot), n, reps,
                                       _stream(stream), ctypes.byref(ms)))
    return ms.value


def copy(src, dst, reps: int = 10, stream=None) -> float:
    """zero_probe_copy of src's bytes into dst; returns the mean kernel ms."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst differ in size")
    ms = ctypes.c_float()
    _check(lib.zero_probe_copy(_ptr(src), _ptr(dst), nbytes, reps, _stream(stream), ctypes.byref(ms)))
    return ms.value
