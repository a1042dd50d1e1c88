"""CPU oracle for one rank's ZeRO-DP shard step.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke entry point and the
benchmark's CPU-baseline leg may import this package.  The product library
(`sharded_zero_partition_amd`) never imports it, and this package imports
nothing from the product.

Contents
  layout.py       partition layout, stage memory model, bucket pack (Python)
  zero_oracle.c   fp16 conversions, R-way reduce, overflow flag, Adam (scalar C)
  (this file)     ctypes wrapper over zero_oracle.c, the loss-scale control and
                  the bucket reduce-to-owner

Every function follows a passage of the ZeRO explainer page (azimuth.plus,
"ZeRO: Memory Optimizations Toward Training Trillion Parameter Models"); the
citations are in each file.  Parity pins: every function here is pinned by a
test under tests/ (closed forms, brute force, library routines).  The
loss-scale control, which the pages do not describe, is pinned against
PyTorch's own dynamic loss-scale update (torch._amp_update_scale_).
"""

import ctypes
import os
import subprocess

import numpy as np

from .layout import (KINDS, KIND_BYTES, PARTITIONED, Layout, Segment,  # noqa: F401
                     flat_window, owner_range, pack_fill, partition_layout,
                     stage_bytes_per_rank)

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "zero_oracle.c")
_LIB = os.path.join(_HERE, "libzero_oracle.so")

# one thread, IEEE single precision per operation: no fast-math, no
# contraction of a*b+c into a fused multiply-add, no vector extensions
CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fno-tree-vectorize",
          "-fPIC", "-shared", "-std=c11"]


def build(force: bool = True) -> str:
    """Compile zero_oracle.c with gcc into libzero_oracle.so (next to it)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def load(path: str):
    """Open a compiled copy of zero_oracle.c and declare its signatures."""
    L = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_float
    L.zo_half_to_float.argtypes = [ctypes.c_uint16]
    L.zo_half_to_float.restype = f32
    L.zo_float_to_half.argtypes = [f32]
    L.zo_float_to_half.restype = ctypes.c_uint16
    L.zo_half_to_float_n.argtypes = [P, P, i64]
    L.zo_float_to_half_n.argtypes = [P, P, i64]
    L.zo_reduce.argtypes = [P, i32, P, i64]
    L.zo_overflow_flag.argtypes = [P, i32, i64]
    L.zo_overflow_flag.restype = i32
    L.zo_adam_apply.argtypes = [P, i32, P, P, P, P, i64, f32, i64,
                                f32, f32, f32, f32, f32]
    return L


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = load(_LIB)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _contrib_table(contribs):
    arrs = [np.ascontiguousarray(c).view(np.uint16) for c in contribs]
    n = arrs[0].size
    for a in arrs:
        if a.size != n:
            raise ValueError("contributions differ in length")
    table = (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])
    return arrs, table, n


def half_to_float(h: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(h.shape, dtype=np.float32)
    lib().zo_half_to_float_n(_ptr(h), _ptr(out), h.size)
    return out


def float_to_half(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    lib().zo_float_to_half_n(_ptr(x), _ptr(out), x.size)
    return out


def reduce(contribs) -> np.ndarray:
    arrs, table, n = _contrib_table(contribs)
    out = np.empty(n, dtype=np.float32)
    lib().zo_reduce(table, len(arrs), _ptr(out), n)
    return out


def overflow_flag(contribs) -> int:
    arrs, table, n = _contrib_table(contribs)
    return int(lib().zo_overflow_flag(table, len(arrs), n))


class AdamHP:
    """Adam hyper-parameters (float32 on both sides of every comparison)."""

    def __init__(self, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.0):
        self.lr, self.beta1, self.beta2 = lr, beta1, beta2
        self.eps, self.weight_decay = eps, weight_decay

    def args(self):
        return (self.lr, self.beta1, self.beta2, self.eps, self.weight_decay)


def adam_apply(contribs, p, m, v, out16, scale: float, t: int, hp: AdamHP):
    """Apply one taken Adam step (step number t >= 1) in place on p, m, v and
    write the fp16 copy of p into out16 (None to skip)."""
    arrs, table, n = _contrib_table(contribs)
    for a in (p, m, v):
        assert a.dtype == np.float32 and a.flags.c_contiguous and a.size == n
    o = None
    if out16 is not None:
        assert out16.dtype == np.uint16 and out16.flags.c_contiguous and out16.size == n
        o = _ptr(out16)
    lib().zo_adam_apply(table, len(arrs), _ptr(p), _ptr(m), _ptr(v), o, n,
                        float(scale), int(t), *hp.args())


class LossScaler:
    """Dynamic loss-scale control around the shard step (host scalar logic).

    Reading (the pages do not describe loss scaling): a step whose reduced
    gradients hold any inf/NaN is skipped -- no state changes, the Adam step
    count does not advance -- and the scale is multiplied by `backoff` (not
    below `min_scale`).  After `growth_interval` consecutive taken steps the
    scale is multiplied by `growth`, unless that product overflows to inf.
    This is standard dynamic loss scaling; with min_scale = 0 it matches
    torch._amp_update_scale_ step for step, which the tests check.
    """

    def __init__(self, scale=1024.0, backoff=0.5, growth=2.0, min_scale=1.0,
                 growth_interval=1000, good_steps=0):
        self.scale = float(scale)
        self.backoff = float(backoff)
        self.growth = float(growth)
        self.min_scale = float(min_scale)
        self.growth_interval = int(growth_interval)
        self.good_steps = int(good_steps)

    def update(self, overflow: bool):
        if overflow:
            self.scale = max(float(np.float32(self.scale * self.backoff)), self.min_scale)
            self.good_steps = 0
        else:
            self.good_steps += 1
            if self.growth_interval > 0 and self.good_steps >= self.growth_interval:
                grown = np.float32(self.scale * self.growth)
                if np.isfinite(grown):
                    self.scale = float(grown)
                self.good_steps = 0


class ShardState:
    """Host copy of one rank's fp32 shard state plus its Adam step count."""

    def __init__(self, p: np.ndarray, m=None, v=None, t: int = 0):
        self.p = np.ascontiguousarray(p, dtype=np.float32).copy()
        self.m = np.zeros_like(self.p) if m is None else np.ascontiguousarray(m, np.float32).copy()
        self.v = np.zeros_like(self.p) if v is None else np.ascontiguousarray(v, np.float32).copy()
        self.t = int(t)


def shard_step(state: ShardState, contribs, scaler: LossScaler, hp: AdamHP,
               out16: np.ndarray = None, flag: int = None) -> int:
    """One rank's shard step: reduce, overflow check, skip or Adam, fp16 cast,
    and the loss-scale update.  `flag` may be given when the overflow decision
    is taken over more elements than this call sees (a sampled subset of a
    large shard, or several ranks); otherwise it is computed here.  Returns
    the overflow flag."""
    if flag is None:
        flag = overflow_flag(contribs)
    if not flag:
        adam_apply(contribs, state.p, state.m, state.v, out16, scaler.scale,
                   state.t + 1, hp)
        state.t += 1
    scaler.update(bool(flag))
    return int(flag)


def reduce_to_owner(contrib_lists, lay: Layout, fill: int, rank: int):
    """Reduce-to-owner of bucket fill `fill` for rank `rank`.

    contrib_lists holds R lists of fp16 tensors (uint16 bit patterns), one
    list per reducing rank, each with the layout's tensor sizes.  For every
    flat index g of the fill that the rank owns (`owner_range`), the owner's
    fp16 gradient shard receives fp16(c_0(g) + c_1(g) + ... + c_{R-1}(g)),
    the sum taken in fp32 left to right and rounded once to fp16 (nearest,
    ties to even).  This is the local arithmetic of the bucketed
    reduce-scatter of the Stage 2 (P_os+g) paragraph combined with the
    constant-size buffer of the ZeRO-R paragraph.

    Returns (offset in the rank's shard of the first element, fp16 values)."""
    lo, hi = owner_range(lay, fill, rank)
    if lo >= hi:
        return 0, np.zeros(0, dtype=np.uint16)
    windows = [flat_window(lst, lo, hi) for lst in contrib_lists]
    return lo - rank * lay.shard, float_to_half(reduce(windows))



def owner_step(contrib_lists, lay: Layout, rank: int, state: ShardState, scaler: LossScaler,
               hp: AdamHP, out16: np.ndarray = None) -> int:
    """The owner's shard step fed straight from the R ranks' gradient tensors.

    contrib_lists holds R lists of fp16 tensors (uint16 bit patterns), one
    list per reducing rank, each with the layout's tensor sizes.  The rank's
    contributions are the windows [rank*S, (rank+1)*S) of the R flattened
    lists, zero past the end of the model (the shard's padding receives no
    gradient); the step is then `shard_step` over all S elements of `state`
    and `out16`: fp32 sum (rank 0 first), overflow flag, Adam and the fp16
    slot.  This is the Stage 2 (P_os+g) reduce-scatter's local arithmetic
    joined to the Stage 1 update of the rank's own partition, without an fp16
    gradient shard in between.  Returns the overflow flag."""
    lo = rank * lay.shard
    contribs = [flat_window(lst, lo, lo + lay.shard) for lst in contrib_lists]
    return shard_step(state, contribs, scaler, hp, out16)
