"""Python binding of libzero_partition.so: one rank's ZeRO-DP shard step on
MI355X (gfx950).

Argument marshalling only: every step of the path (layout, bucket pack,
reduce, overflow check, Adam, fp16 cast) runs in the C++/HIP library.  torch
provides device memory and the stream.  Importing this package fails loudly
when the library has not been built (`python -m sharded_zero_partition_amd.build`).

Names follow the C ABI in include/zero_partition.h:
  partition_layout(...)   -> Layout   (zero_partition_layout and accessors)
  Layout.arena_plan(...)               (zero_arena_plan_for); carve_arena(plan)
  Layout.bind_tensors(...)             (zero_layout_bind_tensors)
  Layout.pack_bucket(...)              (zero_pack_bucket)
  Layout.bind_contributions(...)       (zero_layout_bind_contributions)
  Layout.reduce_to_owner(...)          (zero_reduce_to_owner)
  shard_step(...), PreparedStep(...)   (zero_shard_step; zero_shard_step_noalloc with noalloc=True)
  Layout.owner_step(...)               (zero_owner_step)
  set_kernel_timing, last_kernel_ms, kernel_times   (kernel timing)
"""

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_partition.so")

ZERO_OK = 0
STATUS_NAMES = {
    -1: "INVALID_ARG", -2: "ALIGNMENT", -3: "CAPACITY", -4: "INDEX_OVERFLOW",
    -5: "HIP", -6: "OUT_OF_MEMORY", -7: "STATE",
}


class ZeroError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


# ---------------------------------------------------------------------------
# ABI structs (mirror include/zero_partition.h)
# ---------------------------------------------------------------------------

class LayoutInfo(ctypes.Structure):
    _fields_ = [("psi", ctypes.c_int64), ("shard_elems", ctypes.c_int64),
                ("padded_elems", ctypes.c_int64), ("padding", ctypes.c_int64),
                ("n_tensors", ctypes.c_int64), ("align_elems", ctypes.c_int64),
                ("bucket_elems", ctypes.c_int64), ("n_fills", ctypes.c_int64),
                ("n_segments", ctypes.c_int64), ("n_ranks", ctypes.c_int32),
                ("stage", ctypes.c_int32), ("bytes_param16", ctypes.c_int64),
                ("bytes_grad16", ctypes.c_int64), ("bytes_master", ctypes.c_int64),
                ("bytes_momentum", ctypes.c_int64), ("bytes_variance", ctypes.c_int64),
                ("bytes_total", ctypes.c_int64)]


class Segment(ctypes.Structure):
    _fields_ = [("tensor", ctypes.c_int32), ("owner", ctypes.c_int32),
                ("tensor_off", ctypes.c_int64), ("flat_off", ctypes.c_int64),
                ("len", ctypes.c_int64), ("shard_off", ctypes.c_int64),
                ("fill", ctypes.c_int64), ("bucket_off", ctypes.c_int64)]

    def as_tuple(self):
        return (self.tensor, self.owner, self.tensor_off, self.flat_off, self.len,
                self.shard_off, self.fill, self.bucket_off)


class ShardStateC(ctypes.Structure):
    _fields_ = [("shard_elems", ctypes.c_int64), ("p", ctypes.c_void_p * 2),
                ("m", ctypes.c_void_p * 2), ("v", ctypes.c_void_p * 2),
                ("cur", ctypes.c_int32), ("reserved", ctypes.c_int32), ("t", ctypes.c_int64)]


class AdamHParams(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("weight_decay", ctypes.c_float)]


class LossScaler(ctypes.Structure):
    _fields_ = [("scale", ctypes.c_float), ("backoff", ctypes.c_float),
                ("growth", ctypes.c_float), ("min_scale", ctypes.c_float),
                ("growth_interval", ctypes.c_int32), ("good_steps", ctypes.c_int32)]

    @classmethod
    def make(cls, scale=1024.0, backoff=0.5, growth=2.0, min_scale=1.0,
             growth_interval=1000, good_steps=0):
        return cls(scale, backoff, growth, min_scale, growth_interval, good_steps)


ARENA_KINDS = (["param16", "grad16", "master", "momentum", "variance", "master_alt",
                "momentum_alt", "variance_alt", "bucket"] + [f"contrib{r}" for r in range(16)])


class ArenaPlan(ctypes.Structure):
    _fields_ = [("total_bytes", ctypes.c_int64), ("align_bytes", ctypes.c_int64),
                ("offset", ctypes.c_int64 * 25), ("bytes", ctypes.c_int64 * 25)]

    def as_dict(self):
        return {k: (self.offset[i], self.bytes[i]) for i, k in enumerate(ARENA_KINDS)
                if self.offset[i] >= 0}


ABI_STRUCTS = [LayoutInfo, Segment, ShardStateC, AdamHParams, LossScaler, ArenaPlan]

# exported symbol -> (restype, argtypes)
_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64
SIGNATURES = {
    "zero_partition_layout": (ctypes.c_int, [_P, _I64, _I32, _I32, _I64, _I64, _P]),
    "zero_layout_destroy": (ctypes.c_int, [_P]),
    "zero_layout_get_info": (ctypes.c_int, [_P, _P]),
    "zero_layout_tensor_offsets": (ctypes.c_int, [_P, _P, _I64]),
    "zero_layout_rank_range": (ctypes.c_int, [_P, _I32, _P, _P, _P]),
    "zero_layout_segments": (ctypes.c_int, [_P, _P, _I64, _P]),
    "zero_layout_rank_segments": (ctypes.c_int, [_P, _I32, _P, _I64, _P]),
    "zero_layout_fill_segments": (ctypes.c_int, [_P, _I64, _P, _I64, _P]),
    "zero_arena_plan_for": (ctypes.c_int, [_P, _I32, _I32, _I32, _I64, _P]),
    "zero_layout_bind_tensors": (ctypes.c_int, [_P, _P, _P]),
    "zero_pack_bucket": (ctypes.c_int, [_P, _I64, _P, _P, _P]),
    "zero_layout_bind_contributions": (ctypes.c_int, [_P, _I32, _P, _P]),
    "zero_reduce_to_owner": (ctypes.c_int, [_P, _I64, _I32, _P, _P, _P]),
    "zero_shard_step": (ctypes.c_int, [_P, _P, _I32, _P, _P, _P, _P, _P]),
    "zero_shard_step_noalloc": (ctypes.c_int, [_P, _P, _I32, _P, _P, _P, _P, _P]),
    "zero_owner_step": (ctypes.c_int, [_P, _I32, _P, _P, _P, _P, _P, _P]),
    "zero_set_kernel_timing": (ctypes.c_int, [_I32]),
    "zero_last_kernel_ms": (ctypes.c_int, [_P]),
    "zero_kernel_times": (ctypes.c_int, [_P, _I64, _P]),
    "zero_version": (ctypes.c_int, []),
    "zero_last_error": (ctypes.c_char_p, []),
    "zero_last_hip_error": (ctypes.c_int, []),
    "zero_abi_struct_size": (ctypes.c_int64, [_I32]),
    "zero_device_info": (ctypes.c_int, [_P, _P]),
}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m sharded_zero_partition_amd.build` "
            "(hipcc, gfx950). There is no fallback path.")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    for i, s in enumerate(ABI_STRUCTS):
        got = lib.zero_abi_struct_size(i)
        if got != ctypes.sizeof(s):
            raise ImportError(f"ABI mismatch for {s.__name__}: library {got}, binding {ctypes.sizeof(s)}")
    return lib


# torch brings its own copy of the HIP runtime (same soname).  Importing torch
# first makes this library bind to that copy, so one runtime serves both;
# loaded the other way round, a process would hold two runtimes, and the
# second one initialised can find no device.
import torch  # noqa: E402,F401

lib = _load()


def _check(rc: int):
    if rc != ZERO_OK:
        raise ZeroError(rc, lib.zero_last_error().decode(errors="replace"))


def _ref(x):
    return ctypes.byref(x)


def _stream_ptr(stream) -> Optional[int]:
    """hipStream_t of a torch stream (None -> torch's current stream)."""
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _current_device() -> int:
    import torch
    return torch.cuda.current_device()


def _dev_ptr(t, what: str, dtype_bytes: int, dev: int = None):
    """Device address of a contiguous tensor on the current device (`dev`,
    when the caller already knows it)."""
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if dev is None:
        dev = _current_device()
    if t.device.index != dev:
        raise ValueError(f"{what} is on {t.device}, the current device is cuda:{dev}")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")
    if t.element_size() != dtype_bytes:
        raise ValueError(f"{what}: expected {dtype_bytes}-byte elements")
    return t.data_ptr()


# ---------------------------------------------------------------------------
# layout and pack
# ---------------------------------------------------------------------------

class Layout:
    """Owner of a zero_layout handle."""

    def __init__(self, numels: Sequence[int], n_ranks: int, stage: int = 2,
                 align: int = 1, bucket: int = 0):
        arr = (ctypes.c_int64 * len(numels))(*[int(n) for n in numels])
        h = ctypes.c_void_p()
        _check(lib.zero_partition_layout(arr, len(numels), int(n_ranks), int(stage),
                                         int(align), int(bucket), _ref(h)))
        self._h = h
        self._bound = None
        self._numels = [int(n) for n in numels]
        info = self.info            # fixed for the handle's life
        self._bucket_elems = info.bucket_elems
        self._shard_elems = info.shard_elems

    def close(self):
        if self._h:
            lib.zero_layout_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def info(self) -> LayoutInfo:
        out = LayoutInfo()
        _check(lib.zero_layout_get_info(self._h, _ref(out)))
        return out

    def tensor_offsets(self) -> List[int]:
        n = self.info.n_tensors
        arr = (ctypes.c_int64 * max(1, n))()
        _check(lib.zero_layout_tensor_offsets(self._h, arr, n))
        return list(arr[:n])

    def rank_range(self, rank: int):
        b, re, e = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        _check(lib.zero_layout_rank_range(self._h, int(rank), _ref(b), _ref(re), _ref(e)))
        return b.value, re.value, e.value

    def _query(self, fn, *key) -> List[Segment]:
        n = ctypes.c_int64()
        rc = fn(self._h, *key, None, 0, _ref(n))
        if rc not in (ZERO_OK, -3):
            _check(rc)
        arr = (Segment * max(1, n.value))()
        _check(fn(self._h, *key, arr, n.value, _ref(n)))
        return list(arr[:n.value])

    def segments(self) -> List[Segment]:
        return self._query(lib.zero_layout_segments)

    def rank_segments(self, rank: int) -> List[Segment]:
        return self._query(lib.zero_layout_rank_segments, int(rank))

    def fill_segments(self, fill: int) -> List[Segment]:
        return self._query(lib.zero_layout_fill_segments, int(fill))

    def arena_plan(self, pingpong: bool = False, n_contrib: int = 0, with_bucket: bool = False,
                   align_bytes: int = 0) -> ArenaPlan:
        """zero_arena_plan_for: one rank's buffers in one contiguous block."""
        out = ArenaPlan()
        _check(lib.zero_arena_plan_for(self._h, int(bool(pingpong)), int(n_contrib),
                                       int(bool(with_bucket)), int(align_bytes), _ref(out)))
        return out

    def _check_list(self, tensors, what: str):
        """The library reads numel[i] elements from tensor i: the list must
        match the layout's tensor count and sizes exactly."""
        if len(tensors) != len(self._numels):
            raise ValueError(f"{what} has {len(tensors)} tensors, the layout {len(self._numels)}")
        for i, (t, n) in enumerate(zip(tensors, self._numels)):
            if t.numel() != n:
                raise ValueError(f"{what}: tensor {i} has {t.numel()} elements, the layout {n}")

    def bind_tensors(self, tensors, stream=None):
        """Bind the device fp16 tensors (any 2-byte dtype, contiguous) in
        list order; they must stay alive while packing."""
        self._check_list(tensors, "tensor list")
        ptrs = (ctypes.c_void_p * max(1, len(tensors)))()
        for i, t in enumerate(tensors):
            ptrs[i] = _dev_ptr(t, f"tensor {i}", 2) if t.numel() > 0 else None
        _check(lib.zero_layout_bind_tensors(self._h, ptrs, _stream_ptr(stream)))
        self._bound = list(tensors)

    def pack_bucket(self, fill: int, bucket, stream=None) -> int:
        """Write fill `fill` into the device bucket (B two-byte elements)."""
        if bucket.numel() != self._bucket_elems:
            raise ValueError("bucket must hold bucket_elems elements")
        n = ctypes.c_int64()
        _check(lib.zero_pack_bucket(self._h, int(fill), ctypes.c_void_p(_dev_ptr(bucket, "bucket", 2)),
                                    _stream_ptr(stream), _ref(n)))
        return n.value

    def bind_contributions(self, lists, stream=None):
        """Bind R lists of device fp16 tensors (one list per reducing rank, in
        the layout's tensor order) for reduce_to_owner."""
        R = len(lists)
        nt = len(self._numels)
        ptrs = (ctypes.c_void_p * max(1, R * nt))()
        for r, lst in enumerate(lists):
            self._check_list(lst, f"list {r}")
            for i, t in enumerate(lst):
                ptrs[r * nt + i] = _dev_ptr(t, f"tensor {r}/{i}", 2) if t.numel() > 0 else None
        _check(lib.zero_layout_bind_contributions(self._h, R, ptrs, _stream_ptr(stream)))
        self._contrib = [list(lst) for lst in lists]

    def reduce_to_owner(self, fill: int, rank: int, shard, stream=None) -> int:
        """Write rank `rank`'s share of fill `fill` of the reduce into its fp16
        gradient shard (S two-byte elements); returns the elements written."""
        if shard.numel() != self._shard_elems:
            raise ValueError("shard must hold shard_elems elements")
        n = ctypes.c_int64()
        _check(lib.zero_reduce_to_owner(self._h, int(fill), int(rank),
                                        ctypes.c_void_p(_dev_ptr(shard, "shard", 2)),
                                        _stream_ptr(stream), _ref(n)))
        return n.value


    def owner_step(self, rank: int, state: "ShardState", hparams: "AdamHParams",
                   scaler: "LossScaler", out_slot, stream=None) -> int:
        """zero_owner_step: rank `rank`'s ping-pong shard step with the sum
        taken straight from the bound contribution lists.  Returns the
        overflow flag; updates state.t, state.cur and the scaler in place."""
        S = self._shard_elems
        if not state.pingpong:
            raise ValueError("the owner step needs ping-pong state (p_alt, m_alt, v_alt)")
        if state.shard_elems != S:
            raise ValueError(f"state holds {state.shard_elems} elements, the layout's shard {S}")
        if out_slot.numel() != S:
            raise ValueError(f"out_slot has {out_slot.numel()} elements, expected {S}")
        dev = _current_device()
        c = state._to_c(dev)
        flag = ctypes.c_int32()
        slot = ctypes.c_void_p(_dev_ptr(out_slot, "out_slot", 2, dev) if S else None)
        _check(lib.zero_owner_step(self._h, int(rank), _ref(c), _ref(hparams), _ref(scaler), slot,
                                   _stream_ptr(stream), _ref(flag)))
        state.t = c.t
        state.cur = c.cur
        return flag.value


def partition_layout(numels: Sequence[int], n_ranks: int, stage: int = 2, align: int = 1,
                     bucket: int = 0) -> Layout:
    return Layout(numels, n_ranks, stage, align, bucket)


# ---------------------------------------------------------------------------
# shard step
# ---------------------------------------------------------------------------

@dataclass
class ShardState:
    """One rank's fp32 shard state on the device.  With p_alt/m_alt/v_alt the
    step runs single-pass ping-pong and `cur` names the live set."""
    p: object
    m: object
    v: object
    p_alt: object = None
    m_alt: object = None
    v_alt: object = None
    cur: int = 0
    t: int = 0

    @property
    def shard_elems(self) -> int:
        return self.p.numel()

    @property
    def pingpong(self) -> bool:
        return self.p_alt is not None

    def live(self):
        """(p, m, v) of the live set."""
        if self.cur == 0:
            return self.p, self.m, self.v
        return self.p_alt, self.m_alt, self.v_alt

    def _to_c(self, dev: int) -> ShardStateC:
        c = ShardStateC()
        c.shard_elems = self.shard_elems
        sets = [(self.p, self.m, self.v)]
        if self.pingpong:
            sets.append((self.p_alt, self.m_alt, self.v_alt))
        for k, (p, m, v) in enumerate(sets):
            for name, t in (("p", p), ("m", m), ("v", v)):
                if t.numel() != self.shard_elems:
                    raise ValueError(f"{name}[{k}] has {t.numel()} elements, expected {self.shard_elems}")
                getattr(c, name)[k] = _dev_ptr(t, f"{name}[{k}]", 4, dev) if t.numel() else None
        c.cur = self.cur
        c.t = self.t
        return c


def shard_step(state: ShardState, grads, hparams: AdamHParams, scaler: LossScaler, out_slot,
               stream=None, noalloc: bool = False) -> int:
    """zero_shard_step (zero_shard_step_noalloc with noalloc=True): returns
    the overflow flag; updates state.t, state.cur and the scaler in place."""
    R = len(grads)
    S = state.shard_elems
    dev = _current_device()
    ptrs = (ctypes.c_void_p * max(1, R))()
    for r, g in enumerate(grads):
        if g.numel() != S:
            raise ValueError(f"grads[{r}] has {g.numel()} elements, expected {S}")
        ptrs[r] = _dev_ptr(g, f"grads[{r}]", 2, dev) if S else None
    if out_slot.numel() != S:
        raise ValueError(f"out_slot has {out_slot.numel()} elements, expected {S}")
    c = state._to_c(dev)
    flag = ctypes.c_int32()
    slot = ctypes.c_void_p(_dev_ptr(out_slot, "out_slot", 2, dev) if S else None)
    fn = lib.zero_shard_step_noalloc if noalloc else lib.zero_shard_step
    _check(fn(_ref(c), ptrs, R, _ref(hparams), _ref(scaler), slot, _stream_ptr(stream), _ref(flag)))
    state.t = c.t
    state.cur = c.cur
    return flag.value


class PreparedStep:
    """zero_shard_step with its arguments checked and marshalled once, for
    loops that step the same tensors again and again.

    The object keeps references to the tensors; their storage must not be
    moved or resized while it is in use.  The stream is the one given (or
    torch's current stream) at preparation.  Every call writes state.cur and
    state.t into the C state first and reads them back after, updates the
    scaler in place and returns the overflow flag, like shard_step."""

    def __init__(self, state: ShardState, grads, hparams: AdamHParams, scaler: LossScaler,
                 out_slot, stream=None):
        R = len(grads)
        S = state.shard_elems
        self._dev = _current_device()
        self._ptrs = (ctypes.c_void_p * max(1, R))()
        for r, g in enumerate(grads):
            if g.numel() != S:
                raise ValueError(f"grads[{r}] has {g.numel()} elements, expected {S}")
            self._ptrs[r] = _dev_ptr(g, f"grads[{r}]", 2, self._dev) if S else None
        if out_slot.numel() != S:
            raise ValueError(f"out_slot has {out_slot.numel()} elements, expected {S}")
        self._c = state._to_c(self._dev)
        self._flag = ctypes.c_int32()
        slot = ctypes.c_void_p(_dev_ptr(out_slot, "out_slot", 2, self._dev) if S else None)
        self._args = (_ref(self._c), self._ptrs, R, _ref(hparams), _ref(scaler), slot,
                      _stream_ptr(stream), _ref(self._flag))
        self._state = state
        self._keep = (list(grads), hparams, scaler, out_slot)

    def __call__(self) -> int:
        if _current_device() != self._dev:
            raise ValueError(f"prepared on cuda:{self._dev}, the current device is another")
        st, c = self._state, self._c
        c.cur = st.cur
        c.t = st.t
        _check(lib.zero_shard_step(*self._args))
        st.t = c.t
        st.cur = c.cur
        return self._flag.value


def version() -> int:
    return lib.zero_version()


def device_info():
    arch, mem = ctypes.c_int32(), ctypes.c_int64()
    _check(lib.zero_device_info(_ref(arch), _ref(mem)))
    return arch.value, mem.value


def set_kernel_timing(enable: bool):
    """zero_set_kernel_timing for the calling thread."""
    _check(lib.zero_set_kernel_timing(1 if enable else 0))


def last_kernel_ms() -> float:
    """zero_last_kernel_ms: device time of the last timed call's kernels."""
    ms = ctypes.c_float()
    _check(lib.zero_last_kernel_ms(_ref(ms)))
    return ms.value


def kernel_times() -> list:
    """zero_kernel_times: device time (ms) of every call timed since timing
    was enabled on this thread (at most the last 4096), oldest first."""
    n = ctypes.c_int64()
    buf = (ctypes.c_float * 4096)()
    _check(lib.zero_kernel_times(buf, 4096, _ref(n)))
    return [buf[i] for i in range(n.value)]


def carve_arena(plan: ArenaPlan, device="cuda"):
    """Allocate plan.total_bytes once and return {kind: tensor view} (fp32
    kinds as float32, fp16 kinds as int16 bit patterns)."""
    import torch
    arena = torch.empty(plan.total_bytes, dtype=torch.uint8, device=device)
    views = {"_arena": arena}
    for kind, (off, nbytes) in plan.as_dict().items():
        dt = torch.float32 if kind in ("master", "momentum", "variance", "master_alt",
                                       "momentum_alt", "variance_alt") else torch.int16
        views[kind] = arena[off:off + nbytes].view(dt)
    return views

