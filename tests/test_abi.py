"""CPU checks of the C ABI: the library loads, exports every function the
header declares with the binding's struct layouts, computes layouts
identical to the oracle's (host logic, bit for bit), and rejects bad
arguments with the documented status codes before touching any device."""

import ctypes
import os
import random
import re

import pytest

import oracle.layout as OL
from sharded_zero_partition_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "zero_partition.h")


@pytest.fixture(scope="module")
def zp():
    from sharded_zero_partition_amd import build as zbuild
    if not os.path.exists(zbuild.LIB):
        zbuild.build()
    import sharded_zero_partition_amd as z
    return z


def _declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported(zp):
    names = _declared_functions()
    assert len(names) >= 15
    lib = ctypes.CDLL(zp.binding.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(zp.binding.SIGNATURES), "binding and header disagree"


def test_every_header_is_a_built_library():
    """Each header under include/ declares one library's functions, and that
    library exports every one of them (the probe library loads without a
    device too)."""
    from sharded_zero_partition_amd import build as zbuild
    libs = {"zero_partition.h": zbuild.LIB, "zero_probe.h": zbuild.PROBE_LIB}
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == sorted(libs)
    if not all(os.path.exists(p) for p in libs.values()):
        zbuild.build()
    for h, path in libs.items():
        names = _declared_functions(os.path.join(ROOT, "include", h))
        lib = ctypes.CDLL(path)
        for n in names:
            assert hasattr(lib, n), f"{n} declared in {h} but not exported by {os.path.basename(path)}"
    from sharded_zero_partition_amd import probe
    assert set(_declared_functions(os.path.join(ROOT, "include", "zero_probe.h"))) == set(probe.SIGNATURES)


def test_struct_sizes_and_version(zp):
    for i, s in enumerate(zp.binding.ABI_STRUCTS):
        assert zp.lib.zero_abi_struct_size(i) == ctypes.sizeof(s)
    assert zp.lib.zero_abi_struct_size(99) == -1
    assert zp.version() == 10000


def _compare(zp, numels, n_ranks, stage, align, bucket):
    got = zp.partition_layout(numels, n_ranks, stage, align, bucket)
    want = OL.partition_layout(numels, n_ranks, stage, align, bucket)
    info = got.info
    assert (info.psi, info.shard_elems, info.padded_elems, info.padding, info.n_fills) == \
        (want.psi, want.shard, want.padded, want.padding, want.n_fills)
    assert info.n_segments == len(want.segments)
    rb = want.rank_bytes()
    assert (info.bytes_param16, info.bytes_grad16, info.bytes_master, info.bytes_momentum,
            info.bytes_variance, info.bytes_total) == tuple(rb[k] for k in OL.KINDS + ("total",))
    assert got.tensor_offsets() == want.offsets
    assert [s.as_tuple() for s in got.segments()] == [s.as_tuple() for s in want.segments]
    for r in sorted({0, n_ranks - 1, n_ranks // 2}):
        assert got.rank_range(r) == want.rank_range(r)
        assert [s.as_tuple() for s in got.rank_segments(r)] == \
            [s.as_tuple() for s in want.rank_segments(r)]
    if bucket:
        for k in sorted({0, want.n_fills - 1, want.n_fills // 2}):
            if 0 <= k < want.n_fills:
                assert [s.as_tuple() for s in got.fill_segments(k)] == \
                    [s.as_tuple() for s in want.fill_segments(k)]
    got.close()


def test_layout_matches_oracle_random(zp):
    rng = random.Random(5)
    for _ in range(300):
        n_t = rng.randint(0, 30)
        numels = [rng.choice([0, 1, 2, 3, 8, 17, 100, 4096, 10 ** 5]) for _ in range(n_t)]
        bucket = rng.choice([0, 0, 1, 7, 64, 4096]) if sum(numels) < 5000 else rng.choice([0, 4096])
        _compare(zp, numels, rng.randint(1, 70), rng.randint(0, 3), rng.choice([1, 2, 8, 64, 1000]),
                 bucket)


@pytest.mark.parametrize("name", ["tiny", "gpt2_1p5b", "zero3_13b", "zero3_1t"])
def test_layout_matches_oracle_workloads(zp, name):
    w = W.SHARD_WORKLOADS[name]()
    _compare(zp, w.numels, w.n_ranks, w.stage, w.align, 0)
    _compare(zp, w.numels, w.n_ranks, w.stage, 64, 1 << 26)


def test_layout_matches_oracle_pack_workload(zp):
    w = W.pack_20k()
    _compare(zp, w.numels, w.n_ranks, 2, 1, w.bucket)


def test_layout_errors(zp):
    Z = zp.ZeroError
    for bad in (dict(n_ranks=0), dict(n_ranks=2, align=0), dict(n_ranks=2, bucket=-1),
                dict(n_ranks=2, stage=4), dict(n_ranks=2, stage=-1)):
        with pytest.raises(Z, match="INVALID_ARG"):
            zp.partition_layout([5], **bad)
    with pytest.raises(Z, match="INVALID_ARG"):
        zp.partition_layout([5, -1], 2)
    with pytest.raises(Z, match="INDEX_OVERFLOW"):
        zp.partition_layout([2 ** 62, 2 ** 62], 1)
    with pytest.raises(Z, match="INDEX_OVERFLOW"):
        zp.partition_layout([2 ** 60], 1)                # 16 bytes per element overflow
    with pytest.raises(Z, match="OUT_OF_MEMORY"):
        zp.partition_layout([2 ** 40], 2 ** 30, align=1)  # 2^30 segments
    lay = zp.partition_layout([10, 20], 3, bucket=8)
    n = ctypes.c_int64()
    arr = (zp.Segment * 1)()
    assert zp.lib.zero_layout_segments(lay._h, arr, 1, ctypes.byref(n)) == -3   # CAPACITY
    assert n.value == len(OL.partition_layout([10, 20], 3, bucket=8).segments)
    with pytest.raises(Z, match="INVALID_ARG"):
        lay.rank_range(3)
    with pytest.raises(Z, match="INVALID_ARG"):
        lay.fill_segments(4)
    with pytest.raises(Z, match="STATE"):
        zp.partition_layout([10], 2).fill_segments(0)
    assert zp.lib.zero_layout_destroy(None) == 0


def test_empty_layout(zp):
    lay = zp.partition_layout([], 4, bucket=16)
    i = lay.info
    assert (i.psi, i.shard_elems, i.n_segments, i.n_fills) == (0, 0, 0, 0)
    lay = zp.partition_layout([0, 0], 3, align=8)
    assert lay.info.shard_elems == 0 and lay.segments() == []


def test_shard_step_argument_errors_need_no_device(zp):
    """Invalid calls are rejected by the host checks before any HIP call, so
    they run without a GPU (the fake addresses are never dereferenced)."""
    S = 64
    base = 1 << 32
    st = zp.ShardStateC()
    st.shard_elems = S
    st.p[0], st.m[0], st.v[0] = base, base + 4096, base + 8192
    grads = (ctypes.c_void_p * 2)(base + 16384, base + 20480)
    slot = ctypes.c_void_p(base + 24576)
    hp = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    sc = zp.LossScaler.make(1024.0)
    flag = ctypes.c_int32()
    call = lambda st=st, g=grads, R=2, hp=hp, sc=sc, slot=slot: zp.lib.zero_shard_step(  # noqa: E731
        ctypes.byref(st), g, R, ctypes.byref(hp), ctypes.byref(sc), slot, None, ctypes.byref(flag))
    assert call(R=0) == -1 and call(R=17) == -1
    assert call(hp=zp.AdamHParams(1e-4, 1.0, 0.999, 1e-8, 0.0)) == -1
    assert call(hp=zp.AdamHParams(float("nan"), 0.9, 0.999, 1e-8, 0.0)) == -1
    assert call(hp=zp.AdamHParams(1e-4, 0.9, 0.999, 0.0, 0.0)) == -1       # eps must be > 0
    assert call(sc=zp.LossScaler.make(0.0)) == -1
    assert call(sc=zp.LossScaler.make(float("inf"))) == -1
    # the loss-scale floor: scale and min_scale at least 2^-24
    assert call(sc=zp.LossScaler.make(2.0 ** -25, min_scale=2.0 ** -24)) == -1
    assert call(sc=zp.LossScaler.make(1024.0, min_scale=0.0)) == -1
    assert call(sc=zp.LossScaler.make(1024.0, min_scale=2.0 ** -25)) == -1
    assert b"2^-24" in zp.lib.zero_last_error()
    st_big = zp.ShardStateC.from_buffer_copy(st)
    st_big.shard_elems = 4096 * (2 ** 24 - 1) + 1                   # above ZERO_MAX_SHARD_ELEMS
    assert call(st=st_big) == -1 and b"ZERO_MAX_SHARD_ELEMS" in zp.lib.zero_last_error()
    # the no-allocation variant takes the same checks before any HIP call
    noalloc = lambda st=st, sc=sc: zp.lib.zero_shard_step_noalloc(  # noqa: E731
        ctypes.byref(st), grads, 2, ctypes.byref(hp), ctypes.byref(sc), slot, None, ctypes.byref(flag))
    assert noalloc(st=st_big) == -1
    assert noalloc(sc=zp.LossScaler.make(1024.0, min_scale=0.0)) == -1
    st_mis = zp.ShardStateC.from_buffer_copy(st)
    st_mis.p[0] = base + 8
    assert noalloc(st=st_mis) == -2
    assert call(slot=ctypes.c_void_p(base + 24577)) == -2             # slot odd address
    assert call(g=(ctypes.c_void_p * 2)(base + 16386, base + 20480)) == -2
    assert call(g=(ctypes.c_void_p * 2)(None, base + 20480)) == -1
    assert call(slot=ctypes.c_void_p(base + 100)) == -1               # overlaps p
    st2 = zp.ShardStateC.from_buffer_copy(st)
    st2.p[1] = base + (1 << 20)                                      # partial ping-pong set
    assert call(st=st2) == -1
    st3 = zp.ShardStateC.from_buffer_copy(st)
    st3.cur = 1                                                      # cur = 1 in place
    assert call(st=st3) == -1
    st4 = zp.ShardStateC.from_buffer_copy(st)
    st4.p[0] = base + 8                                              # misaligned state
    assert call(st=st4) == -2
    assert zp.lib.zero_shard_step(None, grads, 2, ctypes.byref(hp), ctypes.byref(sc), slot, None,
                                  None) == -1
    assert b"NULL state" in zp.lib.zero_last_error()
    # nothing was modified
    assert sc.scale == 1024.0 and st.t == 0


def test_loss_scale_control_matches_torch_without_device(zp):
    """The library's own loss-scale control on taken steps, driven through an
    empty shard (no device work): good_steps counts, growth after
    growth_interval clean steps, no growth into inf, the step count advances.
    Checked step by step against torch._amp_update_scale_ (CPU tensors)."""
    import torch
    hp = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    flag = ctypes.c_int32(-1)
    for scale0, growth, interval in ((1024.0, 2.0, 3), (1.0, 3.0, 1), (2.0 ** 126, 2.0, 2),
                                     (2.0 ** -24, 1.5, 7), (65536.0, 2.0, 1000)):
        st = zp.ShardStateC()                       # shard_elems = 0: nothing on the device
        sc = zp.LossScaler.make(scale0, growth=growth, min_scale=2.0 ** -24, growth_interval=interval)
        ts = torch.tensor([scale0], dtype=torch.float32)
        tg = torch.zeros(1, dtype=torch.int32)
        for i in range(2 * interval + 5 if interval < 1000 else 2100):
            assert zp.lib.zero_shard_step(ctypes.byref(st), None, 2, ctypes.byref(hp),
                                          ctypes.byref(sc), None, None, ctypes.byref(flag)) == 0
            torch._amp_update_scale_(ts, tg, torch.zeros(1), growth, 0.5, interval)
            assert flag.value == 0 and st.t == i + 1
            assert (sc.scale, sc.good_steps) == (float(ts.item()), int(tg.item())), (scale0, interval, i)


def test_kernel_timing_calls_need_no_device(zp):
    """The timing calls keep per-thread host state only until a timed call
    records events: before that they answer without a GPU."""
    lib = zp.lib
    n = ctypes.c_int64(-1)
    ms = ctypes.c_float()
    assert lib.zero_set_kernel_timing(1) == 0
    assert lib.zero_last_kernel_ms(ctypes.byref(ms)) == -7            # STATE: nothing timed
    assert lib.zero_kernel_times(None, 0, ctypes.byref(n)) == 0 and n.value == 0
    assert lib.zero_kernel_times(None, 0, None) == -1
    assert lib.zero_last_kernel_ms(None) == -1
    assert lib.zero_set_kernel_timing(0) == 0


def test_reduce_to_owner_argument_errors_need_no_device(zp):
    """Argument checks of the contribution binding and the reduce run before
    any HIP call."""
    lay = zp.partition_layout([10, 20], 2, bucket=16)
    ptrs = (ctypes.c_void_p * 4)(1 << 32, (1 << 32) + 64, (1 << 32) + 128, (1 << 32) + 192)
    assert zp.lib.zero_layout_bind_contributions(lay._h, 0, ptrs, None) == -1      # R < 1
    assert zp.lib.zero_layout_bind_contributions(lay._h, 17, ptrs, None) == -1     # R > 16
    bad = (ctypes.c_void_p * 4)(1 << 32, (1 << 32) + 65, (1 << 32) + 128, (1 << 32) + 192)
    assert zp.lib.zero_layout_bind_contributions(lay._h, 2, bad, None) == -2      # odd address
    nul = (ctypes.c_void_p * 4)(1 << 32, None, (1 << 32) + 128, (1 << 32) + 192)
    assert zp.lib.zero_layout_bind_contributions(lay._h, 2, nul, None) == -1
    nob = zp.partition_layout([10, 20], 2)
    assert zp.lib.zero_layout_bind_contributions(nob._h, 2, ptrs, None) == -7     # no bucket plan
    n = ctypes.c_int64()
    assert zp.lib.zero_reduce_to_owner(lay._h, 0, 0, ctypes.c_void_p(1 << 32), None,
                                       ctypes.byref(n)) == -7                     # not bound
    # a fill is one launch: buckets above ZERO_MAX_SHARD_ELEMS are refused
    big = zp.partition_layout([10, 20], 2, bucket=4096 * (2 ** 24 - 1) + 1)
    assert zp.lib.zero_reduce_to_owner(big._h, 0, 0, ctypes.c_void_p(1 << 32), None,
                                       ctypes.byref(n)) == -1
    assert b"ZERO_MAX_SHARD_ELEMS" in zp.lib.zero_last_error()
    assert zp.lib.zero_pack_bucket(big._h, 0, ctypes.c_void_p(1 << 32), None, ctypes.byref(n)) == -1
    assert b"ZERO_MAX_SHARD_ELEMS" in zp.lib.zero_last_error()
    ok = zp.partition_layout([10, 20], 2, bucket=4096 * (2 ** 24 - 1))
    assert zp.lib.zero_pack_bucket(ok._h, 0, ctypes.c_void_p(1 << 32), None, ctypes.byref(n)) == -7


def test_owner_step_argument_errors_need_no_device(zp):
    """The owner step checks its layout, binding, state mode and scalars
    before any HIP call, and modifies nothing when it refuses."""
    lay = zp.partition_layout([10, 20], 4, bucket=16)         # S = 8, rank 3 holds padding only
    hp = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    sc = zp.LossScaler.make(1024.0)
    flag = ctypes.c_int32(-1)
    base = 1 << 32
    st = zp.ShardStateC()
    st.shard_elems = 8
    for k in range(2):
        st.p[k], st.m[k], st.v[k] = base + 256 * (3 * k), base + 256 * (3 * k + 1), base + 256 * (3 * k + 2)
    slot = ctypes.c_void_p(base + 4096)

    def call(l=lay, rank=0, st=st, hp=hp, sc=sc, slot=slot):
        return zp.lib.zero_owner_step(l._h if l is not None else None, rank, ctypes.byref(st),
                                      ctypes.byref(hp), ctypes.byref(sc), slot, None, ctypes.byref(flag))
    assert call() == -7                                                # contributions not bound
    assert b"not bound" in zp.lib.zero_last_error()
    assert call(l=zp.partition_layout([10, 20], 4)) == -7              # no bucket plan
    assert call(l=None) == -1
    inplace = zp.ShardStateC.from_buffer_copy(st)
    inplace.p[1] = inplace.m[1] = inplace.v[1] = None
    assert call(st=inplace) == -1
    assert b"ping-pong" in zp.lib.zero_last_error()
    assert call(hp=zp.AdamHParams(1e-4, 0.9, 0.999, 0.0, 0.0)) == -1   # eps must be > 0
    # (binding uploads tables, so the rank, size and overlap checks that follow
    # it are covered by the GPU tests)
    assert sc.scale == 1024.0 and sc.good_steps == 0 and st.t == 0 and st.cur == 0


def test_good_step_count_saturates_without_a_device(zp):
    """A shard step over an empty shard launches nothing, so the loss-scale
    bookkeeping of a taken step runs on the CPU: with growth disabled the
    good-step count saturates at INT32_MAX instead of overflowing."""
    st = zp.ShardStateC()
    st.shard_elems = 0
    hp = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    sc = zp.LossScaler.make(1024.0)
    sc.growth_interval = 0
    sc.good_steps = 2 ** 31 - 2
    flag = ctypes.c_int32(-1)
    grads = (ctypes.c_void_p * 1)(None)
    for _ in range(2):
        assert zp.lib.zero_shard_step(ctypes.byref(st), grads, 1, ctypes.byref(hp), ctypes.byref(sc),
                                      None, None, ctypes.byref(flag)) == 0
        assert flag.value == 0 and sc.good_steps == 2 ** 31 - 1 and sc.scale == 1024.0
    assert st.t == 2


def test_arena_plan_matches_oracle(zp):
    rng = random.Random(41)
    for _ in range(200):
        n_t = rng.randint(0, 10)
        numels = [rng.choice([0, 1, 5, 100, 4096, 10 ** 6]) for _ in range(n_t)]
        n_ranks, stage = rng.randint(1, 64), rng.randint(0, 3)
        align, bucket = rng.choice([1, 8, 64]), rng.choice([0, 1 << 16])
        pp, nc = rng.random() < 0.5, rng.randint(0, 4)
        wb = bucket > 0 and rng.random() < 0.5
        ab = rng.choice([256, 4096, 1 << 21])
        lay = zp.partition_layout(numels, n_ranks, stage, align, bucket)
        got = lay.arena_plan(pp, nc, wb, ab)
        want, total = OL.arena_plan(OL.partition_layout(numels, n_ranks, stage, align, bucket,
                                                        with_segments=False), pp, nc, wb, ab)
        assert got.total_bytes == total and got.align_bytes == ab
        assert got.as_dict() == want


def test_arena_plan_errors(zp):
    lay = zp.partition_layout([100], 4)
    with pytest.raises(zp.ZeroError, match="STATE"):
        lay.arena_plan(with_bucket=True)
    for bad in (dict(n_contrib=17), dict(align_bytes=100), dict(align_bytes=768)):
        with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
            lay.arena_plan(**bad)
    assert lay.arena_plan().align_bytes == 1 << 21


def test_one_hip_runtime_whatever_the_import_order():
    """torch ships its own copy of the HIP runtime under the same soname.  The
    binding imports torch before it loads the library, so a process that
    imports the package first still maps one runtime, not two."""
    import subprocess
    import sys
    code = ("import sharded_zero_partition_amd as zp\n"
            "zp.version()\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read()\n"
            "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, check=True)
    assert out.stdout.strip().splitlines()[-1] == "1", out.stdout + out.stderr
