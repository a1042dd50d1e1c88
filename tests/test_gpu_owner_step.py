"""GPU parity of the owner step (zero_owner_step through the C ABI) against
the oracle's owner_step: the shard step of one owner fed straight from the R
ranks' ragged gradient lists.

Bar: overflow flag, step count, loss scale and live-set choice exact; fp32
master, momentum and variance and the fp16 slot bit-exact over the whole
shard, padding included (both sides evaluate the same IEEE operations in the
same order; the padding takes the step with a zero gradient); the gather
buffer around the slot unchanged.  Cases: small ragged layouts with
misaligned tensors, every rank, R = 1..16, several steps with new gradient
values each; inf/NaN inside and outside the owner's range; a rank that holds
only padding; zero padding staying zero over NaN-filled alternates and a
following shard step; the fused shard step on the same sums (cross-check of
the two kernels); argument errors; the 13B model's rank 63 as the benchmark
runs it, the 20,000-tensor stream's first and last owner and a shard past
index 2^31, every element of the shard."""

import ctypes
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from oracle import layout as OL
from sharded_zero_partition_amd import workloads as W
from gpu_harness import SENTINEL, margin_numels

pytestmark = pytest.mark.gpu

HP = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
HPC = zp.AdamHParams(HP.lr, HP.beta1, HP.beta2, HP.eps, HP.weight_decay)


class OwnerRun:
    """One owner's device ping-pong state, slot and scaler beside the
    oracle's.  Set 1 starts as NaN, so a read of it shows; the padding of
    set 0 holds random values, so leaving it unstepped shows."""

    def __init__(self, olay, rank: int, rng, scale=1024.0, slot_offset=3, slot_tail=5, hp=HP):
        self.olay = olay
        self.hp = hp
        self.hpc = zp.AdamHParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
        S, n = olay.shard, _real(olay, rank)
        self.S, self.n = S, n
        p0 = (rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)).astype(np.float32)
        p = torch.from_numpy(p0).cuda()
        nan = lambda: torch.full_like(p, float("nan"))   # noqa: E731
        self.state = zp.ShardState(p, torch.zeros_like(p), torch.zeros_like(p), nan(), nan(), nan())
        self.ostate = oracle.ShardState(p0)
        self.scaler = zp.LossScaler.make(scale)
        self.oscaler = oracle.LossScaler(scale)
        self.gather = torch.full((slot_offset + S + slot_tail,), SENTINEL, dtype=torch.int16, device="cuda")
        self.slot_offset = slot_offset
        self.slot = self.gather[slot_offset:slot_offset + S]
        # the slot starts as fp16 of the master values
        self.out16 = p0.astype(np.float16).view(np.uint16).copy()
        self.slot.copy_(torch.from_numpy(self.out16.view(np.int16)).cuda())

    def step(self, lay, rank, host_lists):
        flag = lay.owner_step(rank, self.state, self.hpc, self.scaler, self.slot)
        torch.cuda.synchronize()
        oflag = oracle.owner_step(host_lists, self.olay, rank, self.ostate, self.oscaler, self.hp, self.out16)
        assert flag == oflag, f"flag {flag} != oracle {oflag}"
        if oflag:
            # a skipped step restores the slot to fp16 of the live master
            self.out16[:] = oracle.float_to_half(self.ostate.p)
        assert self.state.t == self.ostate.t
        assert self.scaler.scale == self.oscaler.scale
        assert self.scaler.good_steps == self.oscaler.good_steps
        self.compare()
        return flag

    def compare(self):
        S = self.S
        for name, got, want in zip("pmv", self.state.live(), (self.ostate.p, self.ostate.m, self.ostate.v)):
            g = got.cpu().numpy()
            bad = np.flatnonzero(g.view(np.uint32) != want.view(np.uint32))
            assert bad.size == 0, f"{name}: {bad.size} of {S} differ, first at {bad[0]}: {g[bad[0]]} vs {want[bad[0]]}"
        slot = self.slot.cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(slot != self.out16)
        assert bad.size == 0, f"slot: {bad.size} differ, first at {bad[0]}"
        g = self.gather
        assert int((g[:self.slot_offset] != SENTINEL).sum()) == 0
        assert int((g[self.slot_offset + self.S:] != SENTINEL).sum()) == 0


def _lists(rng, numels, R, scale=1024.0):
    """R lists of device tensors carved from one buffer per rank at random
    2-byte offsets, fp16(N(0, 1e-3) * scale); returns (buffers, lists)."""
    bufs, out = [], []
    for _ in range(R):
        gaps = rng.integers(0, 9, size=len(numels))
        total = int(sum(numels) + gaps.sum() + 8)
        vals = (rng.standard_normal(total, dtype=np.float32) * np.float32(1e-3 * scale)).astype(np.float16)
        buf = torch.from_numpy(vals.view(np.int16)).cuda()
        lst, off = [], 0
        for n, g in zip(numels, gaps):
            off += int(g)
            lst.append(buf[off:off + n])
            off += n
        bufs.append(buf)
        out.append(lst)
    return bufs, out


def _redraw(rng, bufs, scale=1024.0):
    for b in bufs:
        vals = (rng.standard_normal(b.numel(), dtype=np.float32) * np.float32(1e-3 * scale)).astype(np.float16)
        b.copy_(torch.from_numpy(vals.view(np.int16)))


def _host(lists):
    return [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]


def _real(olay, rank):
    lo = rank * olay.shard
    return max(0, min(lo + olay.shard, olay.psi) - lo)


@pytest.mark.parametrize("R", [1, 2, 7])
def test_boundaries_at_work_order_margins(R):
    """Tensor boundaries just before, at and after the offsets where the
    launch's work order decides which wave takes a span (span starts - 7 and
    + 8, chunk starts), for both owners of a two-rank layout whose second
    shard starts 7 elements past a chunk start; two steps each."""
    rng = np.random.default_rng(800 + R)
    S = 2048 * 30 + 7
    psi = 2 * S
    numels = margin_numels(rng, [0, S], psi)
    lay = zp.partition_layout(numels, 2, stage=2, align=1, bucket=1 << 16)
    olay = OL.partition_layout(numels, 2, 2, 1, 1 << 16)
    assert olay.shard == S
    bufs, lists = _lists(rng, numels, R)
    lay.bind_contributions(lists)
    print(f"[margins] R={R} tensors={len(numels)}", flush=True)
    runs = [OwnerRun(olay, r, rng, slot_offset=int(rng.integers(0, 8))) for r in range(2)]
    for step in range(2):
        host = _host(lists)
        for r, run in enumerate(runs):
            assert run.step(lay, r, host) == 0
        _redraw(rng, bufs)
    lay.close()


@pytest.mark.parametrize("R", [1, 2, 7])
def test_dense_boundaries_run_in_order(R):
    """Thousands of 1..3-element tensors around one longer tensor: the
    boundary waves would far outnumber the owner's spans, so the launch runs
    in order; both owners, two steps each."""
    rng = np.random.default_rng(950 + R)
    numels = ([int(x) for x in rng.integers(1, 4, size=3000)] + [5000]
              + [int(x) for x in rng.integers(1, 4, size=3000)])
    lay = zp.partition_layout(numels, 2, stage=2, align=8, bucket=8192)
    olay = OL.partition_layout(numels, 2, 2, 8, 8192)
    bufs, lists = _lists(rng, numels, R)
    lay.bind_contributions(lists)
    runs = [OwnerRun(olay, r, rng, slot_offset=int(rng.integers(0, 8))) for r in range(2)]
    for step in range(2):
        host = _host(lists)
        for r, run in enumerate(runs):
            assert run.step(lay, r, host) == 0
        _redraw(rng, bufs)
    lay.close()


def test_two_threads_owner_steps():
    """Two host threads on their own streams, each running owner steps for
    both ranks of its own layout, each step checked against the oracle in the
    thread; the library serialises the steps of one device."""
    import threading
    rng = np.random.default_rng(960)
    jobs = []
    for k in range(2):
        numels = [int(x) for x in rng.choice([1, 9, 300, 2049, 5000, 30000], size=40)]
        lay = zp.partition_layout(numels, 2, stage=2, align=8, bucket=4096)
        olay = OL.partition_layout(numels, 2, 2, 8, 4096)
        bufs, lists = _lists(rng, numels, 2)
        lay.bind_contributions(lists)
        runs = [OwnerRun(olay, r, rng, slot_offset=int(rng.integers(0, 8))) for r in range(2)]
        jobs.append((lay, lists, runs))
    torch.cuda.synchronize()   # the set-up copies are done before the threads' streams start
    errors = []

    def work(k):
        try:
            torch.cuda.set_device(0)
            lay, lists, runs = jobs[k]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                host = _host(lists)
                for _ in range(3):
                    for r, run in enumerate(runs):
                        assert run.step(lay, r, host) == 0
        except Exception as e:        # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for lay, _, runs in jobs:
        assert all(run.state.t == 3 for run in runs)
        lay.close()


@pytest.mark.parametrize("R", [1, 2, 3, 4, 7, 9, 16])
def test_small_ragged_layouts_every_rank(R):
    rng = np.random.default_rng(500 + R)
    for trial in range(3):
        numels = [int(x) for x in rng.choice([0, 1, 2, 7, 8, 9, 31, 300, 2049, 5000], size=20)]
        n_ranks = int(rng.integers(1, 6))
        bucket = int(rng.choice([1, 64, 4099]))
        align = int(rng.choice([1, 8]))
        lay = zp.partition_layout(numels, n_ranks, stage=2, align=align, bucket=bucket)
        olay = OL.partition_layout(numels, n_ranks, 2, align, bucket)
        bufs, lists = _lists(rng, numels, R)
        lay.bind_contributions(lists)
        runs = []
        for r in range(n_ranks):
            runs.append(OwnerRun(olay, r, rng, slot_offset=int(rng.integers(0, 8))))
        for step in range(3):
            host = _host(lists)
            for r, run in enumerate(runs):
                assert run.step(lay, r, host) == 0
                assert run.state.cur == (step + 1) % 2
            _redraw(rng, bufs)
        lay.close()


def test_seeded_random_cases():
    """Random tensor lists, rank counts, alignments, R, loss scales and
    hyper-parameters; one to three steps per case with new gradients, and
    now and then an inf or NaN planted at a random flat index."""
    rng = np.random.default_rng(2025)
    for case in range(25):
        numels = [int(x) for x in rng.choice([0, 1, 3, 8, 15, 64, 1000, 1024, 1025, 4097, 20000],
                                             size=int(rng.integers(1, 30)))]
        if sum(numels) == 0:
            numels.append(5)
        n_ranks = int(rng.integers(1, 9))
        align = int(rng.choice([1, 8, 64]))
        R = int(rng.integers(1, 17))
        scale = float(2.0 ** rng.integers(0, 17))
        hp = oracle.AdamHP(lr=float(rng.choice([1e-4, 1e-3, 3e-2])), beta1=float(rng.choice([0.0, 0.9])),
                           beta2=float(rng.choice([0.99, 0.999])), eps=float(rng.choice([1e-8, 1e-6])),
                           weight_decay=float(rng.choice([0.0, 0.05])))
        lay = zp.partition_layout(numels, n_ranks, stage=2, align=align, bucket=1 << 12)
        olay = OL.partition_layout(numels, n_ranks, 2, align, 1 << 12)
        std = float(rng.choice([1e-4, 1e-3, 1e-2]))
        bufs, lists = _lists(rng, numels, R, scale=scale * std / 1e-3)
        lay.bind_contributions(lists)
        rank = int(rng.integers(0, n_ranks))
        run = OwnerRun(olay, rank, rng, scale=scale, slot_offset=int(rng.integers(0, 8)), hp=hp)
        offs = np.concatenate([[0], np.cumsum(numels)])
        for step in range(int(rng.integers(1, 4))):
            if rng.random() < 0.25:
                g = int(rng.integers(0, olay.psi))
                i = int(np.searchsorted(offs, g, side="right") - 1)
                bits = int(np.array(rng.choice([0x7C00, 0xFC00, 0x7E01]), np.uint16).view(np.int16))
                lists[int(rng.integers(0, R))][i][g - int(offs[i])] = bits
            run.step(lay, rank, _host(lists))
            _redraw(rng, bufs, scale=scale * std / 1e-3)
        lay.close()


@pytest.mark.parametrize("R", [2, 7])
def test_runs_of_tiny_tensors(R):
    """Owner steps over layouts with runs of 1..9-element tensors between
    longer ones (spans with dozens, and with more than 64, tensor
    boundaries), every rank, two steps."""
    rng = np.random.default_rng(600 + R)
    numels = []
    for _ in range(10):
        numels += [int(x) for x in rng.integers(1, 10, size=int(rng.choice([5, 40, 120])))]
        numels.append(int(rng.choice([700, 3000, 9000])))
    lay = zp.partition_layout(numels, 3, stage=2, align=8, bucket=1 << 13)
    olay = OL.partition_layout(numels, 3, 2, 8, 1 << 13)
    bufs, lists = _lists(rng, numels, R)
    lay.bind_contributions(lists)
    runs = [OwnerRun(olay, r, rng, slot_offset=int(rng.integers(0, 8))) for r in range(3)]
    for step in range(2):
        host = _host(lists)
        for r, run in enumerate(runs):
            assert run.step(lay, r, host) == 0
        _redraw(rng, bufs)
    lay.close()


def test_every_finite_fp16_class():
    """Contributions drawn as random fp16 bit patterns with a finite
    exponent: subnormals, signed zeros and values up to 65504 (16 of them sum
    to a finite fp32 value, so no step is skipped)."""
    rng = np.random.default_rng(31)
    numels = [int(x) for x in rng.integers(1, 5000, size=30)]
    for R in (2, 5, 16):
        lay = zp.partition_layout(numels, 3, stage=2, bucket=1 << 12)
        olay = OL.partition_layout(numels, 3, 2, 1, 1 << 12)
        lists = []
        for _ in range(R):
            gaps = rng.integers(0, 9, size=len(numels))
            bits = rng.integers(0, 1 << 16, size=int(sum(numels) + gaps.sum() + 8), dtype=np.uint16)
            bits[(bits & 0x7C00) == 0x7C00] &= 0xBFFF            # inf/NaN exponent -> finite
            buf = torch.from_numpy(bits.view(np.int16)).cuda()
            lst, off = [], 0
            for n, g in zip(numels, gaps):
                off += int(g)
                lst.append(buf[off:off + n])
                off += n
            lists.append(lst)
        lay.bind_contributions(lists)
        host = _host(lists)
        for r in range(3):
            run = OwnerRun(olay, r, rng, scale=65536.0)
            assert run.step(lay, r, host) == 0
        lay.close()


@pytest.mark.parametrize("value", [np.inf, -np.inf, np.nan])
def test_special_values_inside_and_outside_the_range(value):
    rng = np.random.default_rng(7)
    numels = [1000, 37, 4096, 5, 2500]
    lay = zp.partition_layout(numels, 3, stage=2, bucket=1024)
    olay = OL.partition_layout(numels, 3, 2, 1, 1024)
    bufs, lists = _lists(rng, numels, 2)
    lay.bind_contributions(lists)
    S = olay.shard
    # flat index S + 17 belongs to rank 1: contribution 1 holds the value there
    offs = np.concatenate([[0], np.cumsum(numels)])
    g = S + 17
    i = int(np.searchsorted(offs, g, side="right") - 1)
    lists[1][i][g - int(offs[i])] = torch.tensor(np.float16(value).view(np.int16))
    host = _host(lists)
    runs = [OwnerRun(olay, r, rng) for r in range(3)]
    for r, run in enumerate(runs):
        live_before = [x.clone() for x in run.state.live()]
        slot_before = run.slot.clone()
        flag = run.step(lay, r, host)
        assert flag == (1 if r == 1 else 0)
        if flag:
            assert run.state.cur == 0 and run.state.t == 0
            assert run.scaler.scale == 512.0
            for a, b in zip(run.state.live(), live_before):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32))
            assert torch.equal(run.slot, slot_before)      # restored from the master values
    # the owner that skipped steps again once the value is gone
    _redraw(rng, bufs)
    assert runs[1].step(lay, 1, _host(lists)) == 0 and runs[1].state.t == 1
    lay.close()


def test_padding_only_rank_steps_its_padding():
    """A rank that holds only padding takes the step over its padding with a
    zero gradient (its random master values move by weight decay alone)."""
    rng = np.random.default_rng(8)
    numels = [4, 5]                                     # psi 9, 4 ranks, S = 3: rank 3 all padding
    lay = zp.partition_layout(numels, 4, stage=2, bucket=16)
    olay = OL.partition_layout(numels, 4, 2, 1, 16)
    _, lists = _lists(rng, numels, 2)
    lay.bind_contributions(lists)
    assert olay.shard == 3 and _real(olay, 3) == 0 and _real(olay, 2) == 3
    run = OwnerRun(olay, 3, rng)
    for step in range(1, 3):
        assert run.step(lay, 3, _host(lists)) == 0
        assert run.state.t == step and run.state.cur == step % 2
    # 64-byte alignment: ragged padding on the last rank, all-padding ranks after it
    numels = [1000, 37, 4096, 5, 2500]
    lay2 = zp.partition_layout(numels, 5, stage=2, align=64, bucket=1024)
    olay2 = OL.partition_layout(numels, 5, 2, 64, 1024)
    _, lists2 = _lists(rng, numels, 3)
    lay2.bind_contributions(lists2)
    for r in range(5):
        run = OwnerRun(olay2, r, rng, slot_offset=int(rng.integers(0, 8)))
        assert run.step(lay2, r, _host(lists2)) == 0
    lay.close()
    lay2.close()


def test_zero_padding_stays_zero_over_nan_alternates():
    """Padding that starts at 0 is 0 in the live set and the slot after the
    flip, although the alternate set it lands in held NaN; a following dense
    shard step on the same state (zero contributions over the padding) keeps
    it at 0 in the slot too."""
    rng = np.random.default_rng(12)
    numels = [1000, 37, 4096, 5, 2500]                  # psi 7638
    lay = zp.partition_layout(numels, 3, stage=2, align=64, bucket=1024)
    S = lay.info.shard_elems                            # 2560: rank 2 has 42 padding elements
    _, lists = _lists(rng, numels, 2)
    lay.bind_contributions(lists)
    r = 2
    n = sum(numels) - r * S
    assert 0 < n < S
    p0 = torch.from_numpy(rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)).cuda()
    p0[n:] = 0
    nan = lambda: torch.full_like(p0, float("nan"))     # noqa: E731
    st = zp.ShardState(p0, torch.zeros_like(p0), torch.zeros_like(p0), nan(), nan(), nan())
    slot = torch.full((S,), SENTINEL, dtype=torch.int16, device="cuda")
    slot[:n] = p0[:n].to(torch.float16).view(torch.int16)
    sc = zp.LossScaler.make(1024.0)
    assert lay.owner_step(r, st, HPC, sc, slot) == 0 and st.cur == 1
    torch.cuda.synchronize()
    for x in st.live():
        assert int(torch.count_nonzero(x[n:])) == 0 and not bool(torch.isnan(x).any())
    assert int(torch.count_nonzero(slot[n:])) == 0
    flat = [torch.cat(lst) for lst in lists]
    dense = []
    for f in flat:
        d = torch.zeros(S, dtype=torch.int16, device="cuda")
        d[:n] = f[r * S:r * S + n]
        dense.append(d)
    assert zp.shard_step(st, dense, HPC, sc, slot) == 0 and st.cur == 0
    torch.cuda.synchronize()
    for x in st.live():
        assert int(torch.count_nonzero(x[n:])) == 0
    assert int(torch.count_nonzero(slot[n:])) == 0
    lay.close()


def test_matches_the_fused_shard_step_on_the_same_sums():
    """The owner step and zero_shard_step are two kernels for one definition:
    given the rank's windows of the R flattened lists as dense contributions
    (zero past the model's end), the shard step must produce the same bits
    over the whole shard."""
    rng = np.random.default_rng(9)
    numels = [int(x) for x in rng.integers(1, 3000, size=40)]
    R, n_ranks = 3, 4
    lay = zp.partition_layout(numels, n_ranks, stage=2, align=64, bucket=1 << 12)
    olay = OL.partition_layout(numels, n_ranks, 2, 64, 1 << 12)
    assert olay.padding > 0
    _, lists = _lists(rng, numels, R)
    lay.bind_contributions(lists)
    S = olay.shard
    flat = [torch.cat(lst) for lst in lists]
    for r in range(n_ranks):
        n = _real(olay, r)
        dense = []
        for f in flat:
            d = torch.zeros(S, dtype=torch.int16, device="cuda")
            d[:n] = f[r * S:r * S + n]
            dense.append(d)
        a = OwnerRun(olay, r, np.random.default_rng(r))
        b = OwnerRun(olay, r, np.random.default_rng(r))
        for _ in range(2):
            fa = lay.owner_step(r, a.state, HPC, a.scaler, a.slot)
            fb = zp.shard_step(b.state, dense, HPC, b.scaler, b.slot)
            assert fa == fb == 0
        for x, y in zip(a.state.live(), b.state.live()):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(a.slot, b.slot)
    lay.close()


def test_errors():
    rng = np.random.default_rng(10)
    numels = [100, 200]
    lay = zp.partition_layout(numels, 2, stage=2, bucket=64)
    olay = OL.partition_layout(numels, 2, 2, 1, 64)
    bufs, lists = _lists(rng, numels, 2)
    S = lay.info.shard_elems
    run = OwnerRun(olay, 0, rng)
    with pytest.raises(zp.ZeroError, match="STATE"):
        lay.owner_step(0, run.state, HPC, run.scaler, run.slot)        # not bound
    lay.bind_contributions(lists)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        lay.owner_step(2, run.state, HPC, run.scaler, run.slot)        # rank out of range
    inplace = zp.ShardState(run.state.p, run.state.m, run.state.v)
    with pytest.raises(ValueError, match="ping-pong"):
        lay.owner_step(0, inplace, HPC, run.scaler, run.slot)
    # state that overlaps a bound contribution tensor
    c = run.state._to_c(torch.cuda.current_device())
    c.p[1] = bufs[1].data_ptr() & ~15
    flag = ctypes.c_int32()
    rc = zp.lib.zero_owner_step(lay._h, 0, ctypes.byref(c), ctypes.byref(HPC), ctypes.byref(run.scaler),
                                ctypes.c_void_p(run.slot.data_ptr()), None, ctypes.byref(flag))
    assert rc == -1 and b"overlaps" in zp.lib.zero_last_error()
    # a shard size other than the layout's
    c = run.state._to_c(torch.cuda.current_device())
    c.shard_elems = S - 1
    rc = zp.lib.zero_owner_step(lay._h, 0, ctypes.byref(c), ctypes.byref(HPC), ctypes.byref(run.scaler),
                                ctypes.c_void_p(run.slot.data_ptr()), None, ctypes.byref(flag))
    assert rc == -1 and b"shard_elems" in zp.lib.zero_last_error()
    # misaligned state
    c = run.state._to_c(torch.cuda.current_device())
    c.m[1] = c.m[1] + 4
    rc = zp.lib.zero_owner_step(lay._h, 0, ctypes.byref(c), ctypes.byref(HPC), ctypes.byref(run.scaler),
                                ctypes.c_void_p(run.slot.data_ptr()), None, ctypes.byref(flag))
    assert rc == -2
    run.compare()                                       # nothing was touched
    assert run.state.t == 0 and run.scaler.scale == 1024.0
    lay.close()


# ---------------------------------------------------------------------------
# full sizes, every element
# ---------------------------------------------------------------------------

def _window(buf, starts, offs, lo, hi):
    """The stream's elements of flat indices [lo, hi), gathered tensor piece by
    tensor piece on the device, as host fp16 bit patterns."""
    first = int(np.searchsorted(offs, lo, side="right") - 1)
    pieces, g = [], lo
    for ti in range(first, len(offs) - 1):
        if g >= hi:
            break
        a, b = g, min(hi, int(offs[ti + 1]))
        if b > a:
            s0 = int(starts[ti] + a - offs[ti])
            pieces.append(buf[s0:s0 + (b - a)])
        g = b
    return torch.cat(pieces).cpu().numpy().view(np.uint16) if pieces else np.zeros(0, np.uint16)


def _whole_owner_steps(numels, n_ranks, rank, R, wid, scale, steps, plant=None):
    """R whole gradient streams (workloads.gradient_stream), the owner step of
    `rank` for `steps` steps with new streams each step, and every element of
    the rank's shard (master, momentum, variance, slot) compared bit for bit
    against the oracle's shard step on the rank's windows of the streams,
    zero over the padding.  The oracle runs over the whole shard in
    contiguous chunks on the host's threads (its C calls release the GIL;
    each element depends only on its own inputs and the shard-wide flag,
    which is the expected one).  The draws are finite and their pairwise
    fp32 sums cannot overflow, so the overflow flag is 0 unless `plant`
    ({step: [(contribution, flat index, fp16 bits)]}) puts a special value
    inside the rank's range on that step.  Returns the flags."""
    psi = int(sum(numels))
    lay = zp.partition_layout(numels, n_ranks, stage=2, bucket=1 << 26)
    S = lay.info.shard_elems
    lo = rank * S
    n = max(0, min(lo + S, psi) - lo)
    offs = np.concatenate([[0], np.cumsum(np.asarray(numels, np.int64))])
    p0 = W.normal_f32(S, 0.02, wid, W.KIND_MASTER, 0, rank, "cuda")
    p0[n:] = 0
    st = zp.ShardState(p0, torch.zeros_like(p0), torch.zeros_like(p0),
                       torch.empty_like(p0), torch.empty_like(p0), torch.empty_like(p0))
    slot = torch.empty(S, dtype=torch.int16, device="cuda")
    ost = oracle.ShardState(p0.cpu().numpy())
    sc, osc = zp.LossScaler.make(scale), oracle.LossScaler(scale)
    out16 = np.empty(S, np.uint16)
    threads = max(1, min(16, os.cpu_count() or 1))
    cuts = np.linspace(0, S, threads * 4 + 1).astype(np.int64)
    parts = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
    print(f"[owner step, whole shard] psi={psi} ranks={n_ranks} rank={rank} S={S} n={n} R={R}", flush=True)
    flags = []
    for step in range(1, steps + 1):
        streams = [W.gradient_stream(numels, wid, r, osc.scale, step, "cuda") for r in range(R)]
        want_flag = 0
        for r, g, bits in (plant or {}).get(step, []):
            buf, starts, _ = streams[r]
            ti = int(np.searchsorted(offs, g, side="right") - 1)
            buf[int(starts[ti] + g - offs[ti])] = int(np.int16(np.uint16(bits)))
            want_flag |= int(lo <= g < lo + n)
        lay.bind_contributions([views for _, _, views in streams])
        flag = lay.owner_step(rank, st, HPC, sc, slot)
        torch.cuda.synchronize()
        assert flag == want_flag, f"step {step}: flag {flag}, expected {want_flag}"
        flags.append(flag)
        contribs = []
        for buf, starts, _ in streams:
            c = np.zeros(S, np.uint16)                      # no gradient over the padding
            c[:n] = _window(buf, starts, offs, lo, lo + n)
            contribs.append(c)
        del streams
        used = osc.scale
        if not want_flag:
            def work(ab):
                a, b = ab
                oracle.adam_apply([c[a:b] for c in contribs], ost.p[a:b], ost.m[a:b], ost.v[a:b],
                                  out16[a:b], used, ost.t + 1, HP)
            with ThreadPoolExecutor(threads) as pool:
                list(pool.map(work, parts))
            ost.t += 1
        else:
            # a skipped step restores the slot to fp16 of the live master
            out16[:] = oracle.float_to_half(ost.p)
        osc.update(bool(want_flag))
        assert st.t == ost.t and sc.scale == osc.scale
        for name, got, want in zip("pmv", st.live(), (ost.p, ost.m, ost.v)):
            gv = got.cpu().numpy()
            bad = np.flatnonzero(gv.view(np.uint32) != want.view(np.uint32))
            assert bad.size == 0, f"step {step} {name}: {bad.size} of {S} differ, first at {bad[0]}"
        sv = slot.cpu().numpy().view(np.uint16)
        bad = np.flatnonzero(sv != out16)
        assert bad.size == 0, f"step {step} slot: {bad.size} differ, first at {bad[0]}"
    lay.close()
    return flags


def test_13b_rank63_whole_shard():
    """The benchmark's owner-step configuration: the 13B model's 484 tensors
    (12.85e9 elements), N = 64, rank 63 (S = 200,752,240), R = 2 streams at
    loss scale 1024, three steps; every element of the shard compared."""
    w = W.zero3_13b()
    _whole_owner_steps(w.numels, w.n_ranks, w.rank, 2, w.wid, w.scale, 3)


def test_13b_rank63_overflow_whole_shard():
    """The benchmark's owner-step configuration with an overflow: on step 2
    contribution 1 holds +inf at a position inside rank 63's range and
    contribution 0 a NaN outside it (rank 62's).  Flags 0, 1, 0; the skipped
    step leaves the state as it was and restores the whole slot to fp16 of
    the master; the loss scale halves and the next step runs at the new
    scale.  Every element of the shard compared against the oracle."""
    w = W.zero3_13b()
    lo = w.rank * w.shard
    plant = {2: [(1, lo + 12_345_678, 0x7C00), (0, lo - 1000, 0x7E00)]}
    flags = _whole_owner_steps(w.numels, w.n_ranks, w.rank, 2, w.wid, w.scale, 3, plant=plant)
    assert flags == [0, 1, 0]


def test_shard_past_2_31_whole_shard():
    """Element indices past the signed 32-bit range: rank 1 of 2 over three
    tensors of 2^32 + 8198 elements in all, so its shard (2^31 + 4099
    elements) starts past flat index 2^31, reaches past 2^32 and holds a
    tensor boundary; R = 2 streams, two steps; every element compared."""
    numels = [(1 << 31) + 4096, (1 << 31) - 7, 4109]
    torch.cuda.empty_cache()
    _whole_owner_steps(numels, 2, 1, 2, W.past_2_31().wid, 1024.0, 2)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("rank", [0, 15])
def test_pack_20k_stream_whole_shard(rank):
    """The 20,000 log-uniform tensors (5.48e9 elements) cut for 16 owners:
    the first owner and the last (whose shard ends in 8 padding elements),
    R = 2, one step; every element of the shard compared."""
    pw = W.pack_20k()
    _whole_owner_steps(pw.numels, pw.n_ranks, rank, 2, pw.wid, 1024.0, 1)
