"""GPU parity of the bucket reduce-to-owner (through the C ABI) against the
oracle: every fill and every owner of small ragged layouts with misaligned
sources and shard bases and R = 1..16 contributions (bit-exact, untouched
elements unchanged), and the 20,000-tensor stream with R = 2 over all 82
fills and 16 owners, every element compared."""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from oracle import layout as OL
from sharded_zero_partition_amd import workloads as W
from gpu_harness import margin_numels

pytestmark = pytest.mark.gpu

SENT = 0x7BCD


def _lists(rng, numels, R):
    """R lists of device tensors carved from one buffer per rank at random
    2-byte offsets, with values up to a few hundred (sums stay finite)."""
    out = []
    for _ in range(R):
        gaps = rng.integers(0, 9, size=len(numels))
        total = int(sum(numels) + gaps.sum() + 8)
        vals = (rng.standard_normal(total, dtype=np.float32) * 100).astype(np.float16)
        buf = torch.from_numpy(vals.view(np.int16)).cuda()
        lst, off = [], 0
        for n, g in zip(numels, gaps):
            off += int(g)
            lst.append(buf[off:off + n])
            off += n
        out.append(lst)
    return out


@pytest.mark.parametrize("R", [1, 2, 3, 4, 7, 9, 16])
def test_small_all_fills_and_owners(R):
    rng = np.random.default_rng(100 + R)
    for trial in range(4):
        numels = [int(x) for x in rng.choice([0, 1, 2, 7, 8, 9, 31, 300, 2049, 5000], size=25)]
        n_ranks = int(rng.integers(1, 6))
        bucket = int(rng.choice([1, 13, 64, 1000, 4099]))
        align = int(rng.choice([1, 8]))
        lay = zp.partition_layout(numels, n_ranks, stage=2, align=align, bucket=bucket)
        olay = OL.partition_layout(numels, n_ranks, 2, align, bucket)
        lists = _lists(rng, numels, R)
        lay.bind_contributions(lists)
        host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
        S = olay.shard
        for r in range(n_ranks):
            mis = int(rng.integers(0, 8))                 # shard base phase
            holder = torch.full((S + 16,), SENT, dtype=torch.int16, device="cuda")
            shard = holder[mis:mis + S]
            want = np.full(S, SENT, np.uint16)
            for k in range(olay.n_fills):
                n = lay.reduce_to_owner(k, r, shard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                assert n == vals.size
                want[off:off + vals.size] = vals
            got = shard.cpu().numpy().view(np.uint16)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)
                raise AssertionError(f"trial {trial} rank {r}: {bad.size} differ, first {bad[0]}")
            h = holder.cpu().numpy().view(np.uint16)
            assert (h[:mis] == SENT).all() and (h[mis + S:] == SENT).all()


@pytest.mark.parametrize("R", [1, 2, 5, 16])
def test_runs_of_tiny_tensors(R):
    """Spans that hold many tensor boundaries: runs of 1..9-element tensors
    (more than 64 tensors in one 1024-element span, and runs of a few dozen)
    between longer tensors, so that the staged path for spans with up to 64
    candidate tensors and the path beyond it both run, across misaligned
    sources and shard bases; every fill and owner against the oracle."""
    rng = np.random.default_rng(300 + R)
    for trial in range(3):
        numels = []
        for _ in range(12):
            numels += [int(x) for x in rng.integers(1, 10, size=int(rng.choice([3, 20, 60, 150])))]
            numels.append(int(rng.choice([100, 1500, 5000, 20000])))
        n_ranks = int(rng.integers(1, 5))
        bucket = int(rng.choice([4096, 1 << 14, 1 << 16]))
        lay = zp.partition_layout(numels, n_ranks, stage=2, align=8, bucket=bucket)
        olay = OL.partition_layout(numels, n_ranks, 2, 8, bucket)
        lists = _lists(rng, numels, R)
        lay.bind_contributions(lists)
        host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
        S = olay.shard
        print(f"[tiny runs] R={R} trial={trial} tensors={len(numels)} psi={olay.psi} ranks={n_ranks} "
              f"fills={olay.n_fills}", flush=True)
        for r in range(n_ranks):
            mis = int(rng.integers(0, 8))
            holder = torch.full((S + 16,), SENT, dtype=torch.int16, device="cuda")
            shard = holder[mis:mis + S]
            want = np.full(S, SENT, np.uint16)
            for k in range(olay.n_fills):
                n = lay.reduce_to_owner(k, r, shard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                assert n == vals.size
                want[off:off + vals.size] = vals
            got = shard.cpu().numpy().view(np.uint16)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)
                raise AssertionError(f"trial {trial} rank {r}: {bad.size} differ, first {bad[0]}")
            h = holder.cpu().numpy().view(np.uint16)
            assert (h[:mis] == SENT).all() and (h[mis + S:] == SENT).all()
        lay.close()


@pytest.mark.parametrize("R", [1, 2, 5])
@pytest.mark.parametrize("mis", [0, 3, 7])
def test_boundaries_at_work_order_margins(R, mis):
    """Tensor boundaries just before, at and after the offsets where the
    launch's work order decides which wave takes a span (span starts - 7 and
    + 8, chunk starts), for both owners of a two-rank layout whose second
    shard starts 7 + mis elements past a chunk start (so that F(w) - 7 falls
    on chunk starts), with the shard base misaligned by mis elements; one fill
    covering everything and 5000-element fills; against the oracle."""
    rng = np.random.default_rng(700 + 10 * R + mis)
    S = 2048 * 30 + 7 + mis
    psi = 2 * S
    numels = margin_numels(rng, [-mis, S - mis], psi)
    lists = _lists(rng, numels, R)
    host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
    for bucket in (psi, 5000):
        lay = zp.partition_layout(numels, 2, stage=2, align=1, bucket=bucket)
        olay = OL.partition_layout(numels, 2, 2, 1, bucket)
        assert olay.shard == S
        lay.bind_contributions(lists)
        print(f"[margins] R={R} mis={mis} tensors={len(numels)} bucket={bucket}", flush=True)
        for r in range(2):
            holder = torch.full((S + 16,), SENT, dtype=torch.int16, device="cuda")
            shard = holder[mis:mis + S]
            want = np.full(S, SENT, np.uint16)
            for k in range(olay.n_fills):
                n = lay.reduce_to_owner(k, r, shard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                assert n == vals.size
                want[off:off + vals.size] = vals
            got = shard.cpu().numpy().view(np.uint16)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)
                raise AssertionError(f"bucket {bucket} rank {r}: {bad.size} differ, first {bad[0]}")
            h = holder.cpu().numpy().view(np.uint16)
            assert (h[:mis] == SENT).all() and (h[mis + S:] == SENT).all()
        lay.close()


@pytest.mark.parametrize("R", [1, 2, 5])
def test_dense_boundaries_run_in_order(R):
    """Thousands of 1..3-element tensors around one longer tensor: the
    boundary waves would far outnumber the spans of each launch, so the
    launch runs in order (each wave its own span); every fill and owner of
    8192-element fills and of one fill, against the oracle."""
    rng = np.random.default_rng(900 + R)
    numels = ([int(x) for x in rng.integers(1, 4, size=3000)] + [5000]
              + [int(x) for x in rng.integers(1, 4, size=3000)])
    lists = _lists(rng, numels, R)
    host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
    psi = sum(numels)
    for bucket in (8192, psi):
        lay = zp.partition_layout(numels, 2, stage=2, align=8, bucket=bucket)
        olay = OL.partition_layout(numels, 2, 2, 8, bucket)
        lay.bind_contributions(lists)
        S = olay.shard
        for r in range(2):
            mis = int(rng.integers(0, 8))
            holder = torch.full((S + 16,), SENT, dtype=torch.int16, device="cuda")
            shard = holder[mis:mis + S]
            want = np.full(S, SENT, np.uint16)
            for k in range(olay.n_fills):
                n = lay.reduce_to_owner(k, r, shard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                assert n == vals.size
                want[off:off + vals.size] = vals
            got = shard.cpu().numpy().view(np.uint16)
            if not np.array_equal(got, want):
                bad = np.flatnonzero(got != want)
                raise AssertionError(f"bucket {bucket} rank {r}: {bad.size} differ, first {bad[0]}")
        lay.close()


def test_errors():
    numels = [10, 20]
    lay = zp.partition_layout(numels, 2, bucket=16)
    shard = torch.zeros(lay.info.shard_elems, dtype=torch.int16, device="cuda")
    with pytest.raises(zp.ZeroError, match="STATE"):
        lay.reduce_to_owner(0, 0, shard)                  # nothing bound
    lists = [[torch.zeros(n, dtype=torch.int16, device="cuda") for n in numels] for _ in range(2)]
    lay.bind_contributions(lists)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        lay.reduce_to_owner(2, 0, shard)                  # fills 0 and 1 only
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        lay.reduce_to_owner(0, 2, shard)                  # ranks 0 and 1 only
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        lay.bind_contributions([lists[0]] * 17)           # R <= 16
    with pytest.raises(zp.ZeroError, match="STATE"):
        zp.partition_layout(numels, 2).bind_contributions(lists)   # no bucket plan
    with pytest.raises(ValueError, match="elements, the layout"):
        lay.bind_contributions([lists[0], [lists[1][0][:-1], lists[1][1]]])
    # psi = 30, S = 15, B = 16: fill 1 is [16, 30), rank 0 owns [0, 15)
    assert lay.reduce_to_owner(1, 0, shard) == 0
    assert lay.reduce_to_owner(0, 1, shard) == 1          # flat index 15 only


def test_pack_20k_two_ranks_full_size():
    w = W.pack_20k()
    print(f"[reduce pack_20k] psi={w.psi} fills={w.n_fills} owners={w.n_ranks}", flush=True)
    lists = [W.pack_sources(w, device="cuda", draw=d) for d in range(2)]
    lay = zp.partition_layout(w.numels, w.n_ranks, stage=2, bucket=w.bucket)
    olay = OL.partition_layout(w.numels, w.n_ranks, 2, 1, w.bucket, with_segments=False)
    lay.bind_contributions(lists)
    S = olay.shard
    flat = torch.full((w.n_ranks * S,), SENT, dtype=torch.int16, device="cuda")
    written = 0
    for k in range(w.n_fills):
        for r in range(w.n_ranks):
            written += lay.reduce_to_owner(k, r, flat[r * S:(r + 1) * S])
    torch.cuda.synchronize()
    assert written == w.psi
    got = flat.cpu().numpy().view(np.uint16)
    assert (got[w.psi:] == SENT).all()                    # padding never written
    host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
    # three whole fills through the oracle's reduce-to-owner, fill by owner
    for k in (0, w.n_fills // 2, w.n_fills - 1):
        for r in range(w.n_ranks):
            off, vals = oracle.reduce_to_owner(host, olay, k, r)
            if vals.size:
                seg = got[r * S + off:r * S + off + vals.size]
                assert np.array_equal(seg, vals), (k, r)
    # every element: the owners' shards tile the flat vector, so flat index g
    # sits at got[g]; the oracle's sum over windows of 2^27 elements in threads
    # (its C calls release the GIL)
    cuts = list(range(0, w.psi, 1 << 27)) + [w.psi]

    def check(ab):
        a, b = ab
        want = oracle.float_to_half(oracle.reduce([OL.flat_window(h, a, b) for h in host]))
        return int(np.count_nonzero(got[a:b] != want))

    with ThreadPoolExecutor(max(1, min(8, os.cpu_count() or 1))) as pool:
        bad = list(pool.map(check, zip(cuts[:-1], cuts[1:])))
    assert sum(bad) == 0, f"{sum(bad)} of {w.psi} elements differ"


def test_special_values_in_contributions():
    """Overflowed gradients reach the reduce before the step's flag sees them:
    +-inf and NaN inputs give exactly the oracle's infinities, NaN wherever
    the oracle has NaN (payload bits unspecified), and every finite sum bit
    for bit."""
    rng = np.random.default_rng(31)
    numels = [1000, 37, 4096 + 5, 3]
    R = 3
    lists = _lists(rng, numels, R)
    specials = np.array([0x7C00, 0xFC00, 0x7E00, 0x7C01], np.uint16).view(np.int16)
    for lst in lists:
        for t in lst:
            n = t.numel()
            pos = torch.from_numpy(rng.integers(0, n, size=max(1, n // 50)))
            t[pos.cuda()] = torch.from_numpy(rng.choice(specials, size=pos.numel())).cuda()
    lay = zp.partition_layout(numels, 2, stage=2, bucket=777)
    olay = OL.partition_layout(numels, 2, 2, 1, 777)
    lay.bind_contributions(lists)
    host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
    S = olay.shard
    for r in range(2):
        shard = torch.full((S,), SENT, dtype=torch.int16, device="cuda")
        want = np.full(S, SENT, np.uint16)
        for k in range(olay.n_fills):
            lay.reduce_to_owner(k, r, shard)
            off, vals = oracle.reduce_to_owner(host, olay, k, r)
            want[off:off + vals.size] = vals
        got = shard.cpu().numpy().view(np.uint16)
        nan = lambda x: ((x & 0x7C00) == 0x7C00) & ((x & 0x3FF) != 0)   # noqa: E731
        assert np.array_equal(nan(got), nan(want))
        assert nan(want).any() and ((want & 0x7FFF) == 0x7C00).any()  # the case holds both
        assert np.array_equal(got[~nan(want)], want[~nan(want)])


def test_every_finite_fp16_class():
    """Random fp16 bit patterns with a finite exponent (subnormals, signed
    zeros, values up to 65504) in every contribution, R = 2, 5 and 16, every
    fill and owner, bit for bit against the oracle."""
    rng = np.random.default_rng(32)
    numels = [int(x) for x in rng.integers(1, 5000, size=30)]
    for R in (2, 5, 16):
        lay = zp.partition_layout(numels, 3, stage=2, bucket=4099)
        olay = OL.partition_layout(numels, 3, 2, 1, 4099)
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
        host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
        S = olay.shard
        for r in range(3):
            shard = torch.full((S,), SENT, dtype=torch.int16, device="cuda")
            want = np.full(S, SENT, np.uint16)
            for k in range(olay.n_fills):
                lay.reduce_to_owner(k, r, shard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                want[off:off + vals.size] = vals
            got = shard.cpu().numpy().view(np.uint16)
            bad = np.flatnonzero(got != want)
            assert bad.size == 0, f"R={R} owner {r}: {bad.size} differ, first at {bad[0]}"
        lay.close()
