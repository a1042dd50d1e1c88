"""GPU parity of the bucket pack (through the C ABI) against the oracle's
window of the concatenated tensors: bit-exact on every fill, with ragged and
misaligned tensors, tiny tensors, odd bucket sizes, special bit patterns, and
the 20,000-tensor workload at full size (82 fills of 2^26)."""

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from sharded_zero_partition_amd import workloads as W
from gpu_harness import margin_numels

pytestmark = pytest.mark.gpu


def _views_at_offsets(rng, numels, misalign=True):
    """Device tensors carved out of one buffer at arbitrary (2-byte) offsets,
    so their addresses cover every alignment phase."""
    gaps = rng.integers(0, 9, size=len(numels)) if misalign else np.zeros(len(numels), np.int64)
    total = int(sum(numels) + gaps.sum() + 16)
    buf = torch.from_numpy(rng.integers(0, 1 << 16, size=total, dtype=np.uint16).view(np.int16)).cuda()
    out, off = [], 0
    for n, gap in zip(numels, gaps):
        off += int(gap)
        out.append(buf[off:off + n])
        off += n
    return out, buf


def _check_all_fills(tensors, numels, bucket, n_ranks=4):
    lay = zp.partition_layout(numels, n_ranks, stage=2, bucket=bucket)
    lay.bind_tensors(tensors)
    host = [t.cpu().numpy().view(np.uint16) for t in tensors]
    b = torch.full((bucket,), 0x1234, dtype=torch.int16, device="cuda")
    info = lay.info
    psi = sum(numels)
    for k in range(info.n_fills):
        n = lay.pack_bucket(k, b)
        assert n == min(bucket, psi - k * bucket)
        got = b.cpu().numpy().view(np.uint16)
        want = oracle.pack_fill(host, k, bucket)
        if not np.array_equal(got, want):
            bad = np.flatnonzero(got != want)
            raise AssertionError(f"fill {k}: {bad.size} elements differ, first at {bad[0]}")
    return info


@pytest.mark.parametrize("bucket", [1, 5, 8, 13, 64, 1000, 4096 + 3])
def test_small_random_lists(bucket):
    rng = np.random.default_rng(bucket)
    numels = [int(x) for x in rng.choice([0, 1, 2, 3, 7, 8, 9, 15, 16, 17, 100, 1023, 5000],
                                         size=60)]
    tensors, _ = _views_at_offsets(rng, numels)
    _check_all_fills(tensors, numels, bucket)


def test_aligned_large_tensors_and_ragged_tail():
    rng = np.random.default_rng(2)
    numels = [1 << 20, 3, (1 << 18) + 5, 1, 77777]
    tensors = [torch.from_numpy(rng.integers(0, 1 << 16, size=n, dtype=np.uint16).view(np.int16)).cuda()
               for n in numels]
    info = _check_all_fills(tensors, numels, 1 << 16)
    assert info.n_fills == -(-sum(numels) // (1 << 16))


def test_special_bit_patterns_survive():
    pats = np.array([0x7E01, 0xFE00, 0x8000, 0x7C00, 0xFC00, 0x0001, 0x7FFF, 0x0000], np.uint16)
    rng = np.random.default_rng(3)
    numels = [3, 5, 8, 1, 19]
    tensors = [torch.from_numpy(np.resize(pats, n).view(np.int16)).cuda() for n in numels]
    _check_all_fills(tensors, numels, 16)
    tensors, _ = _views_at_offsets(rng, [37, 2, 64])
    _check_all_fills(tensors, [37, 2, 64], 24)


@pytest.mark.parametrize("misalign", [False, True])
def test_boundaries_at_work_order_margins(misalign):
    """Tensor boundaries just before, at and after the offsets where the
    launch's work order decides which wave takes a span (span starts - 7 and
    + 8, chunk starts) in every fill of a bucket of 2048 * 10 + 7 elements
    (so that F(w) - 7 of the second fill falls on chunk starts), the last
    fill ending early; tensors aligned or at every alignment phase."""
    rng = np.random.default_rng(40 + misalign)
    bucket = 2048 * 10 + 7
    psi = 4 * bucket + 3001
    numels = margin_numels(rng, [k * bucket for k in range(5)], psi)
    tensors, _ = _views_at_offsets(rng, numels, misalign=misalign)
    print(f"[margins] misalign={misalign} tensors={len(numels)}", flush=True)
    info = _check_all_fills(tensors, numels, bucket)
    assert info.n_fills == 5


def test_dense_boundaries_run_in_order():
    """Thousands of 1..3-element tensors around one longer tensor, 8192- and
    3001-element fills: the boundary waves would far outnumber the spans, so
    each launch runs in order; every fill against the oracle."""
    rng = np.random.default_rng(41)
    numels = ([int(x) for x in rng.integers(1, 4, size=3000)] + [5000]
              + [int(x) for x in rng.integers(1, 4, size=3000)])
    tensors, _ = _views_at_offsets(rng, numels)
    for bucket in (8192, 3001):
        _check_all_fills(tensors, numels, bucket)


def test_errors():
    lay = zp.partition_layout([10, 20], 2, bucket=0)
    with pytest.raises(zp.ZeroError, match="STATE"):
        lay.bind_tensors([torch.zeros(10, dtype=torch.int16, device="cuda"),
                          torch.zeros(20, dtype=torch.int16, device="cuda")])
    lay = zp.partition_layout([10, 20], 2, bucket=16)
    b = torch.zeros(16, dtype=torch.int16, device="cuda")
    with pytest.raises(zp.ZeroError, match="STATE"):
        lay.pack_bucket(0, b)                         # not bound
    t = [torch.zeros(10, dtype=torch.int16, device="cuda"), torch.zeros(20, dtype=torch.int16, device="cuda")]
    lay.bind_tensors(t)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        lay.pack_bucket(2, b)                         # fills are 0 and 1
    big = torch.zeros(24, dtype=torch.int16, device="cuda")
    with pytest.raises(zp.ZeroError, match="ALIGNMENT"):
        lay.pack_bucket(0, big[1:17])                 # bucket must be 16-byte aligned
    # the binding checks the list against the layout before the library reads it
    with pytest.raises(ValueError, match="tensors, the layout"):
        lay.bind_tensors(t[:1])
    with pytest.raises(ValueError, match="elements, the layout"):
        lay.bind_tensors([t[0], t[1][:-1]])


def test_pack_20k_full_size():
    w = W.pack_20k()
    print(f"[pack_20k] tensors={len(w.numels)} psi={w.psi} fills={w.n_fills}", flush=True)
    tensors = W.pack_sources(w, device="cuda")
    info = _check_all_fills(tensors, w.numels, w.bucket, n_ranks=w.n_ranks)
    assert (info.psi, info.n_fills, info.shard_elems, info.padding) == \
        (5_481_113_944, 82, 342_569_622, 8)


def test_pack_20k_views_full_size():
    """The same stream with every tensor a view into one buffer at a 1..7
    element gap: all misalignment phases, bit-exact on every fill."""
    w = W.pack_20k()
    tensors = W.pack_sources(w, device="cuda", views=True)
    _check_all_fills(tensors, w.numels, w.bucket, n_ranks=w.n_ranks)


def test_13b_gradient_stream_all_fills():
    """The 13B model's full fp16 gradient stream (484 tensors, 12.85e9
    elements, 192 fills of 2^26) as the benchmark's rank iteration packs it:
    every fill (the ragged last one included) against the oracle's window of
    the tensors it overlaps (copied to the host slice by slice)."""
    w = W.zero3_13b()
    B = 1 << 26
    numels = w.numels
    print(f"[13B stream] tensors={len(numels)} psi={sum(numels)}", flush=True)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(13)
    tensors = [torch.randint(-32768, 32768, (n,), dtype=torch.int16, device="cuda", generator=gen)
               for n in numels]
    lay = zp.partition_layout(numels, w.n_ranks, stage=w.stage, bucket=B)
    lay.bind_tensors(tensors)
    n_fills = lay.info.n_fills
    assert n_fills == 192
    offs = np.concatenate([[0], np.cumsum(numels)]).astype(np.int64)
    b = torch.empty(B, dtype=torch.int16, device="cuda")
    for k in range(n_fills):
        lo, hi = k * B, (k + 1) * B
        # the slices of the tensors that meet [lo, hi), in list order
        pieces = []
        for i, n in enumerate(numels):
            a, z = max(lo, int(offs[i])), min(hi, int(offs[i]) + n)
            if a < z:
                pieces.append(tensors[i][a - int(offs[i]):z - int(offs[i])].cpu().numpy().view(np.uint16))
        want = oracle.flat_window(pieces, 0, B)
        lay.pack_bucket(k, b)
        got = b.cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), f"fill {k}"
    lay.close()
