"""Seeded random cases of the shard step against the oracle, of the pack and
the reduce-to-owner over random tensor streams, the loss-scale growth rule on
the GPU, two host threads stepping different shards on their own streams at
the same time, and two host threads packing and reducing on their own
layouts and streams at the same time."""

import threading

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from oracle import layout as OL
from gpu_harness import Lockstep, host_contribs, margin_numels

pytestmark = pytest.mark.gpu


def test_random_cases():
    rng = np.random.default_rng(2024)
    for case in range(40):
        S = int(rng.choice([1, 5, 511, 1023, 1024, 1025, 4096, 33333, 123457]))
        R = int(rng.integers(1, 17))
        pingpong = bool(rng.integers(0, 2))
        off = int(rng.integers(0, 8))
        scale = float(2.0 ** rng.integers(0, 17))
        wd = float(rng.choice([0.0, 0.0, 0.05]))
        hp = oracle.AdamHP(lr=float(rng.choice([1e-4, 1e-3, 3e-2])), beta1=float(rng.choice([0.0, 0.9, 0.95])),
                           beta2=float(rng.choice([0.99, 0.999, 0.9999])), eps=float(rng.choice([1e-8, 1e-6])),
                           weight_decay=wd)
        p0 = torch.from_numpy(rng.standard_normal(S, dtype=np.float32) * np.float32(0.05))
        ls = Lockstep(p0, R, hp, scale, pingpong, slot_offset=off, slot_tail=3)
        for step in range(int(rng.integers(1, 5))):
            c = host_contribs(rng, S, R, ls.scaler.scale, std=float(rng.choice([1e-4, 1e-3, 1e-2])))
            if rng.random() < 0.2:
                c[int(rng.integers(0, R))][int(rng.integers(0, S))] = int(
                    np.array(rng.choice([0x7C00, 0xFC00, 0x7E01]), np.uint16).view(np.int16))
            ls.step(c)
        ls.check_sentinels()
        assert ls.bit_exact, case


def _views(rng, numels, scale=100.0):
    """Device tensors carved from one buffer at random 2-byte offsets (every
    alignment phase), fp16 values of moderate size."""
    gaps = rng.integers(0, 9, size=len(numels))
    total = int(sum(numels) + gaps.sum() + 8)
    vals = (rng.standard_normal(total, dtype=np.float32) * np.float32(scale)).astype(np.float16)
    buf = torch.from_numpy(vals.view(np.int16)).cuda()
    out, off = [], 0
    for n, g in zip(numels, gaps):
        off += int(g)
        out.append(buf[off:off + n])
        off += n
    return out


def test_span_kernels_random_layouts():
    """30 seeded random streams (mixes of empty, tiny, span- and chunk-sized
    and long tensors, half of them with boundaries at the work order's
    decision offsets), rank counts, alignments, bucket sizes and R: every fill
    of the pack and every fill and owner of the reduce-to-owner (shard bases
    at random misalignments) against the oracle, bit for bit."""
    rng = np.random.default_rng(4242)
    sent = 0x6B6B
    for case in range(30):
        if case % 2:
            psi = int(rng.integers(3000, 120000))
            numels = margin_numels(rng, [0], psi)
        else:
            numels = []
            for _ in range(int(rng.integers(1, 120))):
                kind = int(rng.integers(0, 5))
                numels.append(int([0, rng.integers(1, 10), rng.integers(1000, 3000),
                                   2048 * int(rng.integers(1, 4)), rng.integers(1, 30000)][kind]))
            if sum(numels) == 0:
                numels.append(17)
        psi = sum(numels)
        n_ranks = int(rng.integers(1, 7))
        align = int(rng.choice([1, 8, 64]))
        bucket = int(rng.choice([1000, 1024, 4093, 8192, 20487, psi]))
        R = int(rng.integers(1, 9))
        print(f"[span fuzz] case {case}: tensors {len(numels)} psi {psi} ranks {n_ranks} align {align} "
              f"bucket {bucket} R {R}", flush=True)
        lay = zp.partition_layout(numels, n_ranks, stage=2, align=align, bucket=bucket)
        olay = OL.partition_layout(numels, n_ranks, 2, align, bucket)
        # pack
        tensors = _views(rng, numels)
        lay.bind_tensors(tensors)
        host_t = [t.cpu().numpy().view(np.uint16) for t in tensors]
        b = torch.full((bucket,), sent, dtype=torch.int16, device="cuda")
        for k in range(olay.n_fills):
            lay.pack_bucket(k, b)
            got = b.cpu().numpy().view(np.uint16)
            assert np.array_equal(got, oracle.pack_fill(host_t, k, bucket)), (case, k)
        # reduce-to-owner
        lists = [_views(rng, numels) for _ in range(R)]
        lay.bind_contributions(lists)
        host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
        S = olay.shard
        for r in range(n_ranks):
            mis = int(rng.integers(0, 8))
            holder = torch.full((S + 16,), sent, dtype=torch.int16, device="cuda")
            shard = holder[mis:mis + S]
            want = np.full(S, sent, np.uint16)
            for k in range(olay.n_fills):
                n = lay.reduce_to_owner(k, r, shard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                assert n == vals.size
                want[off:off + vals.size] = vals
            got = shard.cpu().numpy().view(np.uint16)
            # a NaN sum's payload bits are not specified: compare NaN-ness there
            nan_w = ((want & 0x7C00) == 0x7C00) & ((want & 0x3FF) != 0)
            nan_g = ((got & 0x7C00) == 0x7C00) & ((got & 0x3FF) != 0)
            assert np.array_equal(nan_w, nan_g), (case, r)
            assert np.array_equal(got[~nan_w], want[~nan_w]), (case, r, int(np.flatnonzero(got != want)[0]))
            h = holder.cpu().numpy().view(np.uint16)
            assert (h[:mis] == sent).all() and (h[mis + S:] == sent).all()
        lay.close()


def test_loss_scale_growth_matches_oracle():
    rng = np.random.default_rng(7)
    S = 3000
    ls = Lockstep(torch.from_numpy(rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)), 2,
                  oracle.AdamHP(), 256.0, True)
    # growth after every 2 good steps; an overflow in between resets the count
    ls.scaler.growth_interval = 2
    ls.oscaler.growth_interval = 2
    plan = [0, 0, 0, 1, 0, 0, 0]
    for bad in plan:
        c = host_contribs(rng, S, 2, ls.scaler.scale)
        if bad:
            c[0][5] = int(np.array(0x7C00, np.uint16).view(np.int16))
        ls.step(c)
    assert ls.flags == plan
    assert ls.scales == [256.0, 256.0, 512.0, 512.0, 256.0, 256.0, 512.0]
    assert ls.bit_exact


def test_two_threads_two_streams():
    rng = np.random.default_rng(9)
    S = [200_003, 150_001]
    runs = [Lockstep(torch.from_numpy(rng.standard_normal(n, dtype=np.float32) * np.float32(0.02)), 2,
                     oracle.AdamHP(), 1024.0, k == 0) for k, n in enumerate(S)]
    inputs = [[host_contribs(rng, n, 2, 1024.0) for _ in range(4)] for n in S]
    # the device work of each thread goes to its own stream
    errors = []

    def work(k):
        try:
            torch.cuda.set_device(0)
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for c in inputs[k]:
                    runs[k].step(c)
        except Exception as e:        # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for r in runs:
        assert r.ts == [1, 2, 3, 4] and r.bit_exact


def test_two_threads_pack_and_reduce():
    """Two host threads, each with its own layout and stream, pack and reduce
    to owner at the same time (the launch planning and kernel timing are
    per call and per thread); every fill and owner against the oracle."""
    rng = np.random.default_rng(10)
    cases = []
    for k in range(2):
        numels = [int(x) for x in rng.choice([1, 7, 300, 2049, 5000, 40000], size=60)]
        bucket = [4093, 20487][k]
        lay = zp.partition_layout(numels, 3, stage=2, align=8, bucket=bucket)
        olay = OL.partition_layout(numels, 3, 2, 8, bucket)
        tensors = _views(rng, numels)
        lists = [_views(rng, numels) for _ in range(2)]
        cases.append((numels, bucket, lay, olay, tensors, lists))
    torch.cuda.synchronize()   # the set-up copies are done before the threads' streams start
    results = [None, None]
    errors = []

    def work(k):
        try:
            torch.cuda.set_device(0)
            numels, bucket, lay, olay, tensors, lists = cases[k]
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                lay.bind_tensors(tensors, stream=s)
                lay.bind_contributions(lists, stream=s)
                fills = []
                b = torch.empty(bucket, dtype=torch.int16, device="cuda")
                for f in range(olay.n_fills):
                    lay.pack_bucket(f, b, stream=s)
                    fills.append(b.clone())
                S = olay.shard
                flat = torch.full((3 * S,), 0x6B6B, dtype=torch.int16, device="cuda")
                for f in range(olay.n_fills):
                    for r in range(3):
                        lay.reduce_to_owner(f, r, flat[r * S:(r + 1) * S], stream=s)
                s.synchronize()
                results[k] = ([x.cpu().numpy().view(np.uint16) for x in fills], flat.cpu().numpy().view(np.uint16))
        except Exception as e:        # reported below
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not errors, errors
    for k in range(2):
        numels, bucket, lay, olay, tensors, lists = cases[k]
        fills, flat = results[k]
        host_t = [t.cpu().numpy().view(np.uint16) for t in tensors]
        for f in range(olay.n_fills):
            assert np.array_equal(fills[f], oracle.pack_fill(host_t, f, bucket)), (k, f)
        host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
        S = olay.shard
        for r in range(3):
            want = np.full(S, 0x6B6B, np.uint16)
            for f in range(olay.n_fills):
                off, vals = oracle.reduce_to_owner(host, olay, f, r)
                want[off:off + vals.size] = vals
            assert np.array_equal(flat[r * S:(r + 1) * S], want), (k, r)
        lay.close()
