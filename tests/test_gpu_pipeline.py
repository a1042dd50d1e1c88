"""GPU tests that chain the path's calls the way one rank of a bucketed
ZeRO-2 step uses them, and the degenerate cases of the method.

  * pipeline: R ranks' ragged gradient tensors -> bucket-by-bucket
    reduce-to-owner into this rank's fp16 gradient shard -> shard step on
    that shard (R = 1) -> fp16 slot of the gather buffer, against the same
    chain in the oracle, for every rank of a small model;
  * N = 1 (one rank owns the whole model), shards made only of padding
    (fewer elements than ranks), a bucket larger than the model (one fill
    with a long zero tail);
  * every call given an explicit side stream rather than torch's current
    one.
"""

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from gpu_harness import Lockstep
from oracle import layout as OL

pytestmark = pytest.mark.gpu

HP = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8)


def _rank_lists(rng, numels, R, scale):
    lists = []
    for _ in range(R):
        lst = []
        for n in numels:
            x = (rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3 * scale)).astype(np.float16)
            lst.append(torch.from_numpy(x.view(np.int16)).cuda())
        lists.append(lst)
    return lists


@pytest.mark.parametrize("n_ranks,align,bucket", [(4, 1, 1000), (3, 8, 4096), (5, 64, 777)])
def test_bucketed_stage2_step_every_rank(n_ranks, align, bucket):
    rng = np.random.default_rng(n_ranks * 100 + align)
    numels = [3000, 7, 1, 12345, 640, 0, 2049, 99]
    R, scale, steps = 3, 1024.0, 3
    lay = zp.partition_layout(numels, n_ranks, stage=2, align=align, bucket=bucket)
    olay = OL.partition_layout(numels, n_ranks, 2, align, bucket)
    S = olay.shard
    p_full = np.zeros(olay.padded, np.float32)
    p_full[:olay.psi] = rng.standard_normal(olay.psi, dtype=np.float32) * np.float32(0.02)
    gather = torch.from_numpy(p_full.astype(np.float16).view(np.int16)).cuda()
    ranks = []
    for r in range(n_ranks):
        ls = Lockstep(torch.from_numpy(p_full[r * S:(r + 1) * S].copy()), 1, HP, scale, r % 2 == 0,
                      gather=gather, slot_offset=r * S, slot_tail=gather.numel() - (r + 1) * S)
        ranks.append(ls)
    for step in range(steps):
        lists = _rank_lists(rng, numels, R, scale)
        lay.bind_contributions(lists)
        host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
        for r, ls in enumerate(ranks):
            # this rank's fp16 gradient shard, filled bucket by bucket; padding 0
            gshard = torch.zeros(S, dtype=torch.int16, device="cuda")
            want = np.zeros(S, np.uint16)
            for k in range(olay.n_fills):
                lay.reduce_to_owner(k, r, gshard)
                off, vals = oracle.reduce_to_owner(host, olay, k, r)
                want[off:off + vals.size] = vals
            assert np.array_equal(gshard.cpu().numpy().view(np.uint16), want), (step, r)
            ls.step([gshard])
        assert all(ls.bit_exact for ls in ranks)
    # every slot of the gather buffer now holds fp16 of its rank's master
    for r, ls in enumerate(ranks):
        assert np.array_equal(gather[r * S:(r + 1) * S].cpu().numpy().view(np.uint16), ls.out16)


def test_single_rank_owns_everything():
    numels = [5000, 3, 70001]
    lay = zp.partition_layout(numels, 1, stage=3)
    assert lay.info.shard_elems == sum(numels) and lay.info.padding == 0
    assert lay.info.bytes_total == 16 * sum(numels) // 1
    rng = np.random.default_rng(1)
    S = sum(numels)
    ls = Lockstep(torch.from_numpy(rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)), 2, HP,
                  1024.0, True)
    for _ in range(2):
        c = [torch.from_numpy((rng.standard_normal(S, dtype=np.float32) * np.float32(1.0))
                              .astype(np.float16).view(np.int16)).cuda() for _ in range(2)]
        ls.step(c)
    assert ls.bit_exact


def test_all_padding_shard():
    """Fewer elements than ranks with alignment 64: the last ranks own only
    padding; their step runs, stays zero and writes zeros to the slot."""
    lay = zp.partition_layout([3, 2], 8, stage=2, align=64)
    info = lay.info
    assert info.shard_elems == 64 and info.psi == 5
    b, real_end, e = lay.rank_range(7)
    assert real_end == b                       # nothing but padding
    S = info.shard_elems
    ls = Lockstep(torch.zeros(S), 2, HP, 1024.0, True)
    for _ in range(3):
        ls.step([torch.zeros(S, dtype=torch.int16, device="cuda")] * 2)
    p, m, v = ls.state.live()
    assert not p.any() and not m.any() and not v.any() and not ls.slot.any()
    assert ls.ts == [1, 2, 3] and ls.bit_exact


def test_bucket_larger_than_model():
    numels = [17, 1, 300]
    rng = np.random.default_rng(3)
    tensors = [torch.from_numpy(rng.integers(0, 1 << 16, size=n, dtype=np.uint16).view(np.int16)).cuda()
               for n in numels]
    lay = zp.partition_layout(numels, 2, stage=2, bucket=1 << 20)
    assert lay.info.n_fills == 1
    lay.bind_tensors(tensors)
    bucket = torch.full((1 << 20,), 0x1111, dtype=torch.int16, device="cuda")
    assert lay.pack_bucket(0, bucket) == 318
    got = bucket.cpu().numpy().view(np.uint16)
    want = oracle.pack_fill([t.cpu().numpy().view(np.uint16) for t in tensors], 0, 1 << 20)
    assert np.array_equal(got, want) and not got[318:].any()


def test_every_call_on_an_explicit_side_stream():
    """Each call of the path given an explicit side stream (not torch's
    current one): pack, reduce-to-owner, owner step and shard step, each
    checked bit for bit against the oracle once that stream has drained."""
    rng = np.random.default_rng(77)
    numels = [3000, 7, 1, 12345, 640, 0, 2049, 99]
    n_ranks, bucket, R, scale = 3, 1000, 2, 1024.0
    hpc = zp.AdamHParams(HP.lr, HP.beta1, HP.beta2, HP.eps, HP.weight_decay)
    lay = zp.partition_layout(numels, n_ranks, stage=2, bucket=bucket)
    olay = OL.partition_layout(numels, n_ranks, 2, 1, bucket)
    S = olay.shard
    lists = _rank_lists(rng, numels, R, scale)
    host = [[t.cpu().numpy().view(np.uint16) for t in lst] for lst in lists]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()

    lay.bind_tensors(lists[0], stream=s)
    bucket_t = torch.zeros(bucket, dtype=torch.int16, device="cuda")
    torch.cuda.synchronize()
    for k in range(olay.n_fills):
        lay.pack_bucket(k, bucket_t, stream=s)
        s.synchronize()
        want = OL.pack_fill(host[0], k, bucket)
        assert np.array_equal(bucket_t.cpu().numpy().view(np.uint16), want), k

    lay.bind_contributions(lists, stream=s)
    for r in range(n_ranks):
        gshard = torch.zeros(S, dtype=torch.int16, device="cuda")
        torch.cuda.synchronize()
        want = np.zeros(S, np.uint16)
        for k in range(olay.n_fills):
            lay.reduce_to_owner(k, r, gshard, stream=s)
            off, vals = oracle.reduce_to_owner(host, olay, k, r)
            want[off:off + vals.size] = vals
        s.synchronize()
        assert np.array_equal(gshard.cpu().numpy().view(np.uint16), want), r

        p0 = rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)
        p = torch.from_numpy(p0).cuda()
        st = zp.ShardState(p, torch.zeros_like(p), torch.zeros_like(p),
                           torch.empty_like(p), torch.empty_like(p), torch.empty_like(p))
        slot = torch.from_numpy(p0.astype(np.float16).view(np.int16)).cuda()
        sc = zp.LossScaler.make(scale)
        ost, osc = oracle.ShardState(p0), oracle.LossScaler(scale)
        out16 = p0.astype(np.float16).view(np.uint16).copy()
        torch.cuda.synchronize()
        flag = lay.owner_step(r, st, hpc, sc, slot, stream=s)
        s.synchronize()
        assert flag == oracle.owner_step(host, olay, r, ost, osc, HP, out16) == 0
        for got, wnt in zip(st.live(), (ost.p, ost.m, ost.v)):
            assert np.array_equal(got.cpu().numpy().view(np.uint32), wnt.view(np.uint32)), r
        assert np.array_equal(slot.cpu().numpy().view(np.uint16), out16), r

        # the fused shard step on the reduced fp16 shard, same side stream
        p1 = torch.from_numpy(p0).cuda()
        st1 = zp.ShardState(p1, torch.zeros_like(p1), torch.zeros_like(p1),
                            torch.empty_like(p1), torch.empty_like(p1), torch.empty_like(p1))
        slot1 = torch.empty(S, dtype=torch.int16, device="cuda")
        sc1 = zp.LossScaler.make(scale)
        ost1, osc1 = oracle.ShardState(p0), oracle.LossScaler(scale)
        out1 = np.zeros(S, np.uint16)
        torch.cuda.synchronize()
        flag = zp.shard_step(st1, [gshard], hpc, sc1, slot1, stream=s)
        s.synchronize()
        assert flag == oracle.shard_step(ost1, [want], osc1, HP, out1) == 0
        for got, wnt in zip(st1.live(), (ost1.p, ost1.m, ost1.v)):
            assert np.array_equal(got.cpu().numpy().view(np.uint32), wnt.view(np.uint32)), r
        assert np.array_equal(slot1.cpu().numpy().view(np.uint16), out1), r
    lay.close()
