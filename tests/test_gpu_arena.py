"""The contiguous arena on the GPU: one rank's state, alternate set,
contributions and bucket carved out of one allocation per the plan; the
shard step and the pack run on those views bit-exactly against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("stage", [1, 2, 3])
def test_step_and_pack_on_arena(stage):
    rng = np.random.default_rng(50 + stage)
    numels = [40000, 3, 77777, 1, 5000]
    n_ranks, rank, R, B = 4, 3, 2, 1 << 14
    lay = zp.partition_layout(numels, n_ranks, stage=stage, align=8, bucket=B)
    S = lay.info.shard_elems
    plan = lay.arena_plan(pingpong=True, n_contrib=R, with_bucket=True, align_bytes=4096)
    views = zp.carve_arena(plan)
    assert views["_arena"].numel() == plan.total_bytes
    b, real_end, e = lay.rank_range(rank)
    p0 = np.zeros(S, np.float32)
    p0[:real_end - b] = rng.standard_normal(real_end - b, dtype=np.float32) * np.float32(0.02)
    views["master"].copy_(torch.from_numpy(p0))
    views["momentum"].zero_()
    views["variance"].zero_()
    st = zp.ShardState(views["master"], views["momentum"], views["variance"],
                       views["master_alt"], views["momentum_alt"], views["variance_alt"])
    slot = views["param16"][:S] if stage == 3 else views["param16"][rank * S:(rank + 1) * S]
    slot.copy_(torch.from_numpy(p0.astype(np.float16).view(np.int16)))
    hp = oracle.AdamHP(1e-3, 0.9, 0.999, 1e-8, 0.0)
    hpc = zp.AdamHParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
    sc, osc = zp.LossScaler.make(1024.0), oracle.LossScaler(1024.0)
    ost = oracle.ShardState(p0)
    out16 = p0.astype(np.float16).view(np.uint16).copy()
    for _ in range(3):
        cs = []
        for r in range(R):
            x = (rng.standard_normal(S, dtype=np.float32) * np.float32(1.024)).astype(np.float16)
            x[real_end - b:] = 0
            views[f"contrib{r}"].copy_(torch.from_numpy(x.view(np.int16)))
            cs.append(x.view(np.uint16))
        assert zp.shard_step(st, [views[f"contrib{r}"] for r in range(R)], hpc, sc, slot) == 0
        oracle.shard_step(ost, cs, osc, hp, out16)
    for got, want in zip(st.live(), (ost.p, ost.m, ost.v)):
        assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    assert np.array_equal(slot.cpu().numpy().view(np.uint16), out16)
    # the bucket view: pack every fill of the rank's gradient tensors
    tensors = [torch.from_numpy(rng.integers(0, 1 << 16, size=n, dtype=np.uint16).view(np.int16)).cuda()
               for n in numels]
    lay.bind_tensors(tensors)
    host = [t.cpu().numpy().view(np.uint16) for t in tensors]
    for k in range(lay.info.n_fills):
        lay.pack_bucket(k, views["bucket"])
        assert np.array_equal(views["bucket"].cpu().numpy().view(np.uint16), oracle.pack_fill(host, k, B))
