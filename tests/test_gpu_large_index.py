"""Element indices past the signed 32-bit range, on the device.

The shard step runs on one rank's shard of 2^31 + 4099 elements (51.5 GB of
ping-pong fp32 state, 4.3 GB of fp16 gradients, 4.3 GB of fp16 slot), two
steps, compared with the oracle on a sample that includes the elements on
both sides of index 2^31 and the ragged tail.  The bucket pack writes a
bucket of 2^31 + 24 elements from three tensors whose boundaries straddle
index 2^31, compared with the oracle's pack on windows around every
boundary.  Each element's result depends only on its own inputs (and the
global overflow decision), so the samples are exact checks."""

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from gpu_harness import Lockstep
from sharded_zero_partition_amd import workloads as W

pytestmark = pytest.mark.gpu

B31 = 1 << 31


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_shard_step_past_2_31():
    _free()
    w = W.past_2_31()
    S = w.shard
    assert S == B31 + 4099
    rng = np.random.default_rng(31)
    tiles = np.arange(0, S, 1024, dtype=np.int64)           # one element of every 1024-element tile
    idx = np.concatenate([np.arange(8192), np.arange(B31 - 8192, B31 + 4099),
                          rng.integers(0, S, size=200_000),
                          np.minimum(tiles + rng.integers(0, 1024, size=tiles.size), S - 1)])
    sample = np.unique(idx).astype(np.int64)
    print(f"[past_2_31] S={S} R={w.n_contrib} steps={w.steps} sample={sample.size}", flush=True)
    p0 = W.master_init(w, device="cuda")
    hp = oracle.AdamHP(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    ls = Lockstep(p0, w.n_contrib, hp, w.scale, True, slot_offset=8, slot_tail=8, sample=sample)
    del p0
    for step in range(1, w.steps + 1):
        c = [W.grad_contribution(w, step, r, ls.scaler.scale, device="cuda")
             for r in range(w.n_contrib)]
        # every draw is finite (checked over the whole shard on the inputs);
        # the oracle's flag over the sample is then the global one
        for x in c:
            assert bool(torch.isfinite(x.view(torch.float16)).all())
        flag = oracle.overflow_flag([x[torch.from_numpy(sample).cuda()].cpu().numpy().view(np.uint16)
                                     for x in c])
        ls.step(c, global_flag=flag)
        print(f"[past_2_31] step {step}: flag={ls.flags[-1]} t={ls.ts[-1]}", flush=True)
        del c
    ls.check_sentinels()
    assert ls.flags == [0, 0] and ls.ts == [1, 2]
    assert ls.bit_exact
    del ls
    _free()


def test_pack_bucket_past_2_31():
    _free()
    # three tensors: a misaligned one ending 5 elements before 2^31, one
    # crossing 2^31, and a short one ending 3 elements before the bucket end
    numels = [B31 - 5, 13, 13]
    bucket = B31 + 24
    print(f"[pack past 2^31] numels={numels} bucket={bucket}", flush=True)
    wk = W.pack_20k()
    tensors = [W.normal_f32(n, 1e-3, wk.wid, W.KIND_PACK, 7, i, "cuda").to(torch.float16).view(torch.int16)
               for i, n in enumerate(numels)]
    lay = zp.partition_layout(numels, 3, stage=2, bucket=bucket)
    assert lay.info.n_fills == 1
    lay.bind_tensors(tensors)
    out = torch.full((bucket,), 0x5A5A, dtype=torch.int16, device="cuda")
    lay.pack_bucket(0, out)
    torch.cuda.synchronize()
    psi = sum(numels)
    windows = [(0, 4096), (B31 - 4096, B31 + 24), (psi - 64, bucket)]
    rng = np.random.default_rng(32)
    interior = np.unique(rng.integers(0, B31 - 5, size=100_000)).astype(np.int64)
    # the oracle reads host copies of the same tensors, holding the values at
    # the checked positions (the windows and the interior sample) and zeros
    # elsewhere, which no checked position reads
    host = []
    off = 0
    for t, n in zip(tensors, numels):
        keep = np.zeros(n, np.uint16)
        for lo, hi in windows:
            a, b = max(lo, off), min(hi, off + n)
            if a < b:
                keep[a - off:b - off] = t[a - off:b - off].cpu().numpy().view(np.uint16)
        host.append(keep)
        off += n
    gi = torch.from_numpy(interior).cuda()
    host[0][interior] = tensors[0][gi].cpu().numpy().view(np.uint16)
    for lo, hi in windows:
        want = oracle.flat_window(host, lo, hi)
        got = out[lo:hi].cpu().numpy().view(np.uint16)
        assert np.array_equal(got, want), (lo, hi)
    want = np.array([oracle.flat_window(host, int(g), int(g) + 1)[0] for g in interior], np.uint16)
    assert np.array_equal(out[gi].cpu().numpy().view(np.uint16), want)
    del tensors, out, lay
    _free()
