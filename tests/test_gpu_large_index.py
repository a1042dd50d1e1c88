"""Element indices past the signed 32-bit range, on the device.

The shard step runs on one rank's shard of 2^31 + 4099 elements (51.5 GB of
ping-pong fp32 state, 4.3 GB of fp16 gradients, 4.3 GB of fp16 slot), two
steps, every element compared with the oracle (run over the whole shard in
chunks on the host's threads).  The bucket pack writes a
bucket of 2^31 + 24 elements from three tensors whose boundaries straddle
index 2^31, every element compared with the oracle's pack."""

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
    print(f"[past_2_31] S={S} R={w.n_contrib} steps={w.steps}, every element", flush=True)
    p0 = W.master_init(w, device="cuda")
    hp = oracle.AdamHP(w.lr, w.beta1, w.beta2, w.eps, w.weight_decay)
    ls = Lockstep(p0, w.n_contrib, hp, w.scale, True, slot_offset=8, slot_tail=8)
    del p0
    for step in range(1, w.steps + 1):
        c = [W.grad_contribution(w, step, r, ls.scaler.scale, device="cuda")
             for r in range(w.n_contrib)]
        ls.step(c)
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
    # every element of the bucket against the oracle's fill over host copies
    host = [t.cpu().numpy().view(np.uint16) for t in tensors]
    want = oracle.pack_fill(host, 0, bucket)
    got = out.cpu().numpy().view(np.uint16)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"{bad.size} of {bucket} differ, first at {bad[0]}"
    del tensors, out, lay
    _free()
