"""zero_shard_step_noalloc (the shard step for callers that cannot allocate)
against zero_shard_step, through the C ABI: the same inputs on two separate
states, two calls in a row, the second on a smaller shard, in both state
modes and with an overflow; flags, step counts, loss scales, fp32 state and
the fp16 slot must agree bit for bit."""

import numpy as np
import pytest
import torch

import sharded_zero_partition_amd as zp
from gpu_harness import SENTINEL, device_state

pytestmark = pytest.mark.gpu

HPC = zp.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)


def _contribs(rng, S, R, scale):
    return [torch.from_numpy((rng.standard_normal(S, dtype=np.float32) * np.float32(1e-3 * scale))
                             .astype(np.float16).view(np.int16)).cuda() for _ in range(R)]


def _pair(p0, pingpong, slot_offset):
    S = p0.numel()
    out = []
    for _ in range(2):
        st = device_state(p0, pingpong)
        gather = torch.full((slot_offset + S + 5,), SENTINEL, dtype=torch.int16, device="cuda")
        slot = gather[slot_offset:slot_offset + S]
        slot.copy_(p0.to(torch.float16).view(torch.int16))
        out.append((st, gather, slot, zp.LossScaler.make(1024.0)))
    return out


def _same(a, b):
    (sa, ga, _, ca), (sb, gb, _, cb) = a, b
    assert (sa.t, sa.cur, ca.scale, ca.good_steps) == (sb.t, sb.cur, cb.scale, cb.good_steps)
    for x, y in zip(sa.live(), sb.live()):
        assert torch.equal(x.view(torch.int32), y.view(torch.int32))
    assert torch.equal(ga, gb)


@pytest.mark.parametrize("pingpong", [True, False], ids=["pingpong", "inplace"])
@pytest.mark.parametrize("R", [1, 2, 5])
def test_noalloc_matches_shard_step(pingpong, R):
    rng = np.random.default_rng(100 + R + 10 * pingpong)
    for S, offset in ((3 * 4096 + 1029, 3), (1000, 0)):          # second call: a smaller shard
        print(f"[noalloc] S={S} R={R} pingpong={pingpong}", flush=True)
        p0 = torch.from_numpy(rng.standard_normal(S, dtype=np.float32) * np.float32(0.02)).cuda()
        ref, new = _pair(p0, pingpong, offset)
        for step in range(3):
            c = _contribs(rng, S, R, ref[3].scale)
            if step == 1:
                c[R - 1][S // 2] = 0x7C00                           # overflow: skipped, scale halves
            fa = zp.shard_step(ref[0], c, HPC, ref[3], ref[2])
            fb = zp.shard_step(new[0], c, HPC, new[3], new[2], noalloc=True)
            torch.cuda.synchronize()
            assert fa == fb == int(step == 1)
            _same(ref, new)


def test_noalloc_two_calls_in_a_row_then_smaller():
    """Back-to-back calls on one stream, the second with a smaller input,
    without synchronising in between beyond what each call does itself."""
    rng = np.random.default_rng(7)
    S1, S2 = 200_000, 777
    p1 = torch.from_numpy(rng.standard_normal(S1, dtype=np.float32) * np.float32(0.02)).cuda()
    p2 = torch.from_numpy(rng.standard_normal(S2, dtype=np.float32) * np.float32(0.02)).cuda()
    ref1, new1 = _pair(p1, True, 1)
    ref2, new2 = _pair(p2, True, 2)
    c1, c2 = _contribs(rng, S1, 2, 1024.0), _contribs(rng, S2, 2, 1024.0)
    assert zp.shard_step(new1[0], c1, HPC, new1[3], new1[2], noalloc=True) == 0
    assert zp.shard_step(new2[0], c2, HPC, new2[3], new2[2], noalloc=True) == 0
    assert zp.shard_step(ref1[0], c1, HPC, ref1[3], ref1[2]) == 0
    assert zp.shard_step(ref2[0], c2, HPC, ref2[3], ref2[2]) == 0
    torch.cuda.synchronize()
    _same(ref1, new1)
    _same(ref2, new2)


def test_noalloc_argument_errors_match():
    S = 64
    p0 = torch.zeros(S, device="cuda")
    (st, _, slot, sc), = _pair(p0, True, 0)[:1]
    g = _contribs(np.random.default_rng(1), S, 2, 1024.0)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        zp.shard_step(st, g, zp.AdamHParams(1e-3, 1.0, 0.999, 1e-8, 0.0), sc, slot, noalloc=True)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        zp.shard_step(st, g, HPC, zp.LossScaler.make(1024.0, min_scale=0.0), slot, noalloc=True)
    assert st.t == 0 and sc.scale == 1024.0
