"""GPU parity of the fused shard step (through the C ABI) against the CPU
oracle: ragged sizes spanning several tiles, every contribution count path,
both state modes, every slot alignment class, the overflow/skip path, fp16
subnormals, padding, weight decay and the empty shard."""

import numpy as np
import pytest
import torch

import oracle
from gpu_harness import SENTINEL, Lockstep, host_contribs

pytestmark = pytest.mark.gpu

HP = oracle.AdamHP(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def _p0(rng, S):
    return torch.from_numpy(rng.standard_normal(S, dtype=np.float32) * np.float32(0.02))


@pytest.mark.parametrize("pingpong", [True, False], ids=["pingpong", "inplace"])
@pytest.mark.parametrize("R", [1, 2, 3, 4, 7, 9, 16])
@pytest.mark.parametrize("S", [1, 7, 8, 9, 1024, 1025, 4093, 4096, 3 * 65536 + 5])
def test_small_shards(S, R, pingpong):
    rng = np.random.default_rng(1000 * S + 10 * R + int(pingpong))
    ls = Lockstep(_p0(rng, S), R, HP, 1024.0, pingpong, slot_offset=8, slot_tail=9)
    for _ in range(3):
        ls.step(host_contribs(rng, S, R, 1024.0))
    ls.check_sentinels()
    assert ls.ts == [1, 2, 3]
    assert ls.bit_exact


@pytest.mark.parametrize("offset", [0, 1, 2, 3, 4, 6])
def test_slot_alignment_classes(offset):
    """The slot may start at any element of the gather buffer (odd S makes
    odd rank offsets): 16-, 8-, 4- and 2-byte aligned store paths."""
    rng = np.random.default_rng(77 + offset)
    S = 70001
    ls = Lockstep(_p0(rng, S), 2, HP, 1024.0, True, slot_offset=offset, slot_tail=5)
    for _ in range(2):
        ls.step(host_contribs(rng, S, 2, 1024.0))
    ls.check_sentinels()
    assert ls.bit_exact


@pytest.mark.parametrize("pingpong", [True, False], ids=["pingpong", "inplace"])
@pytest.mark.parametrize("where", ["first", "last", "tail", "middle"])
@pytest.mark.parametrize("value", [0x7C00, 0xFC00, 0x7E00])
def test_overflow_skips_step(pingpong, where, value):
    rng = np.random.default_rng(5)
    S, R = 50_003, 3
    ls = Lockstep(_p0(rng, S), R, HP, 65536.0, pingpong, slot_offset=3)
    ls.step(host_contribs(rng, S, R, 65536.0))
    before = [x.clone() for x in ls.state.live()] + [ls.slot.clone()]
    c = host_contribs(rng, S, R, 65536.0)
    idx = {"first": 0, "last": S - 1, "tail": S - 2, "middle": S // 2}[where]
    c[1][idx] = int(np.array(value, dtype=np.uint16).view(np.int16))
    assert ls.step(c) == 1
    after = list(ls.state.live()) + [ls.slot]
    for a, b in zip(before, after):
        assert torch.equal(a.view(torch.int32) if a.dtype == torch.float32 else a,
                           b.view(torch.int32) if b.dtype == torch.float32 else b)
    assert ls.scaler.scale == 32768.0 and ls.state.t == 1
    ls.step(host_contribs(rng, S, R, 32768.0))
    assert ls.flags == [0, 1, 0] and ls.ts == [1, 1, 2]
    ls.check_sentinels()
    assert ls.bit_exact


def test_fp16_subnormal_contributions():
    rng = np.random.default_rng(9)
    S, R = 65_539, 2
    ls = Lockstep(_p0(rng, S), R, HP, 1.0, True)
    for _ in range(3):
        c = []
        for _ in range(R):
            bits = rng.integers(0, 0x0400, size=S, dtype=np.uint16)   # subnormals and zeros
            bits |= (rng.integers(0, 2, size=S, dtype=np.uint16) << 15)
            c.append(torch.from_numpy(bits.view(np.int16)).to("cuda"))
        ls.step(c)
    assert ls.bit_exact


def test_padding_stays_zero():
    rng = np.random.default_rng(10)
    S, real = 4096 + 13, 4000
    p0 = _p0(rng, S)
    p0[real:] = 0
    ls = Lockstep(p0, 2, HP, 1024.0, True)
    for _ in range(3):
        c = host_contribs(rng, S, 2, 1024.0)
        for x in c:
            x[real:] = 0
        ls.step(c)
    p, m, v = ls.state.live()
    assert not p[real:].any() and not m[real:].any() and not v[real:].any()
    assert not ls.slot[real:].any()
    assert ls.bit_exact


@pytest.mark.parametrize("pingpong", [True, False], ids=["pingpong", "inplace"])
def test_weight_decay(pingpong):
    rng = np.random.default_rng(11)
    S = 30_001
    hp = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01)
    ls = Lockstep(_p0(rng, S), 2, hp, 1024.0, pingpong)
    for _ in range(4):
        ls.step(host_contribs(rng, S, 2, 1024.0))
    assert ls.bit_exact


def test_many_contributions_and_repeated_inputs():
    """R = 16 (the largest count) and aliased contribution buffers."""
    rng = np.random.default_rng(12)
    S = 9_999
    ls = Lockstep(_p0(rng, S), 16, HP, 1024.0, False)
    base = host_contribs(rng, S, 4, 1024.0)
    ls.step([base[i % 4] for i in range(16)])
    assert ls.bit_exact


def test_empty_shard():
    import sharded_zero_partition_amd as zp
    e = torch.empty(0, dtype=torch.float32, device="cuda")
    st = zp.ShardState(e, e.clone(), e.clone())
    sc = zp.LossScaler.make(1024.0)
    hpc = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    g = torch.empty(0, dtype=torch.int16, device="cuda")
    assert zp.shard_step(st, [g, g], hpc, sc, g) == 0
    assert st.t == 1 and sc.good_steps == 1


def test_errors_leave_state_untouched():
    import sharded_zero_partition_amd as zp
    S = 1024
    p = torch.zeros(S, device="cuda")
    st = zp.ShardState(p, torch.zeros_like(p), torch.zeros_like(p))
    sc = zp.LossScaler.make(1024.0)
    hpc = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    g = torch.zeros(S + 8, dtype=torch.int16, device="cuda")
    slot = torch.full((S,), SENTINEL, dtype=torch.int16, device="cuda")
    with pytest.raises(zp.ZeroError, match="ALIGNMENT"):
        zp.shard_step(st, [g[1:S + 1]], hpc, sc, slot)     # 2-byte aligned gradient
    bad_hp = zp.AdamHParams(1e-4, 1.0, 0.999, 1e-8, 0.0)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        zp.shard_step(st, [g[:S]], bad_hp, sc, slot)
    with pytest.raises(zp.ZeroError, match="INVALID_ARG"):
        zp.shard_step(st, [g[:S]], hpc, sc, p.view(torch.int16)[:S])   # slot overlaps p
    assert st.t == 0 and sc.scale == 1024.0 and not p.any()
    assert int((slot != SENTINEL).sum()) == 0


def test_kernel_timing_api():
    """zero_set_kernel_timing / zero_last_kernel_ms: STATE before anything is
    timed, a positive time after a timed step, STATE again once re-enabled."""
    import sharded_zero_partition_amd as zp
    rng = np.random.default_rng(13)
    S = 1 << 20
    ls = Lockstep(_p0(rng, S), 2, HP, 1024.0, True)
    zp.set_kernel_timing(True)
    with pytest.raises(zp.ZeroError, match="STATE"):
        zp.last_kernel_ms()
    ls.step(host_contribs(rng, S, 2, 1024.0))
    ms = zp.last_kernel_ms()
    assert 0.0 < ms < 1000.0
    zp.set_kernel_timing(True)
    with pytest.raises(zp.ZeroError, match="STATE"):
        zp.last_kernel_ms()
    assert zp.kernel_times() == []
    zp.set_kernel_timing(False)
    ls.step(host_contribs(rng, S, 2, 1024.0))      # untimed calls still work
    assert ls.bit_exact


def test_kernel_times_back_to_back():
    """zero_kernel_times: one duration per call timed back to back, oldest
    first, the last one equal to zero_last_kernel_ms; cleared by disabling."""
    import torch
    import sharded_zero_partition_amd as zp
    rng = np.random.default_rng(14)
    S = 1 << 20
    p0 = _p0(rng, S).cuda()
    st = zp.ShardState(p0, torch.zeros_like(p0), torch.zeros_like(p0),
                       torch.empty_like(p0), torch.empty_like(p0), torch.empty_like(p0))
    g = [torch.zeros(S, dtype=torch.int16, device="cuda") for _ in range(2)]
    slot = torch.empty(S, dtype=torch.int16, device="cuda")
    sc = zp.LossScaler.make(1024.0)
    hpc = zp.AdamHParams(1e-4, 0.9, 0.999, 1e-8, 0.0)
    zp.set_kernel_timing(True)
    for _ in range(5):
        assert zp.shard_step(st, g, hpc, sc, slot) == 0
    times = zp.kernel_times()
    assert len(times) == 5 and all(0.0 < t < 1000.0 for t in times)
    assert zp.last_kernel_ms() == times[-1]
    zp.set_kernel_timing(False)
    assert zp.kernel_times() == [] and st.t == 5


@pytest.mark.parametrize("pingpong", [True, False], ids=["pingpong", "inplace"])
def test_prepared_step_matches_shard_step(pingpong):
    """PreparedStep: the same results, bit for bit, as shard_step on a copy of
    the state, over taken and skipped steps, with cur/t written back."""
    import torch
    import sharded_zero_partition_amd as zp
    rng = np.random.default_rng(15)
    S, R = 70_001, 2
    p0 = _p0(rng, S).cuda()

    def make():
        alt = [torch.empty_like(p0) for _ in range(3)] if pingpong else [None] * 3
        return zp.ShardState(p0.clone(), torch.zeros_like(p0), torch.zeros_like(p0), *alt)

    sa, sb = make(), make()
    ga = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(R)]
    gb = [torch.empty(S, dtype=torch.int16, device="cuda") for _ in range(R)]
    slot_a = torch.empty(S, dtype=torch.int16, device="cuda")
    slot_b = torch.empty(S, dtype=torch.int16, device="cuda")
    hpc = zp.AdamHParams(1e-3, 0.9, 0.999, 1e-8, 0.01)
    sca, scb = zp.LossScaler.make(1024.0), zp.LossScaler.make(1024.0)
    prepared = zp.PreparedStep(sb, gb, hpc, scb, slot_b)
    for k in range(6):
        contribs = host_contribs(rng, S, R, 1024.0)
        if k == 3:
            contribs[1][S // 2] = 0x7C00          # +inf: this step is skipped
        for g_dev in (ga, gb):
            for r in range(R):
                g_dev[r].copy_(contribs[r])
        fa = zp.shard_step(sa, ga, hpc, sca, slot_a)
        fb = prepared()
        assert fa == fb == (1 if k == 3 else 0)
        assert (sa.t, sa.cur) == (sb.t, sb.cur)
        assert (sca.scale, sca.good_steps) == (scb.scale, scb.good_steps)
        for x, y in zip(sa.live(), sb.live()):
            assert torch.equal(x.view(torch.int32), y.view(torch.int32))
        assert torch.equal(slot_a, slot_b)
    assert sb.t == 5
