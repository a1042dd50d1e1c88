"""Pins for the oracle's reduce, overflow flag, Adam update and loss-scale
control.  Each test fixes the oracle against something other than itself:

  first step      closed form p1 = p0 - lr * g / (|g| + eps) from a zero state
  constant g      closed form p_t = p0 - t * lr * g / (|g| + eps)
  zero g          the state does not move, padding stays zero
  torch Adam      torch.optim.Adam (CPU, fp32) within the scaled tolerance,
                  with and without L2 weight decay
  overflow        brute-force any(!isfinite) over numpy float32 sums; a flagged
                  step leaves every state bit unchanged; the loss-scale trace of
                  the 1T workload (flags 0,1,0,0,0)
  sharded = DP    the concatenated per-rank steps equal the full-vector step
                  bit for bit (the method is a drop-in for data parallelism)
  reduce          R = 2 sums equal the once-rounded double sum; R = 4 sums
                  equal numpy's left-to-right float32 sums; a sum, not a mean
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import layout as OL
from parity import adam_operand_scales, assert_scaled_close

F32 = np.float32
HP = oracle.AdamHP(lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8)


def _contribs(rng, n, R, scale, tiny_frac=0.0):
    out = []
    for _ in range(R):
        x = (rng.standard_normal(n, dtype=F32) * F32(1e-3) * F32(scale)).astype(np.float16)
        if tiny_frac:
            k = int(n * tiny_frac)
            idx = rng.choice(n, size=k, replace=False)
            # fp16 subnormals and near-zero values: small |g| separates the
            # eps-outside-sqrt reading from the eps-inside-step-size one
            x[idx] = (rng.integers(1, 64, size=k) * (2.0 ** -24)).astype(np.float16)
        out.append(x.view(np.uint16))
    return out


def _ulp32(x):
    x = np.abs(np.asarray(x, dtype=F32))
    return np.spacing(x).astype(np.float64)


def test_first_step_closed_form():
    rng = np.random.default_rng(1)
    n, R, scale = 200_000, 4, 1024.0
    c = _contribs(rng, n, R, scale, tiny_frac=0.01)
    p0 = rng.standard_normal(n, dtype=F32) * F32(0.02)
    st = oracle.ShardState(p0)
    out16 = np.zeros(n, np.uint16)
    sc = oracle.LossScaler(scale)
    assert oracle.shard_step(st, c, sc, HP, out16) == 0
    # closed form in double precision from the same float32 inputs
    g = sum(x.view(np.float16).astype(np.float64) for x in c) / scale
    lr, eps = float(F32(HP.lr)), float(F32(HP.eps))
    delta = lr * g / (np.abs(g) + eps)
    want = p0.astype(np.float64) - delta
    err = np.abs(st.p.astype(np.float64) - want)
    bound = 0.5 * _ulp32(st.p) + 4 * 2.0 ** -23 * np.abs(delta)
    assert (err <= bound).all(), float((err / bound).max())
    assert st.t == 1
    # the fp16 slot is the new master rounded by numpy's float16 conversion
    assert np.array_equal(out16, st.p.astype(np.float16).view(np.uint16))
    # the alternative reading (eps scaled by 1/sqrt(1-beta2) inside the step
    # size) differs far beyond the bound on the small-gradient elements
    alt = p0.astype(np.float64) - lr * g / (np.abs(g) + eps / np.sqrt(1 - float(F32(HP.beta2))))
    assert (np.abs(st.p - alt) > bound).sum() > 100


def test_constant_gradient_closed_form():
    rng = np.random.default_rng(2)
    n, R, scale, T = 50_000, 2, 1024.0, 10
    c = _contribs(rng, n, R, scale)
    p0 = rng.standard_normal(n, dtype=F32) * F32(0.02)
    st = oracle.ShardState(p0)
    sc = oracle.LossScaler(scale)
    g = sum(x.view(np.float16).astype(np.float64) for x in c) / scale
    lr, eps = float(F32(HP.lr)), float(F32(HP.eps))
    step = lr * g / (np.abs(g) + eps)
    for t in range(1, T + 1):
        oracle.shard_step(st, c, sc, HP)
        want = p0.astype(np.float64) - t * step
        err = np.abs(st.p.astype(np.float64) - want)
        # per step: half an ulp of p for the subtraction, plus relative error
        # of the update growing with the number of roundings in m and v
        bound = t * 0.5 * _ulp32(np.maximum(np.abs(st.p), np.abs(p0))) \
            + (t * (t + 1) + 8 * t) * 2.0 ** -23 * np.abs(step)
        assert (err <= bound).all(), (t, float((err / bound).max()))
    assert st.t == T


def test_zero_gradient_is_inert_and_padding_stays_zero():
    rng = np.random.default_rng(3)
    n = 10_000
    c = [np.zeros(n, np.uint16), np.full(n, 0x8000, np.uint16)]    # +0 and -0
    p0 = rng.standard_normal(n, dtype=F32) * F32(0.02)
    p0[-100:] = 0.0                                                  # padding
    st = oracle.ShardState(p0)
    out16 = np.zeros(n, np.uint16)
    for _ in range(3):
        oracle.shard_step(st, c, oracle.LossScaler(1024.0), HP, out16)
    assert np.array_equal(st.p.view(np.uint32), p0.view(np.uint32))
    assert not st.m.any() and not st.v.any()
    assert not out16[-100:].any()
    assert np.array_equal(out16, p0.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("wd", [0.0, 0.01])
def test_matches_torch_adam(wd):
    rng = np.random.default_rng(4)
    n, T, scale = 100_000, 5, 1024.0
    hp = oracle.AdamHP(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=wd)
    p0 = rng.standard_normal(n, dtype=F32) * F32(0.02)
    st = oracle.ShardState(p0)
    tp = torch.nn.Parameter(torch.from_numpy(p0.copy()))
    # both sides take the hyper-parameters as float32 values (torch would
    # otherwise form 1 - beta2 from the double 0.999, 1.3e-5 away relatively)
    f = lambda x: float(F32(x))  # noqa: E731
    opt = torch.optim.Adam([tp], lr=f(hp.lr), betas=(f(hp.beta1), f(hp.beta2)), eps=f(hp.eps),
                           weight_decay=f(wd), foreach=False, fused=False)
    for t in range(T):
        c = _contribs(rng, n, 1, scale)
        m_prev, v_prev, p_prev = st.m.copy(), st.v.copy(), st.p.copy()
        oracle.shard_step(st, c, oracle.LossScaler(scale), hp)
        g = c[0].view(np.float16).astype(F32) / F32(scale)        # exact (power of two)
        # each step starts torch from the oracle's previous state, so that the
        # comparison judges one update and no divergence carried from earlier
        with torch.no_grad():
            tp.copy_(torch.from_numpy(p_prev))
        if t > 0:
            s = opt.state[tp]
            s["exp_avg"].copy_(torch.from_numpy(m_prev))
            s["exp_avg_sq"].copy_(torch.from_numpy(v_prev))
        tp.grad = torch.from_numpy(g.copy())
        opt.step()
        s = opt.state[tp]
        assert int(s["step"]) == st.t
        # magnitude of the gradient's terms (g and the L2 term can cancel)
        g_mag = np.abs(g).astype(np.float64) + abs(wd) * np.abs(p_prev).astype(np.float64)
        s_m, s_v, s_p = adam_operand_scales(m_prev, v_prev, p_prev, g_mag, st.p, hp.beta1,
                                            hp.beta2, hp.lr, st.t, st.v, hp.eps)
        assert_scaled_close(s["exp_avg"].numpy(), st.m, s_m, f"m step {t + 1}", rtol=2e-6)
        assert_scaled_close(s["exp_avg_sq"].numpy(), st.v, s_v, f"v step {t + 1}", rtol=2e-6)
        assert_scaled_close(tp.detach().numpy(), st.p, s_p, f"p step {t + 1}", rtol=2e-6)


def test_overflow_flag_brute_force_and_skip():
    rng = np.random.default_rng(5)
    n, R = 30_000, 3
    for special in (0x7C00, 0xFC00, 0x7E00, 0x7C01, None):
        c = _contribs(rng, n, R, 1024.0)
        if special is not None:
            i = int(rng.integers(0, n))
            c[int(rng.integers(0, R))][i] = special
        s32 = c[0].view(np.float16).astype(F32)
        with np.errstate(invalid="ignore"):   # 0x7C01 is a signalling NaN
            for x in c[1:]:
                s32 = s32 + x.view(np.float16).astype(F32)
        want = int((~np.isfinite(s32)).any())
        assert oracle.overflow_flag(c) == want == int(special is not None)
        p0 = rng.standard_normal(n, dtype=F32)
        st = oracle.ShardState(p0, m=rng.random(n, dtype=F32), v=rng.random(n, dtype=F32), t=7)
        before = (st.p.copy(), st.m.copy(), st.v.copy())
        out16 = np.full(n, 0x5A5A, np.uint16)
        sc = oracle.LossScaler(4096.0)
        flag = oracle.shard_step(st, c, sc, HP, out16)
        if flag:
            for a, b in zip((st.p, st.m, st.v), before):
                assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
            assert (out16 == 0x5A5A).all() and st.t == 7 and sc.scale == 2048.0
        else:
            assert st.t == 8 and sc.scale == 4096.0 and not (out16 == 0x5A5A).all()


def test_overflow_flag_at_the_ends():
    """A single non-finite sum at the first or the last element, in the first
    or the last contribution, raises the flag (brute force over the sums)."""
    rng = np.random.default_rng(6)
    for n in (1, 2, 17, 4096):
        for where in {0, n - 1}:
            for r in (0, 2):
                c = _contribs(rng, n, 3, 1024.0)
                assert oracle.overflow_flag(c) == 0
                c[r][where] = 0x7E00
                assert oracle.overflow_flag(c) == 1, (n, where, r)


def test_inf_minus_inf_is_flagged():
    c = [np.array([0x7C00, 0x3C00], np.uint16), np.array([0xFC00, 0x3C00], np.uint16)]
    assert oracle.overflow_flag(c) == 1
    assert np.isnan(oracle.reduce(c)[0])


def test_loss_scale_trace_of_1t_workload():
    """Flags 0,1,0,0,0; scale used 65536, 65536, 32768, 32768, 32768; step
    count after each step 1, 1, 2, 3, 4 (inf/NaN injected on step 2)."""
    from sharded_zero_partition_amd import workloads as W
    w = W.zero3_1t()
    n = 1 << 22                                    # a slice of the shard
    w.special_fraction = 3e-6                      # a few specials within the slice
    st = oracle.ShardState(W.master_init(w, n).numpy())
    sc = oracle.LossScaler(w.scale)
    flags, used, ts = [], [], []
    for step in range(1, w.steps + 1):
        c = [W.grad_contribution(w, step, r, sc.scale, n).numpy().view(np.uint16)
             for r in range(w.n_contrib)]
        used.append(sc.scale)
        flags.append(oracle.shard_step(st, c, sc, HP))
        ts.append(st.t)
    assert flags == [0, 1, 0, 0, 0]
    assert used == [65536.0, 65536.0, 32768.0, 32768.0, 32768.0]
    assert ts == [1, 1, 2, 3, 4]


def test_loss_scale_matches_torch_amp_update_scale():
    """The loss-scale control against PyTorch's own dynamic loss-scale update
    (torch._amp_update_scale_, CPU tensors): on an overflow the scale is
    multiplied by the backoff factor and the good-step counter reset; after
    growth_interval consecutive good steps the scale is multiplied by the
    growth factor (kept when that product is not finite) and the counter
    reset.  torch has no floor, so the oracle runs with min_scale = 0.
    Seeded flag sequences with long clean runs and dense overflows, growth
    intervals 1, 2, 3, 7 and 1000, factors other than 2 and 1/2, and scales
    near the top and the bottom of the float32 range (growth into inf, backoff
    into subnormals)."""
    import torch
    rng = np.random.default_rng(11)
    cases = [(65536.0, 2.0, 0.5), (1.0, 3.0, 0.25), (float(np.float32(3.0e38)), 2.0, 0.5),
             (2.0 ** 127, 4.0, 0.5), (2.0 ** -120, 2.0, 0.5), (1024.0, 1.5, 0.75)]
    for interval in (1, 2, 3, 7, 1000):
        for scale0, growth, backoff in cases:
            for p_over in (0.0, 0.0004, 0.05, 0.5):
                n = 2600 if interval == 1000 else 300
                flags = rng.random(n) < p_over
                sc = oracle.LossScaler(scale0, backoff=backoff, growth=growth, min_scale=0.0,
                                       growth_interval=interval)
                ts = torch.tensor([scale0], dtype=torch.float32)
                tg = torch.zeros(1, dtype=torch.int32)
                assert float(ts.item()) == sc.scale
                for i, f in enumerate(flags):
                    with np.errstate(over="ignore"):
                        sc.update(bool(f))
                    torch._amp_update_scale_(ts, tg, torch.tensor([1.0 if f else 0.0]),
                                             growth, backoff, interval)
                    assert (sc.scale, sc.good_steps) == (float(ts.item()), int(tg.item())), \
                        (interval, scale0, growth, backoff, p_over, i)


def test_loss_scale_growth_and_floor():
    sc = oracle.LossScaler(8.0, growth_interval=3, min_scale=2.0)
    for _ in range(3):
        sc.update(False)
    assert sc.scale == 16.0 and sc.good_steps == 0
    for _ in range(5):
        sc.update(True)
    assert sc.scale == 2.0


def test_sharded_step_equals_full_vector_step():
    rng = np.random.default_rng(6)
    numels = [1000, 3, 0, 4097, 512, 77]
    for n_ranks, inject in ((1, False), (4, False), (7, False), (5, True)):
        lay = OL.partition_layout(numels, n_ranks, stage=2, align=8)
        S, NS = lay.shard, lay.padded
        p = np.zeros(NS, F32)
        p[:lay.psi] = rng.standard_normal(lay.psi, dtype=F32) * F32(0.02)
        c = [np.zeros(NS, np.uint16) for _ in range(2)]
        for x in c:
            x[:lay.psi] = (rng.standard_normal(lay.psi, dtype=F32) * F32(1.0)).astype(np.float16).view(np.uint16)
        if inject:
            c[1][int(rng.integers(0, lay.psi))] = 0x7C00
        full = oracle.ShardState(p)
        full_out = np.zeros(NS, np.uint16)
        full_flag = oracle.shard_step(full, c, oracle.LossScaler(1.0), HP, full_out)
        # each rank decides on the global flag (OR of the per-rank flags)
        flags = [oracle.overflow_flag([x[r * S:(r + 1) * S] for x in c]) for r in range(n_ranks)]
        gflag = int(any(flags))
        assert gflag == full_flag == int(inject)
        parts, outs = [], []
        for r in range(n_ranks):
            st = oracle.ShardState(p[r * S:(r + 1) * S])
            o = np.zeros(S, np.uint16)
            oracle.shard_step(st, [x[r * S:(r + 1) * S].copy() for x in c],
                              oracle.LossScaler(1.0), HP, o, flag=gflag)
            parts.append(st)
            outs.append(o)
        for name in ("p", "m", "v"):
            cat = np.concatenate([getattr(s, name) for s in parts])
            assert np.array_equal(cat.view(np.uint32), getattr(full, name).view(np.uint32)), name
        assert np.array_equal(np.concatenate(outs), full_out)
        # padding never moves
        assert not full.p[lay.psi:].any()


def test_reduce_r2_is_once_rounded_double_sum():
    rng = np.random.default_rng(7)
    n = 1 << 20
    a = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    b = rng.integers(0, 1 << 16, size=n, dtype=np.uint16)
    fin = ((a & 0x7C00) != 0x7C00) & ((b & 0x7C00) != 0x7C00)
    a, b = a[fin], b[fin]
    got = oracle.reduce([a, b])
    want = (a.view(np.float16).astype(np.float64) + b.view(np.float16).astype(np.float64)).astype(F32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_reduce_r4_left_to_right_and_is_a_sum():
    rng = np.random.default_rng(8)
    n = 1 << 18
    c = [(rng.standard_normal(n, dtype=F32) * F32(10.0 ** e)).astype(np.float16).view(np.uint16)
         for e in (0, -3, 2, -5)]
    got = oracle.reduce(c)
    want = c[0].view(np.float16).astype(F32)
    for x in c[1:]:
        want = want + x.view(np.float16).astype(F32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    same = oracle.reduce([c[0]] * 4)
    assert np.array_equal(same, c[0].view(np.float16).astype(F32) * F32(4))
