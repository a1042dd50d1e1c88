"""Lock-step runner for the GPU parity tests: the HIP shard step (through the
C ABI) and the CPU oracle take the same seeded inputs step by step, and every
step's flag, loss scale, step count, fp32 state and fp16 slot are compared.

Comparison bar (written into the checks below):
  * overflow flag, step count, loss scale, untouched gather slots: exact;
  * fp32 master/momentum/variance: bit-exact (the kernel evaluates the same
    operations in the same order with IEEE rounding), and in any case within
    1e-6 of the operand scale;
  * fp16 slot: bit-exact, and in any case within 1 fp16 ulp.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle
import sharded_zero_partition_amd as zp
from parity import adam_operand_scales, assert_fp16_close, assert_scaled_close

SENTINEL = 0x5A5A

# The span kernels (pack, reduce-to-owner, owner step) give each wave a span
# of 1024 consecutive elements, span w starting at flat index F(w) = s0 +
# 1024 w, and decide which wave takes a span from where tensor boundaries
# fall: boundary b belongs to span w's decision when cs(F(w) - 7) < b <
# F(w + 1) + 8, cs being the start of the 2048-element chunk holding its
# argument.  Boundaries at these offsets from a span start and from a chunk
# start sit on either side of those inequalities.
SPAN_MARGINS = (-9, -8, -7, -6, -1, 0, 1, 6, 7, 8, 9)
CHUNK_MARGINS = (-1, 0, 1, 6, 7, 8)


def margin_numels(rng, span0s, psi, span=1024, chunk=2048):
    """Tensor sizes (summing to psi) whose starts fall at F(w) + d for the
    span grids that start at each flat index in span0s (d from SPAN_MARGINS,
    about every other span), at chunk starts + d (CHUNK_MARGINS), and in a
    few runs of 1..4-element tensors."""
    starts = set()
    for s0 in span0s:
        for f in range(s0 + span, psi, span):
            if rng.random() < 0.5:
                starts.add(f + int(rng.choice(SPAN_MARGINS)))
    for c in range(chunk, psi, chunk):
        if rng.random() < 0.3:
            starts.add(c + int(rng.choice(CHUNK_MARGINS)))
    for _ in range(4):
        p = int(rng.integers(1, psi - 200))
        for _ in range(int(rng.integers(2, 30))):
            p += int(rng.integers(1, 5))
            starts.add(p)
    bounds = [0] + sorted(x for x in starts if 0 < x < psi) + [psi]
    return [b - a for a, b in zip(bounds, bounds[1:])]


def device_state(p0: torch.Tensor, pingpong: bool) -> "zp.ShardState":
    p = p0.to("cuda", torch.float32).contiguous().clone()
    m = torch.zeros_like(p)
    v = torch.zeros_like(p)
    if not pingpong:
        return zp.ShardState(p, m, v)
    # the alternate set starts as NaN so that a read of it would show
    alt = [torch.full_like(p, float("nan")) for _ in range(3)]
    return zp.ShardState(p, m, v, *alt)


class Lockstep:
    """One rank's shard on the device and its oracle twin.

    p0:           initial fp32 master shard (host or device tensor)
    R, hp, scale: contributions per step, Adam hyper-parameters, loss scale
    pingpong:     single-pass ping-pong state or in-place two-pass
    slot_offset:  element offset of the rank's slot inside a gather buffer of
                  slot_offset + S + slot_tail elements pre-filled with SENTINEL
    sample:       None to compare every element, or sorted int64 indices
    """

    def __init__(self, p0, R: int, hp: "oracle.AdamHP", scale: float, pingpong: bool,
                 slot_offset: int = 0, slot_tail: int = 0, sample=None, gather=None):
        self.S = p0.numel()
        self.R = R
        self.hp = hp
        self.hpc = zp.AdamHParams(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay)
        self.scaler = zp.LossScaler.make(scale)
        self.oscaler = oracle.LossScaler(scale)
        self.state = device_state(p0, pingpong)
        if gather is None:
            gather = torch.full((slot_offset + self.S + slot_tail,), SENTINEL,
                                dtype=torch.int16, device="cuda")
        self.gather = gather
        self.slot_offset = slot_offset
        self.slot = gather[slot_offset:slot_offset + self.S]
        self.sample = sample
        p0_host = p0.detach().to("cpu", torch.float32).numpy()
        if sample is not None:
            p0_host = p0_host[sample]
        self.ostate = oracle.ShardState(p0_host)
        # initial slot: fp16 of the master weights (numpy's rounding)
        self.out16 = p0_host.astype(np.float16).view(np.uint16).copy()
        init = torch.from_numpy(p0.detach().to("cpu", torch.float32).numpy()
                                .astype(np.float16).view(np.int16)).to("cuda")
        self.slot.copy_(init)
        self.flags = []
        self.scales = []
        self.ts = []
        self.bit_exact = True

    def _host(self, t: torch.Tensor) -> np.ndarray:
        if self.sample is not None:
            idx = torch.from_numpy(self.sample).to(t.device)
            t = t[idx]
        return t.cpu().numpy()

    def _oracle_step(self, ch, used, global_flag):
        """The oracle's shard step on the host copies, over contiguous chunks
        in parallel threads (its C calls release the GIL): the overflow flag
        of every chunk first (ORed), then, when no chunk overflowed, Adam on
        every chunk.  Each element depends only on its own inputs and the
        shard-wide flag, so this equals one call over the whole shard.  Also
        returns the state before the step and the unscaled gradients, for the
        tolerance fallback (None on a skipped step, which must leave the
        state as it was)."""
        n = ch[0].size
        threads = max(1, min(16, os.cpu_count() or 1))
        cuts = np.linspace(0, n, max(1, min(threads * 4, n // (1 << 18) + 1)) + 1).astype(np.int64)
        parts = [(int(a), int(b)) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]
        st = self.ostate
        with ThreadPoolExecutor(threads) as pool:
            if global_flag is None:
                flag = int(any(pool.map(lambda ab: oracle.overflow_flag([c[ab[0]:ab[1]] for c in ch]), parts)))
            else:
                flag = int(global_flag)
            prev = g = None
            if not flag:
                prev = (np.empty_like(st.p), np.empty_like(st.m), np.empty_like(st.v))
                g = np.empty(n, np.float32)
                inv = np.float32(1.0 / used)

                def work(ab):
                    a, b = ab
                    cc = [c[a:b] for c in ch]
                    for dst, src in zip(prev, (st.p, st.m, st.v)):
                        dst[a:b] = src[a:b]
                    g[a:b] = oracle.reduce(cc) * inv
                    oracle.adam_apply(cc, st.p[a:b], st.m[a:b], st.v[a:b], self.out16[a:b], used,
                                      st.t + 1, self.hp)

                list(pool.map(work, parts))
                st.t += 1
        self.oscaler.update(bool(flag))
        return flag, prev, g

    def step(self, contribs, global_flag=None):
        """contribs: R device int16 tensors of S fp16 patterns.  global_flag:
        the expected overflow decision when only a sample is compared (the
        oracle then applies it to the sampled elements)."""
        used = self.scaler.scale
        assert used == self.oscaler.scale
        flag = zp.shard_step(self.state, contribs, self.hpc, self.scaler, self.slot)
        torch.cuda.synchronize()
        ch = [self._host(c).view(np.uint16) for c in contribs]
        oflag, prev, g = self._oracle_step(ch, used, global_flag)
        assert flag == oflag, f"overflow flag {flag} != oracle {oflag}"
        assert self.state.t == self.ostate.t
        assert self.scaler.scale == self.oscaler.scale
        assert self.scaler.good_steps == self.oscaler.good_steps
        self.flags.append(flag)
        self.scales.append(used)
        self.ts.append(self.state.t)
        self.compare(prev, g)
        return flag

    def _operand_scales(self, prev, g):
        op = self.ostate.p, self.ostate.m, self.ostate.v
        if prev is None:
            return [np.abs(x) for x in op]
        g_mag = np.abs(g).astype(np.float64) + abs(self.hp.weight_decay) * np.abs(prev[0])
        sc = adam_operand_scales(prev[1], prev[2], prev[0], g_mag, op[0], self.hp.beta1,
                                 self.hp.beta2, self.hp.lr, max(self.ostate.t, 1), op[2],
                                 self.hp.eps)
        return sc[2], sc[0], sc[1]

    def compare(self, prev=None, g=None):
        p, m, v = self.state.live()
        op = self.ostate.p, self.ostate.m, self.ostate.v
        scales = None                   # only needed when the bits differ
        for k, (name, dev, want) in enumerate(zip("pmv", (p, m, v), op)):
            got = self._host(dev)
            if not np.array_equal(got.view(np.uint32), want.view(np.uint32)):
                self.bit_exact = False
                if scales is None:
                    scales = self._operand_scales(prev, g)
                assert_scaled_close(got, want, scales[k], f"{name} (state)")
            del got
        slot = self._host(self.slot).view(np.uint16)
        if not np.array_equal(slot, self.out16):
            self.bit_exact = False
            assert_fp16_close(slot, self.out16, "fp16 slot")

    def check_sentinels(self):
        g = self.gather
        if self.slot_offset:
            assert int((g[:self.slot_offset] != SENTINEL).sum()) == 0, "gather buffer before the slot changed"
        tail = g[self.slot_offset + self.S:]
        if tail.numel():
            assert int((tail != SENTINEL).sum()) == 0, "gather buffer after the slot changed"


def host_contribs(rng: np.random.Generator, S: int, R: int, scale: float, std: float = 1e-3):
    """R fp16 contributions fp16(float32(N(0, std)) * scale) drawn on the host
    and copied to the device (int16 views)."""
    out = []
    for _ in range(R):
        x = (rng.standard_normal(S, dtype=np.float32) * np.float32(std) * np.float32(scale))
        out.append(torch.from_numpy(x.astype(np.float16).view(np.int16)).to("cuda"))
    return out
