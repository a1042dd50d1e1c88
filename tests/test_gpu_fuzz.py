"""Seeded random cases of the shard step against the oracle, the loss-scale
growth rule on the GPU, and two host threads stepping different shards on
their own streams at the same time."""

import threading

import numpy as np
import pytest
import torch

import oracle
import sharded_zero_partition_amd as zp
from gpu_harness import Lockstep, host_contribs

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
