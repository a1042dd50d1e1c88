"""The achievable-bandwidth probes (libzero_probe.so) do what they state:
the step-pattern probe copies p, m, v to the write set and writes the XOR of
the contributions' bits into the slot, over whole tiles and a ragged tail;
the copy probe copies; both report a positive kernel time; bad arguments are
rejected."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n,R", [(1, 1), (1023, 2), (4096, 2), (3 * 4096 + 1029, 2), (70_001, 3), (5000, 16)])
def test_step_pattern_moves_the_step_bytes(n, R):
    from sharded_zero_partition_amd import probe
    print(f"[probe step pattern] n={n} R={R}", flush=True)
    g = torch.Generator(device="cuda").manual_seed(n * 31 + R)
    grads = [torch.randint(-32768, 32767, (n,), dtype=torch.int16, device="cuda", generator=g) for _ in range(R)]
    p, m, v = (torch.randn(n, device="cuda", generator=g) for _ in range(3))
    outs = [torch.full((n,), float("nan"), device="cuda") for _ in range(3)]
    slot = torch.zeros(n, dtype=torch.int16, device="cuda")
    ms = probe.step_pattern(grads, p, m, v, *outs, slot, reps=3)
    torch.cuda.synchronize()
    assert ms > 0
    for a, b in zip((p, m, v), outs):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    want = grads[0].cpu().numpy().view(np.uint16).copy()
    for x in grads[1:]:
        want ^= x.cpu().numpy().view(np.uint16)
    assert np.array_equal(slot.cpu().numpy().view(np.uint16), want)


@pytest.mark.parametrize("nbytes", [16, 4096, 16 * 1024 + 48, (1 << 22) + 16 * 7])
def test_copy_probe_copies(nbytes):
    from sharded_zero_partition_amd import probe
    print(f"[probe copy] bytes={nbytes}", flush=True)
    src = torch.randint(0, 255, (nbytes,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    assert probe.copy(src, dst, reps=2) > 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_argument_errors():
    import ctypes
    from sharded_zero_partition_amd import probe
    x = torch.zeros(64, dtype=torch.uint8, device="cuda")
    y = torch.zeros(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(RuntimeError, match="multiple of 16"):
        probe.copy(x[:40], y[:40])
    ms = ctypes.c_float()
    assert probe.lib.zero_probe_copy(x.data_ptr() + 8, y.data_ptr(), 32, 1, None, ctypes.byref(ms)) == -1
    f = torch.zeros(16, device="cuda")
    ptrs = (ctypes.c_void_p * 1)(x.data_ptr())
    assert probe.lib.zero_probe_step_pattern(ptrs, 0, f.data_ptr(), f.data_ptr(), f.data_ptr(), f.data_ptr(),
                                             f.data_ptr(), f.data_ptr(), x.data_ptr(), 16, 1, None,
                                             ctypes.byref(ms)) == -1
