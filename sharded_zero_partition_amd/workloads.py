"""Synthetic workloads for the shard step and the bucket pack, and their
seeded input generators.

This module holds shapes, sizes, value distributions and random draws only --
none of the method's arithmetic.  The same bytes it produces feed both the HIP
path and the CPU checker.

The five workloads (sizes as the method's page motivates them: the GPT-2 1.5B
example of the "Model states" paragraph, the 13B-without-model-parallelism
result and the 1T-on-1024-GPUs analysis of the ZeRO explainer page):

  tiny       Psi = 2^20 in one tensor, N = 4, rank 0, R = 4, scale 1024, 3 steps
  gpt2_1p5b  GPT-2 1.5B tensor list, N = 64, rank 63, R = 2, scale 1024, 10 steps
  zero3_13b  13B GPT-style tensor list, N = 64, rank 63, R = 2, scale 1024,
             5 steps, fp16 output into a 64-slot gather buffer
  pack_20k   20,000 fp16 tensors, sizes log-uniform in [1, 2^22], bucket 2^26,
             N = 16 shard cuts
  zero3_1t   Psi = 1e12 (virtual), N = 1024, rank 1023, R = 2, scale 65536,
             5 steps, 1e-7 of the elements set to +inf/-inf/NaN on step 2

Values: master weights N(0, 0.02) fp32 (standard deviation 0.02); each of the
R gradient contributions is fp16(float32(N(0, 1e-3)) * scale) with
round-to-nearest-even, using the scale in force at that step.

Seeds: seed 0 everywhere.  Arrays of up to 2^25 elements are drawn on the host
with numpy PCG64(SeedSequence(0, spawn_key=(workload, kind, step, index))).
Larger arrays are drawn on the device with torch's generator seeded with a
splitmix64 fold of the same key (fast; both sides still read the same bytes).
"""

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

HOST_RNG_LIMIT = 1 << 25

KIND_MASTER = 0
KIND_GRAD = 1
KIND_SPECIAL = 2
KIND_PACK = 3
KIND_SIZES = 4
KIND_STREAM = 5


def gpt2_tensor_numels(n_layers: int, hidden: int, ffn: int, vocab: int,
                       n_positions: int = 1024) -> List[int]:
    """Parameter tensors of a GPT-2-style decoder in module order: token and
    position embeddings, then per layer ln_1 (w, b), attention qkv (w, b),
    attention projection (w, b), ln_2 (w, b), MLP up (w, b), MLP down (w, b),
    then the final layer norm (w, b).  The LM head is tied to the token
    embedding."""
    h = hidden
    out = [vocab * h, n_positions * h]
    for _ in range(n_layers):
        out += [h, h,                # ln_1
                h * 3 * h, 3 * h,    # c_attn
                h * h, h,            # attn c_proj
                h, h,                # ln_2
                h * ffn, ffn,        # c_fc
                ffn * h, h]          # mlp c_proj
    out += [h, h]                    # ln_f
    return out


def pack_tensor_numels(n_tensors: int = 20000, max_elems: int = 1 << 22,
                       seed: int = 0) -> List[int]:
    """Sizes log-uniform in [1, max_elems]: u ~ U(0, ln(max_elems + 1)),
    size = clip(floor(exp(u)), 1, max_elems)."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(0.0, np.log(max_elems + 1.0), n_tensors)
    return [int(s) for s in np.clip(np.floor(np.exp(u)), 1, max_elems).astype(np.int64)]


@dataclass
class ShardWorkload:
    name: str
    wid: int
    numels: List[int]
    n_ranks: int
    rank: int
    n_contrib: int
    scale: float
    steps: int
    stage: int
    lr: float = 1e-4
    beta1: float = 0.9
    beta2: float = 0.999
    eps: float = 1e-8
    weight_decay: float = 0.0
    align: int = 1
    gather_slots: int = 1              # slots allocated in the gather buffer
    special_step: Optional[int] = None  # 1-based step that gets inf/NaN values
    special_fraction: float = 0.0
    # Sizes, written out per workload as data (the layout computes them; the
    # tests check that it reproduces these numbers):
    psi: int = 0          # elements of the flattened model
    shard: int = 0        # elements per rank's shard
    real: int = 0         # elements of this rank's shard inside the model (the rest is padding)


@dataclass
class PackWorkload:
    name: str
    wid: int
    numels: List[int]
    bucket: int
    n_ranks: int
    psi: int              # elements of the flattened stream (sum of the drawn sizes)
    n_fills: int          # bucket fills that cover the stream


def tiny() -> ShardWorkload:
    return ShardWorkload("tiny", 1, [1 << 20], n_ranks=4, rank=0, n_contrib=4,
                         scale=1024.0, steps=3, stage=2, gather_slots=4,
                         psi=1_048_576, shard=262_144, real=262_144)


def gpt2_1p5b() -> ShardWorkload:
    return ShardWorkload("gpt2_1p5b", 2, gpt2_tensor_numels(48, 1600, 6400, 50257),
                         n_ranks=64, rank=63, n_contrib=2, scale=1024.0, steps=10,
                         stage=2, gather_slots=64,
                         psi=1_557_611_200, shard=24_337_675, real=24_337_675)


def zero3_13b() -> ShardWorkload:
    return ShardWorkload("zero3_13b", 3, gpt2_tensor_numels(40, 5120, 20480, 50257),
                         n_ranks=64, rank=63, n_contrib=2, scale=1024.0, steps=5,
                         stage=3, gather_slots=64,
                         psi=12_848_143_360, shard=200_752_240, real=200_752_240)


def pack_20k() -> PackWorkload:
    return PackWorkload("pack_20k", 4, pack_tensor_numels(), bucket=1 << 26, n_ranks=16,
                        psi=5_481_113_944, n_fills=82)


def zero3_1t() -> ShardWorkload:
    return ShardWorkload("zero3_1t", 5, [10 ** 12], n_ranks=1024, rank=1023, n_contrib=2,
                         scale=65536.0, steps=5, stage=3, gather_slots=1,
                         special_step=2, special_fraction=1e-7,
                         psi=10 ** 12, shard=976_562_500, real=976_562_500)


def past_2_31() -> ShardWorkload:
    """Edge case, not one of the five workloads: a single rank's shard of
    2^31 + 4099 elements, so element indices pass the signed 32-bit range and
    the shard ends in a ragged tail; R = 1, scale 1024, 2 steps."""
    return ShardWorkload("past_2_31", 9, [(1 << 31) + 4099], n_ranks=1, rank=0, n_contrib=1,
                         scale=1024.0, steps=2, stage=3, gather_slots=1,
                         psi=(1 << 31) + 4099, shard=(1 << 31) + 4099, real=(1 << 31) + 4099)


SHARD_WORKLOADS = {w().name: w for w in (tiny, gpt2_1p5b, zero3_13b, zero3_1t)}


# ---------------------------------------------------------------------------
# seeded generators
# ---------------------------------------------------------------------------

def _mix64(*key: int) -> int:
    """splitmix64 fold of a tuple of non-negative integers (seed for torch)."""
    mask = (1 << 64) - 1
    h = 0
    for k in key:
        h = (h + 0x9E3779B97F4A7C15 + (k & mask)) & mask
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & mask
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & mask
        h = z ^ (z >> 31)
    return h & ((1 << 63) - 1)


def host_rng(wid: int, kind: int, step: int, index: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence(0, spawn_key=(wid, kind, step, index))))


def normal_f32(n: int, std: float, wid: int, kind: int, step: int, index: int,
               device=None):
    """n float32 draws of N(0, std).  Returns a torch tensor on `device`
    (numpy-drawn and copied when n <= 2^25, drawn on the device otherwise)."""
    import torch
    if n <= HOST_RNG_LIMIT:
        a = host_rng(wid, kind, step, index).standard_normal(n, dtype=np.float32)
        a *= np.float32(std)
        t = torch.from_numpy(a)
        return t.to(device) if device is not None else t
    if device is None or torch.device(device).type != "cuda":
        raise ValueError("arrays above 2^25 elements are drawn on the GPU")
    g = torch.Generator(device=device)
    g.manual_seed(_mix64(0, wid, kind, step, index))
    t = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    t.mul_(std)
    return t


def master_init(w: ShardWorkload, n: int = None, device=None):
    """fp32 master weights of the rank's shard, N(0, 0.02); padding is 0."""
    n = w.shard if n is None else n
    t = normal_f32(n, 0.02, w.wid, KIND_MASTER, 0, w.rank, device)
    if w.real < n:            # the shard's padding holds zeros
        t[w.real:] = 0
    return t


def grad_contribution(w: ShardWorkload, step: int, index: int, scale: float,
                      n: int = None, device=None):
    """Contribution `index` of step `step` (1-based): fp16 bit patterns
    (torch.int16 view) of fp16(float32(N(0, 1e-3)) * scale)."""
    import torch
    n = w.shard if n is None else n
    t = normal_f32(n, 1e-3, w.wid, KIND_GRAD, step, index, device)
    t.mul_(np.float32(scale).item())
    if w.real < n:            # no gradient over the shard's padding
        t[w.real:] = 0
    h = t.to(torch.float16)
    if w.special_step is not None and step == w.special_step:
        pos, vals = special_positions(w, n)
        for j in range(len(pos)):
            if j % w.n_contrib == index:
                h[int(pos[j])] = float(vals[j])
    return h.view(torch.int16)


def special_positions(w: ShardWorkload, n: int = None) -> Tuple[np.ndarray, np.ndarray]:
    """Positions and values (+inf, -inf, NaN by j mod 3) injected on the
    special step: round(fraction * n) distinct positions; item j goes into
    contribution j mod R."""
    n = w.shard if n is None else n
    k = int(round(w.special_fraction * n))
    rng = host_rng(w.wid, KIND_SPECIAL, w.special_step or 0, w.rank)
    pos = np.sort(rng.choice(n, size=k, replace=False)) if k > 0 else np.zeros(0, np.int64)
    vals = np.array([(np.inf, -np.inf, np.nan)[j % 3] for j in range(k)], dtype=np.float32)
    return pos.astype(np.int64), vals


def pack_sources(w: PackWorkload, device=None, views: bool = False, draw: int = 0):
    """The fp16 gradient tensors of the pack workload, N(0, 1e-3), as a list
    of torch.int16 tensors on `device`.  Drawn in one flat array (host array
    when small) and split into separately allocated tensors, or, with
    views=True, as views of one freshly drawn buffer with a 1..7-element gap
    before each tensor (same distribution and alignment mix, and no
    per-tensor copy at all).  `draw` selects an independent set of values
    with the same shapes (another rank's gradients for the reduce)."""
    import torch
    out = []
    total = w.psi
    if views:
        gaps = host_rng(w.wid, KIND_PACK, 1, 0).integers(1, 8, size=len(w.numels))
        n_buf = total + int(gaps.sum()) + 8
        buf = normal_f32(n_buf, 1e-3, w.wid, KIND_PACK, 2, draw, device).to(torch.float16)
        off = 0
        for n, gap in zip(w.numels, gaps):
            off += int(gap)
            out.append(buf[off:off + n].view(torch.int16))
            off += n
        return out
    if total <= HOST_RNG_LIMIT:
        flat = normal_f32(total, 1e-3, w.wid, KIND_PACK, 0, draw).to(torch.float16)
        if device is not None:
            flat = flat.to(device)
    else:
        flat = normal_f32(total, 1e-3, w.wid, KIND_PACK, 0, draw, device).to(torch.float16)
    off = 0
    for n in w.numels:
        out.append(flat[off:off + n].clone().view(torch.int16))
        off += n
    del flat
    return out


def gradient_stream(numels, wid: int, index: int, scale: float = 1.0, step: int = 1,
                    device=None):
    """Rank `index`'s whole fp16 gradient stream over the tensors `numels`:
    fp16(float32(N(0, 1e-3)) * scale) bit patterns (torch.int16) in one
    buffer, with a 0..7-element gap before each tensor so that every
    alignment phase occurs.  Returns (buffer, starts, views): starts[i]
    (numpy int64) is tensor i's first element in the buffer and views[i] the
    tensor.  The gaps depend on the workload only, the values on (step,
    index)."""
    import torch
    numels = [int(n) for n in numels]
    gaps = host_rng(wid, KIND_STREAM, 0, 0).integers(0, 8, size=len(numels))
    ends = np.cumsum(np.asarray(numels, np.int64) + gaps)
    starts = ends - np.asarray(numels, np.int64)
    n_buf = (int(ends[-1]) if numels else 0) + 8
    t = normal_f32(n_buf, 1e-3, wid, KIND_STREAM, step, index, device)
    t.mul_(np.float32(scale).item())
    buf = t.to(torch.float16).view(torch.int16)
    del t
    views = [buf[int(s):int(s) + n] for s, n in zip(starts, numels)]
    return buf, starts, views
