"""Partition layout, stage memory model and bucket pack -- plain Python oracle.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke entry and the
benchmark's CPU-baseline leg, never by the product library.

Source: the ZeRO explainer page ("ZeRO: Memory Optimizations Toward Training
Trillion Parameter Models", azimuth.plus):
  * model-states paragraph: per parameter, 2 bytes of fp16
    parameter, 2 bytes of fp16 gradient, and 12 bytes of fp32 Adam state
    (4 master copy + 4 momentum + 4 variance), 16 bytes in all.
  * core-idea paragraph: the model states are partitioned across the N ranks
    rather than replicated.
  * Stage 1 (P_os) paragraph: each rank keeps 1/N of
    the optimizer state.
  * Stage 2 (P_os+g) paragraph: each rank also keeps only
    the gradient slice matching its optimizer partition.
  * Stage 3 (P_os+g+p) paragraph: each rank also keeps
    only 1/N of the fp16 parameters.
  * constant-size buffers paragraph (ZeRO-R): many small tensors are fused into one
    fixed-size buffer whose size does not depend on the model size.

Readings where the page is silent:
  * the model states are flattened in tensor-list order with no per-tensor
    padding; the flat vector is cut into N equal shards of S elements, S the
    smallest multiple of the alignment A with N*S >= Psi; rank r owns
    [r*S, (r+1)*S) and indices >= Psi are padding;
  * the bucket of B elements holds the consecutive window [k*B, (k+1)*B) of
    the flat gradient stream ("fill" k); positions past Psi are zero;
  * replicated kinds are counted over the unpadded Psi, partitioned kinds
    over the padded shard S.

All integer work uses Python integers, which cannot overflow.
"""

from dataclasses import dataclass, field
from typing import List, Sequence

import numpy as np

# bytes per element of each model-state kind, in this order
KINDS = ("param16", "grad16", "master", "momentum", "variance")
KIND_BYTES = {"param16": 2, "grad16": 2, "master": 4, "momentum": 4, "variance": 4}

# which kinds are partitioned (S elements per rank) at each stage; the others
# are replicated (Psi elements on every rank)
PARTITIONED = {
    0: set(),                                                   # plain data parallelism
    1: {"master", "momentum", "variance"},                      # P_os
    2: {"grad16", "master", "momentum", "variance"},            # P_os+g
    3: {"param16", "grad16", "master", "momentum", "variance"},  # P_os+g+p
}


@dataclass
class Segment:
    tensor: int
    owner: int
    tensor_off: int
    flat_off: int
    length: int
    shard_off: int
    fill: int          # -1 when no bucket plan was requested
    bucket_off: int    # -1 when no bucket plan was requested

    def as_tuple(self):
        return (self.tensor, self.owner, self.tensor_off, self.flat_off,
                self.length, self.shard_off, self.fill, self.bucket_off)


@dataclass
class Layout:
    numels: List[int]
    n_ranks: int
    stage: int
    align: int
    bucket: int
    psi: int = 0
    offsets: List[int] = field(default_factory=list)
    shard: int = 0
    n_fills: int = 0
    segments: List[Segment] = field(default_factory=list)

    @property
    def padded(self) -> int:
        return self.n_ranks * self.shard

    @property
    def padding(self) -> int:
        return self.padded - self.psi

    def rank_range(self, r: int):
        """(begin, real_end, end): rank r owns [begin, end), of which
        [begin, real_end) are model elements and [real_end, end) padding."""
        begin = r * self.shard
        end = (r + 1) * self.shard
        real_end = max(begin, min(end, self.psi))
        return begin, real_end, end

    def rank_bytes(self):
        """Per-rank bytes of each model-state kind for this stage."""
        out = {}
        for kind in KINDS:
            count = self.shard if kind in PARTITIONED[self.stage] else self.psi
            out[kind] = KIND_BYTES[kind] * count
        out["total"] = sum(out[k] for k in KINDS)
        return out

    def rank_segments(self, r: int):
        return [s for s in self.segments if s.owner == r]

    def fill_segments(self, k: int):
        return [s for s in self.segments if s.fill == k]


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def partition_layout(numels: Sequence[int], n_ranks: int, stage: int = 2,
                     align: int = 1, bucket: int = 0, with_segments: bool = True) -> Layout:
    """Flatten the tensor list and partition it into n_ranks equal padded shards."""
    if n_ranks < 1:
        raise ValueError("n_ranks must be >= 1")
    if stage not in PARTITIONED:
        raise ValueError("stage must be 0, 1, 2 or 3")
    if align < 1:
        raise ValueError("align must be >= 1")
    if bucket < 0:
        raise ValueError("bucket must be >= 0")
    numels = [int(n) for n in numels]
    if any(n < 0 for n in numels):
        raise ValueError("tensor sizes must be >= 0")

    lay = Layout(numels=numels, n_ranks=n_ranks, stage=stage, align=align, bucket=bucket)

    # flat offsets: each tensor starts where the previous one ends
    off = 0
    for n in numels:
        lay.offsets.append(off)
        off += n
    lay.psi = off

    # equal shards: ceil(Psi / N) rounded up to a multiple of the alignment
    lay.shard = _ceil_div(_ceil_div(lay.psi, n_ranks), align) * align
    lay.n_fills = _ceil_div(lay.psi, bucket) if bucket > 0 else 0

    # segments: each tensor's flat interval cut at every shard boundary and,
    # with a bucket plan, at every bucket boundary
    for i, n in enumerate(numels if with_segments else ()):
        start = lay.offsets[i]
        end = start + n
        cur = start
        while cur < end:
            owner = cur // lay.shard
            cut = min(end, (owner + 1) * lay.shard)
            if bucket > 0:
                fill = cur // bucket
                cut = min(cut, (fill + 1) * bucket)
                bucket_off = cur - fill * bucket
            else:
                fill = -1
                bucket_off = -1
            lay.segments.append(Segment(
                tensor=i, owner=owner, tensor_off=cur - start, flat_off=cur,
                length=cut - cur, shard_off=cur - owner * lay.shard,
                fill=fill, bucket_off=bucket_off))
            cur = cut
    return lay


def stage_bytes_per_rank(psi: int, n_ranks: int, stage: int, align: int = 1) -> int:
    """Total model-state bytes held by one rank (the memory model)."""
    lay = partition_layout([psi], n_ranks, stage, align, with_segments=False)
    return lay.rank_bytes()["total"]


# ---------------------------------------------------------------------------
# bucket pack
# ---------------------------------------------------------------------------

def flat_window(tensors: Sequence[np.ndarray], lo: int, hi: int) -> np.ndarray:
    """Elements [lo, hi) of the concatenation of the tensors (uint16 bit
    patterns, copied bit for bit); positions past the last tensor are zero."""
    out = np.zeros(max(0, hi - lo), dtype=np.uint16)
    off = 0
    for t in tensors:
        flat = np.asarray(t).reshape(-1).view(np.uint16)
        a = max(off, lo)
        b = min(off + flat.size, hi)
        if a < b:
            out[a - lo:b - lo] = flat[a - off:b - off]
        off += flat.size
    return out


def pack_fill(tensors: Sequence[np.ndarray], fill: int, bucket: int) -> np.ndarray:
    """Fill `fill` of the constant-size bucket: the window
    [fill*bucket, (fill+1)*bucket) of the concatenation of the fp16 tensors
    (given as uint16 bit patterns, copied bit for bit), zeros past the end."""
    return flat_window(tensors, fill * bucket, fill * bucket + bucket)


def owner_range(lay: Layout, fill: int, rank: int):
    """Flat range [lo, hi) of fill `fill` that rank `rank` owns (lo >= hi when
    empty): the intersection of the fill window, the rank's shard and the
    model (padding is never reduced)."""
    lo = max(fill * lay.bucket, rank * lay.shard)
    hi = min((fill + 1) * lay.bucket, (rank + 1) * lay.shard, lay.psi)
    return lo, hi


# ---------------------------------------------------------------------------
# contiguous arena (memory defragmentation paragraph, ZeRO-R)
# ---------------------------------------------------------------------------

ARENA_KINDS = (["param16", "grad16", "master", "momentum", "variance",
                "master_alt", "momentum_alt", "variance_alt", "bucket"]
               + [f"contrib{r}" for r in range(16)])
ARENA_ORDER = (["master", "momentum", "variance", "master_alt", "momentum_alt", "variance_alt",
                "grad16"] + [f"contrib{r}" for r in range(16)] + ["param16", "bucket"])


def arena_plan(lay: Layout, pingpong: bool = False, n_contrib: int = 0,
               with_bucket: bool = False, align_bytes: int = 1 << 21):
    """One rank's buffers laid out in one contiguous block, each starting on
    an align_bytes boundary.  The model-states paragraph fixes the element
    sizes (fp16 parameters and gradients, fp32 master/momentum/variance) and
    the stage paragraphs which of them are 1/N slices:

      param16             S at stage 3, else the padded N*S vector
      grad16              S at stages 2-3, else N*S
      master/momentum/
      variance (+ alt)    S at stages 1-3, else N*S
      contrib0..R-1       S each (the R fp16 contributions of the shard step)
      bucket              B (the constant-size buffer)

    Returns {kind: (offset, bytes)} for the kinds present and the total size.
    Order in the block: fp32 state, alternate state, gradients,
    contributions, parameters, bucket."""
    S, P = lay.shard, lay.padded
    st = lay.stage
    elems = {
        "param16": (S if st >= 3 else P, 2),
        "grad16": (S if st >= 2 else P, 2),
        "master": (S if st >= 1 else P, 4),
        "momentum": (S if st >= 1 else P, 4),
        "variance": (S if st >= 1 else P, 4),
    }
    if pingpong:
        for k in ("master", "momentum", "variance"):
            elems[k + "_alt"] = elems[k]
    for r in range(n_contrib):
        elems[f"contrib{r}"] = (S, 2)
    if with_bucket:
        elems["bucket"] = (lay.bucket, 2)
    plan = {}
    off = 0
    for kind in ARENA_ORDER:
        if kind not in elems:
            continue
        n, size = elems[kind]
        off = -(-off // align_bytes) * align_bytes
        plan[kind] = (off, n * size)
        off += n * size
    return plan, off

