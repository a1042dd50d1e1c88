"""The C ABI from plain C: tests/c_consumer.c includes only
include/zero_partition.h, is compiled as strict C99 with warnings as errors
and linked against libzero_partition.so.  It checks the struct sizes a C
compiler lays out against the library's, then prints the layout the library
builds for a tensor list; every figure is compared with the oracle's layout
(host logic only, no device).  Also: the sizing protocol of the segment
queries (CAPACITY with a short array) and argument errors from C."""

import os
import subprocess

import pytest

import oracle.layout as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "c_consumer.c")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(ROOT, "sharded_zero_partition_amd")

ARENA_KINDS = ["param16", "grad16", "master", "momentum", "variance", "master_alt",
               "momentum_alt", "variance_alt", "bucket"] + [f"contrib{r}" for r in range(16)]


@pytest.fixture(scope="module")
def consumer(tmp_path_factory):
    from sharded_zero_partition_amd import build as zbuild
    if not os.path.exists(zbuild.LIB):
        zbuild.build()
    exe = str(tmp_path_factory.mktemp("c_consumer") / "c_consumer")
    subprocess.check_call(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                           "-I", INCLUDE, SRC, "-o", exe, "-L", LIBDIR, "-lzero_partition",
                           f"-Wl,-rpath,{LIBDIR}"])
    return exe


def _run(exe, numels, n_ranks, stage, align, bucket):
    out = subprocess.run([exe, str(n_ranks), str(stage), str(align), str(bucket),
                          *[str(n) for n in numels]], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    return out.stdout.splitlines()


@pytest.mark.parametrize("numels,n_ranks,stage,align,bucket", [
    ([1000, 3, 0, 777, 4096, 5], 6, 2, 8, 300),
    ([10, 20, 30], 4, 0, 1, 0),
    ([1 << 20], 4, 3, 1, 1 << 16),
    ([5, 1, 300, 8, 77, 1024, 3], 5, 1, 64, 777),
    ([0, 0, 9], 3, 3, 1, 4),
])
def test_c_program_sees_the_oracle_layout(consumer, numels, n_ranks, stage, align, bucket):
    lines = _run(consumer, numels, n_ranks, stage, align, bucket)
    assert lines[0] == "sizes OK"
    lay = OL.partition_layout(numels, n_ranks, stage, align, bucket)
    rb = lay.rank_bytes()
    recs = {}
    for ln in lines[1:]:
        k, *vals = ln.split(" ")
        recs.setdefault(k, []).append(vals)
    info = [int(x) for x in recs["info"][0]]
    assert info == [lay.psi, lay.shard, lay.padded, lay.padding, lay.n_fills, len(lay.segments),
                    rb["param16"], rb["grad16"], rb["master"], rb["momentum"], rb["variance"],
                    rb["total"]]
    assert [[int(x) for x in v] for v in recs["offset"]] == [[i, o] for i, o in enumerate(lay.offsets)]
    for r, v in enumerate(recs["rank"]):
        b, re_, e, n = (int(x) for x in v[1:])
        assert (b, e) == (r * lay.shard, (r + 1) * lay.shard)
        assert re_ == max(b, min(e, lay.psi))
        assert n == len(lay.rank_segments(r))
    segs = [[int(x) for x in v] for v in recs.get("seg", [])]
    assert segs == [[s.tensor, s.owner, s.tensor_off, s.flat_off, s.length, s.shard_off,
                     s.fill, s.bucket_off] for s in lay.segments]
    arena = [int(x) for x in recs["arena"][0]]
    plan, total = OL.arena_plan(lay, True, 2, bucket > 0, 1 << 21)
    assert arena[0] == total
    got = {ARENA_KINDS[arena[i]]: (arena[i + 1], arena[i + 2]) for i in range(1, len(arena), 3)}
    assert got == plan
    # errors from C: the documented status codes and a message
    errs = [v for v in recs["error"]]
    codes = [int(v[0]) for v in errs]
    assert codes[-3:] == [-1, -1, -1]
    assert all(len(" ".join(v[1:])) > 0 for v in errs)
    if lay.segments:
        assert codes[0] == -3             # CAPACITY with one slot too few
