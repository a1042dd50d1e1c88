"""The product path has no CPU fallback and never reaches the oracle: without
its built library the first use of any call of the path (or an import of the
binding) fails with a clear error, and no source of the package imports the
oracle package."""

import os
import re
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "sharded_zero_partition_amd")


def test_package_sources_never_import_the_oracle():
    pat = re.compile(r"^\s*(import\s+oracle\b|from\s+oracle\b)|\boracle\.", re.M)
    for dirpath, _, files in os.walk(PKG):
        for f in files:
            if f.endswith((".py", ".cpp", ".hpp", ".hip", ".h")):
                with open(os.path.join(dirpath, f)) as fh:
                    text = fh.read()
                assert not pat.search(text), f"{f} refers to the oracle"


def test_import_without_the_library_fails_loudly(tmp_path):
    # a copy of the package's Python files only: no libzero_partition.so
    dst = tmp_path / "sharded_zero_partition_amd"
    dst.mkdir()
    for f in os.listdir(PKG):
        if f.endswith(".py"):
            shutil.copy(os.path.join(PKG, f), dst / f)
    env = dict(os.environ, PYTHONPATH=str(tmp_path))
    for code in ("import sharded_zero_partition_amd as zp; zp.partition_layout([1], 1)",
                 "import sharded_zero_partition_amd as zp; zp.ShardState",
                 "from sharded_zero_partition_amd import binding"):
        out = subprocess.run([sys.executable, "-c", code], cwd=str(tmp_path), env=env,
                             capture_output=True, text=True)
        assert out.returncode != 0, code
        assert "ImportError" in out.stderr and "libzero_partition.so is missing" in out.stderr, code
        assert "no fallback" in out.stderr.lower(), code
