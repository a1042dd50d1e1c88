"""sharded_zero_partition_amd -- one rank's ZeRO-DP shard step on MI355X (gfx950).

The compute path is libzero_partition.so (C ABI in include/zero_partition.h,
HIP kernels under csrc/); `binding` is its thin ctypes wrapper.  The binding's
names are re-exported here on first use, so `import sharded_zero_partition_amd`
itself does not need the built library, but any call into the path does and
fails loudly (ImportError) when the library is missing -- there is no
fallback.  `workloads` holds the synthetic workload shapes and seeded input
generators; `build` compiles the library.
"""

__all__ = ["partition_layout", "Layout", "ShardState", "shard_step", "PreparedStep", "AdamHParams",
           "LossScaler", "ZeroError", "version", "device_info", "set_kernel_timing",
           "last_kernel_ms", "kernel_times", "carve_arena", "ArenaPlan"]


def __getattr__(name):
    if name in __all__ or name in ("binding", "lib", "Segment", "LayoutInfo", "ShardStateC"):
        import importlib
        binding = importlib.import_module(__name__ + ".binding")
        return binding if name == "binding" else getattr(binding, name)
    raise AttributeError(name)
