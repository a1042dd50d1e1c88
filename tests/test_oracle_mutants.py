"""Sensitivity of the oracle's pins.

Each case plants one plausible mistake -- a dropped term, a wrong sign, a
swapped coefficient, an off-by-one index, a wrong rounding rule -- into a
copy of one oracle source (the scalar C file, the layout module or the
package's Python part), swaps the copy in for the real one, and runs the
oracle's pins (test_oracle_adam, test_oracle_fp16, test_oracle_layout)
against it.  The case passes when at least one pin fails on the mutant.  The
real oracle sources are never modified; mutants live in pytest's temporary
directory and in memory.

Every substitution must match the source the stated number of times, so a
case that no longer applies to the oracle fails loudly instead of testing
nothing.
"""

import os
import subprocess
import sys
import types
import warnings

import pytest

import oracle
import oracle.layout as real_layout

TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)

import test_oracle_adam as TA      # noqa: E402
import test_oracle_fp16 as TF      # noqa: E402
import test_oracle_layout as TL    # noqa: E402

ORACLE_DIR = os.path.dirname(os.path.abspath(oracle.__file__))


def _pins():
    """(name, callable) for every oracle pin, cheapest first."""
    pins = []
    for mod in (TF, TL, TA):
        for name in dir(mod):
            if not name.startswith("test_"):
                continue
            fn = getattr(mod, name)
            if name == "test_float_to_half_exhaustive":
                continue        # the stratified and random-pattern pins already catch every mutant
            if name == "test_matches_torch_adam":
                pins.append((f"{name}[0.01]", lambda fn=fn: fn(0.01)))
                pins.append((f"{name}[0.0]", lambda fn=fn: fn(0.0)))
            elif "oracle_lib" in fn.__code__.co_varnames[:fn.__code__.co_argcount]:
                pins.append((name, lambda fn=fn: fn(oracle)))
            else:
                pins.append((name, fn))
    slow = {"test_matches_torch_adam[0.0]", "test_loss_scale_trace_of_1t_workload",
            "test_float_to_half_stratified", "test_float_to_half_random_bits"}
    return sorted(pins, key=lambda p: p[0] in slow)


def _first_failing_pin():
    """Run the pins until one fails; return its name, or None when all pass."""
    for name, fn in _pins():
        with warnings.catch_warnings():
            warnings.simplefilter("ignore")
            try:
                fn()
            except Exception:          # an assertion, or the pin's own check raising
                return name
    return None


def _mutate(path, edits):
    """Apply one (old, new, count) substitution, or a list of them in order."""
    with open(path) as f:
        src = f.read()
    for old, new, count in ([edits] if isinstance(edits, tuple) else edits):
        assert src.count(old) == count, f"{os.path.basename(path)}: {old!r} occurs {src.count(old)} times"
        src = src.replace(old, new)
    return src


# ---------------------------------------------------------------------------
# scalar C oracle: fp16 conversions, reduce, overflow flag, Adam
# ---------------------------------------------------------------------------

C_MUTANTS = {
    # Adam (textbook form: both moments, both bias corrections, eps outside sqrt)
    "momentum_uses_beta2": ("float mi = beta1 * m[i]", "float mi = beta2 * m[i]", 1),
    "variance_uses_one_minus_beta1": ("one_minus_b2 * (g * g)", "one_minus_b1 * (g * g)", 1),
    "variance_of_abs_g": ("one_minus_b2 * (g * g)", "one_minus_b2 * fabsf(g)", 1),
    "eps_inside_sqrt": ("sqrtf(vhat) + eps", "sqrtf(vhat + eps)", 1),
    "no_first_moment_bias_correction": ("float mhat = mi / bc1;", "float mhat = mi;", 1),
    "no_second_moment_bias_correction": ("float vhat = vi / bc2;", "float vhat = vi;", 1),
    "bias_correction_step_off_by_one": ("(double)t));\n    float bc2", "(double)(t + 1)));\n    float bc2", 1),
    "ascent_instead_of_descent": ("p[i] - lr * (mhat / denom)", "p[i] + lr * (mhat / denom)", 1),
    "lr_dropped": ("p[i] - lr * (mhat / denom)", "p[i] - (mhat / denom)", 1),
    "gradient_not_unscaled": ("reduce_one(contrib, R, i) * inv_scale;", "reduce_one(contrib, R, i);", 1),
    "weight_decay_sign": ("g = g + wd * p[i];", "g = g - wd * p[i];", 1),
    "weight_decay_ignored": ("if (wd != 0.0f)", "if (0)", 1),
    "momentum_not_stored": ("m[i] = mi;", "m[i] = m[i];", 1),
    "variance_not_stored": ("v[i] = vi;", "v[i] = v[i];", 1),
    "fp16_slot_of_old_master": [("float pi = p[i] - lr", "float p_old = p[i];\n        float pi = p[i] - lr", 1),
                                ("out16[i] = zo_float_to_half(pi);", "out16[i] = zo_float_to_half(p_old);", 1)],
    # reduce and overflow flag
    "reduce_drops_last_contribution": ("for (int32_t r = 1; r < R; ++r)", "for (int32_t r = 1; r < R - 1; ++r)", 1),
    "reduce_skips_first_contribution": ("float sum = zo_half_to_float(contrib[0][i]);",
                                        "float sum = 0.0f * zo_half_to_float(contrib[0][i]);", 1),
    "reduce_is_a_mean": ("    return sum;\n}", "    return sum / (float)R;\n}", 1),
    "reduce_in_fp16": ("sum = sum + zo_half_to_float(contrib[r][i]);",
                       "sum = zo_half_to_float(zo_float_to_half(sum + zo_half_to_float(contrib[r][i])));", 1),
    "flag_misses_nan": ("if (!isfinite(s))", "if (isinf(s))", 1),
    "flag_misses_inf": ("if (!isfinite(s))", "if (isnan(s))", 1),
    "flag_skips_last_element": ("for (int64_t i = 0; i < n; ++i) {\n        float s",
                                "for (int64_t i = 0; i + 1 < n; ++i) {\n        float s", 1),
    # binary16 -> float
    "half_subnormal_scale": ("ldexpf((float)frac, -24)", "ldexpf((float)frac, -25)", 1),
    "half_exponent_bias": ("expo - 25);", "expo - 24);", 1),
    "half_nan_read_as_inf": ("(frac == 0) ? INFINITY : NAN", "INFINITY", 1),
    "half_sign_dropped": ("return sign ? -mag : mag;", "return mag;", 1),
    # float -> binary16 (nearest, ties to even)
    "round_ties_away": ("if (fmodf(whole, 2.0f) != 0.0f)", "if (1)", 1),
    "round_ties_down": ("if (fmodf(whole, 2.0f) != 0.0f)", "if (0)", 1),
    "round_truncates": ("if (frac > 0.5f) {", "if (0) {", 1),
    "subnormal_boundary": ("(floor_log2 < -14) ? -24", "(floor_log2 < -15) ? -24", 1),
    "overflow_at_max_finite": ("if (r >= 65536.0)", "if (r >= 65504.0)", 1),
    "nan_encoded_as_inf": ("return (uint16_t)(sign | 0x7E00);", "return (uint16_t)(sign | 0x7C00);", 1),
    "negative_zero_loses_sign": ("if (a == 0.0f)\n        return sign;", "if (a == 0.0f)\n        return 0;", 1),
}


@pytest.fixture(scope="module")
def real_oracle_lib():
    oracle.build(force=False)
    return oracle.lib()


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_fails_a_pin(name, tmp_path, monkeypatch, real_oracle_lib):
    src = tmp_path / "zero_oracle_mutant.c"
    src.write_text(_mutate(os.path.join(ORACLE_DIR, "zero_oracle.c"), C_MUTANTS[name]))
    so = tmp_path / "libzero_oracle_mutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.load(str(so)))
    caught = _first_failing_pin()
    assert caught is not None, f"C mutant {name!r} passes every pin"


# ---------------------------------------------------------------------------
# Python oracle: layout, memory model, pack window, owner range; loss scale,
# shard/owner step and reduce-to-owner glue
# ---------------------------------------------------------------------------

LAYOUT_MUTANTS = {
    "shard_rounds_down": ("lay.shard = _ceil_div(_ceil_div(lay.psi, n_ranks), align) * align",
                          "lay.shard = _ceil_div(lay.psi // n_ranks, align) * align", 1),
    "shard_ignores_alignment": ("lay.shard = _ceil_div(_ceil_div(lay.psi, n_ranks), align) * align",
                                "lay.shard = _ceil_div(lay.psi, n_ranks)", 1),
    "no_bucket_cut": ("cut = min(cut, (fill + 1) * bucket)", "cut = cut", 1),
    "shard_offset_from_tensor_start": ("shard_off=cur - owner * lay.shard", "shard_off=cur - start", 1),
    "bucket_offset_off_by_one": ("bucket_off = cur - fill * bucket", "bucket_off = cur - fill * bucket + 1", 1),
    "psi_drops_last_tensor": ("lay.psi = off", "lay.psi = off - (numels[-1] if numels else 0)", 1),
    "fp32_state_counted_as_fp16": ('"master": 4, "momentum": 4', '"master": 2, "momentum": 4', 1),
    "stage2_keeps_full_gradients": ('2: {"grad16", "master", "momentum", "variance"}',
                                    '2: {"master", "momentum", "variance"}', 1),
    "stage1_partitions_gradients": ('1: {"master", "momentum", "variance"}',
                                    '1: {"grad16", "master", "momentum", "variance"}', 1),
    "replicated_kinds_count_padding": ("count = self.shard if kind in PARTITIONED[self.stage] else self.psi",
                                       "count = self.shard if kind in PARTITIONED[self.stage] else self.padded", 1),
    "pack_tail_not_zero": ("out = np.zeros(max(0, hi - lo), dtype=np.uint16)",
                           "out = np.full(max(0, hi - lo), 1, dtype=np.uint16)", 1),
    "pack_window_shifted": ("return flat_window(tensors, fill * bucket, fill * bucket + bucket)",
                            "return flat_window(tensors, fill * bucket + 1, fill * bucket + bucket + 1)", 1),
    "window_skips_tensor_offset": ("out[a - lo:b - lo] = flat[a - off:b - off]",
                                   "out[a - lo:b - lo] = flat[a - lo:b - lo][:b - a]", 1),
    "owner_range_takes_padding": ("hi = min((fill + 1) * lay.bucket, (rank + 1) * lay.shard, lay.psi)",
                                  "hi = min((fill + 1) * lay.bucket, (rank + 1) * lay.shard)", 1),
    "owner_range_ignores_fill": ("lo = max(fill * lay.bucket, rank * lay.shard)",
                                 "lo = rank * lay.shard", 1),
    # contiguous arena (memory defragmentation paragraph)
    "arena_params_partitioned_at_stage2": ('"param16": (S if st >= 3 else P, 2)',
                                           '"param16": (S if st >= 2 else P, 2)', 1),
    "arena_grads_partitioned_at_stage1": ('"grad16": (S if st >= 2 else P, 2)',
                                          '"grad16": (S if st >= 1 else P, 2)', 1),
    "arena_alternates_as_fp16": ('elems[k + "_alt"] = elems[k]',
                                 'elems[k + "_alt"] = (elems[k][0], 2)', 1),
    "arena_buffers_unaligned": ("off = -(-off // align_bytes) * align_bytes", "off = off", 1),
}

INIT_MUTANTS = {
    "backoff_grows_scale": ("np.float32(self.scale * self.backoff)", "np.float32(self.scale * self.growth)", 1),
    "backoff_ignores_floor": ("max(float(np.float32(self.scale * self.backoff)), self.min_scale)",
                              "float(np.float32(self.scale * self.backoff))", 1),
    "scaler_never_sees_overflow": ("scaler.update(bool(flag))", "scaler.update(False)", 1),
    # loss-scale growth (pinned against torch's dynamic loss-scale update)
    "growth_one_step_late": ("self.good_steps >= self.growth_interval", "self.good_steps > self.growth_interval", 1),
    "growth_one_step_early": ("self.good_steps >= self.growth_interval",
                              "self.good_steps >= self.growth_interval - 1", 1),
    "growth_by_inverse_backoff": ("np.float32(self.scale * self.growth)", "np.float32(self.scale / self.backoff)", 1),
    "growth_keeps_counter": ("                self.good_steps = 0\n", "                pass\n", 1),
    "growth_into_inf": ("if np.isfinite(grown):", "if True:", 1),
    "overflow_keeps_counter": ("            self.good_steps = 0\n        else:", "            pass\n        else:", 1),
    "skipped_step_still_updates": ("    if not flag:\n        adam_apply(contribs, state.p, state.m",
                                   "    if True:\n        adam_apply(contribs, state.p, state.m", 1),
    "skipped_step_advances_t": ("        state.t += 1\n    scaler.update(bool(flag))\n    return int(flag)\n\n\ndef reduce_to_owner",
                                "    state.t += 1\n    scaler.update(bool(flag))\n    return int(flag)\n\n\ndef reduce_to_owner", 1),
    "step_number_off_by_one": ("state.t + 1, hp)", "state.t + 2, hp)", 1),
    "reduce_to_owner_offset_in_fill": ("return lo - rank * lay.shard, float_to_half(reduce(windows))",
                                       "return lo - fill * lay.bucket, float_to_half(reduce(windows))", 1),
    "reduce_to_owner_reads_rank0_only": ("windows = [flat_window(lst, lo, hi) for lst in contrib_lists]",
                                         "windows = [flat_window(contrib_lists[0], lo, hi) for lst in contrib_lists]", 1),
    "owner_step_window_off_by_one_rank": ("contribs = [flat_window(lst, lo, lo + lay.shard) for lst in contrib_lists]",
                                          "contribs = [flat_window(lst, lo + lay.shard, lo + 2 * lay.shard) "
                                          "for lst in contrib_lists]", 1),
    "owner_step_window_off_by_one_element": ("contribs = [flat_window(lst, lo, lo + lay.shard) for lst in contrib_lists]",
                                             "contribs = [flat_window(lst, lo + 1, lo + 1 + lay.shard) "
                                             "for lst in contrib_lists]", 1),
}


def _exec_module(name, path, source):
    mod = types.ModuleType(name)
    mod.__file__ = path
    mod.__package__ = "oracle"
    sys.modules[name] = mod
    try:
        exec(compile(source, path, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


def _swap_in(monkeypatch, mutant, targets, exclude=()):
    """Point every name the mutant defines at its version, in each target
    namespace that already holds a name of the same origin."""
    swaps = []
    for key, val in vars(mutant).items():
        if key.startswith("__") or key in exclude:
            continue
        for tgt, origin in targets:
            if key in vars(tgt) and (origin is None or vars(tgt)[key] is vars(origin).get(key)):
                swaps.append((tgt, key, val))
    for tgt, key, val in swaps:         # decided before any swap changes an origin
        monkeypatch.setattr(tgt, key, val)


@pytest.mark.parametrize("name", sorted(LAYOUT_MUTANTS))
def test_layout_mutant_fails_a_pin(name, monkeypatch, real_oracle_lib):
    path = os.path.join(ORACLE_DIR, "layout.py")
    mut = _exec_module("oracle._layout_mutant", path, _mutate(path, LAYOUT_MUTANTS[name]))
    _swap_in(monkeypatch, mut, [(real_layout, None), (oracle, real_layout)])
    caught = _first_failing_pin()
    assert caught is not None, f"layout mutant {name!r} passes every pin"


@pytest.mark.parametrize("name", sorted(INIT_MUTANTS))
def test_python_oracle_mutant_fails_a_pin(name, monkeypatch, real_oracle_lib):
    path = os.path.join(ORACLE_DIR, "__init__.py")
    mut = _exec_module("oracle._init_mutant", path, _mutate(path, INIT_MUTANTS[name]))
    mut._lib = real_oracle_lib          # the mutant's C calls go to the real library
    _swap_in(monkeypatch, mut, [(oracle, None)], exclude={"build", "load", "lib", "_lib"})
    caught = _first_failing_pin()
    assert caught is not None, f"oracle mutant {name!r} passes every pin"


def test_unmutated_copies_pass_every_pin(tmp_path, monkeypatch, real_oracle_lib):
    """The harness itself: unmodified copies swapped in the same way pass."""
    src = tmp_path / "zero_oracle_copy.c"
    with open(os.path.join(ORACLE_DIR, "zero_oracle.c")) as f:
        src.write_text(f.read())
    so = tmp_path / "libzero_oracle_copy.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "_lib", oracle.load(str(so)))
    path = os.path.join(ORACLE_DIR, "layout.py")
    with open(path) as f:
        lay = _exec_module("oracle._layout_copy", path, f.read())
    _swap_in(monkeypatch, lay, [(real_layout, None), (oracle, real_layout)])
    path = os.path.join(ORACLE_DIR, "__init__.py")
    with open(path) as f:
        init = _exec_module("oracle._init_copy", path, f.read())
    init._lib = oracle._lib
    _swap_in(monkeypatch, init, [(oracle, None)], exclude={"build", "load", "lib", "_lib"})
    assert _first_failing_pin() is None
