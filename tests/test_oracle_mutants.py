"""Planted mistakes in the oracle: each must fail at least one pin.

Every mutant is a plausible error in the oracle, made on the CPU only. The C
mutants are textual edits of oracle/step.c, compiled into a temporary library
that stands in for the real one. The Python mutants are textual edits of
oracle/layout.py or oracle/step.py, executed as fresh modules whose functions
replace the real ones. The pins are the tests in test_oracle_*.py, run
unchanged against the mutant. A mutant that every pin accepts would be a
mistake the pins cannot see; this file fails then.
"""

import os
import sys
import tempfile
import types

import pytest

import oracle.build as OB
import oracle.layout as OL
import oracle.numerics as ON
import oracle.step as OS
import test_oracle_layout as TL
import test_oracle_numerics as TN
import test_oracle_sharding as TS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _numeric_pins():
    return [
        TN.test_narrow_matches_torch_structured,
        TN.test_narrow_special_values,
        TN.test_allreduce_worked_example,
        TN.test_single_contribution_is_identity,
        lambda: TN.test_reduce_equals_exact_sum(8, 0.125),
        lambda: TN.test_reduce_equals_exact_sum(3, 0.5),
        TN.test_reduce_small_integers_exact,
        TN.test_reduce_order_is_fixed_rank_order,
        TN.test_scale_applied_before_reduce,
        TN.test_bias_correction,
        TN.test_adam_step1_closed_form,
        TN.test_adam_special_cases,
        TN.test_adam_matches_torch_adamw,
        TN.test_step_is_reduce_then_adam,
        TN.test_norm_sq_exact_on_integers,
        TN.test_clip_coefficient_matches_torch,
        TN.test_clip_coefficient_special_cases,
        TN.test_clipped_step,
    ]


def _layout_pins():
    return [
        TL.test_page_demo_ranges,
        TL.test_tiny_golden_pieces,
        lambda: TL.test_workload_invariants("frag"),
        lambda: TL.test_workload_invariants("gpt2_small"),
        TL.test_brute_force_owner_scan,
        TL.test_padding_and_padding_only_rank,
        TS.test_tiny_ten_steps_union_equals_unsharded,
        lambda: TS.test_random_layouts_union_equals_unsharded(3),
        lambda: TS.test_random_layouts_union_equals_unsharded(7),
        TS.test_split_parameter_is_updated_as_one,
        TS.test_all_reduce_restricted_is_reduce_scatter,
        TS.test_writeback_touches_owned_range_only,
        lambda: TS.test_all_gather_closes_the_zero1_loop(0),
        lambda: TS.test_all_gather_closes_the_zero1_loop(1),
        lambda: TS.test_rank_norm_sq_exact_and_summing_to_the_global_norm(0),
        lambda: TS.test_rank_norm_sq_exact_and_summing_to_the_global_norm(1),
        lambda: TS.test_rank_state_is_the_zero1_share("frag"),
        lambda: TS.test_rank_state_is_the_zero1_share("gpt2_small"),
    ]


def _caught(pins) -> list:
    failed = []
    for i, pin in enumerate(pins):
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            failed.append(i)
    return failed


# ---- the C arithmetic ----------------------------------------------------------------------------

C_MUTANTS = {
    "scale applied after the reduction": [
        ("float acc = widen(narrow(widen(rep[0][i]) * scale));", "float acc = widen(rep[0][i]);"),
        ("float term = widen(narrow(widen(rep[j][i]) * scale));", "float term = widen(rep[j][i]);"),
        ("    return narrow(acc);\n}", "    return narrow(acc * scale);\n}"),
    ],
    "scaled terms not rounded to bf16": [
        ("float acc = widen(narrow(widen(rep[0][i]) * scale));", "float acc = widen(rep[0][i]) * scale;"),
        ("float term = widen(narrow(widen(rep[j][i]) * scale));", "float term = widen(rep[j][i]) * scale;"),
    ],
    "sum started from +0": [
        ("float acc = widen(narrow(widen(rep[0][i]) * scale));\n    for (int32_t j = 1;",
         "float acc = 0.0f;\n    for (int32_t j = 0;"),
    ],
    "ranks summed in reverse order": [
        ("float acc = widen(narrow(widen(rep[0][i]) * scale));\n    for (int32_t j = 1; j < n_rep; ++j) {\n"
         "        float term = widen(narrow(widen(rep[j][i]) * scale));",
         "float acc = widen(narrow(widen(rep[n_rep - 1][i]) * scale));\n    for (int32_t j = 1; j < n_rep; ++j) {\n"
         "        float term = widen(narrow(widen(rep[n_rep - 1 - j][i]) * scale));"),
    ],
    "reduced sum truncated instead of rounded": [
        ("    return narrow(acc);\n}",
         "    uint32_t bits;\n    memcpy(&bits, &acc, sizeof bits);\n    return (uint16_t)(bits >> 16);\n}")],
    "norm squares of rank 0's contribution only": [
        ("double g = (double)widen(reduce_one(n_rep, rep, i, scale));", "double g = (double)widen(rep[0][i]);")],
    "norm squares without the scaling": [
        ("double g = (double)widen(reduce_one(n_rep, rep, i, scale));",
         "double g = (double)widen(reduce_one(n_rep, rep, i, 1.0f));")],
    "clip coefficient from the squared norm": [("double norm = sqrt(total);", "double norm = total;")],
    "clip coefficient not capped at 1": [("return (float)(c < 1.0 ? c : 1.0);", "return (float)c;")],
    "found-inf not detected": [("    if (!isfinite(norm))\n        return NAN;\n", "")],
    "clipping coefficient ignored": [
        ("float g = widen(reduce_one(n_rep, rep, i, scale)) * grad_coeff;",
         "float g = widen(reduce_one(n_rep, rep, i, scale));")],
    "weight decay with the wrong sign": [("float u2 = u + wdp;", "float u2 = u - wdp;")],
    "weight decay not scaled by lr": [("float st = hp->lr * u2;", "float st = hp->lr * u + wdp;")],
    "weight decay dropped": [("float u2 = u + wdp;", "float u2 = u;")],
    "first moment not bias-corrected": [("float mh = mn / hp->bc1;", "float mh = mn;")],
    "second moment not bias-corrected": [("float vh = vn / hp->bc2;", "float vh = vn;")],
    "eps inside the square root": [("float den = sqrtf(vh) + hp->eps;", "float den = sqrtf(vh + hp->eps);")],
    "beta1 used for the second moment": [("float v1 = hp->beta2 * *v;", "float v1 = hp->beta1 * *v;")],
    "gradient not squared": [("float gg = g * g;", "float gg = g;")],
    "bias correction one step late": [("for (int64_t i = 0; i < t; ++i)", "for (int64_t i = 0; i <= t; ++i)")],
    "ties rounded away from zero": [("(dropped == 0x8000u && (toward & 1u))", "(dropped == 0x8000u)")],
    "bf16 by truncation": [("toward = (uint16_t)(toward + 1u);", "toward = toward;")],
    "NaN not kept as NaN": [("if ((u & 0x7fffffffu) > 0x7f800000u)", "if (0)")],
    "write-back of the old parameter": [
        ("        adam_one(&hp, g, &master[i], &m[i], &v[i]);\n        if (param_out)\n"
         "            param_out[i] = narrow(master[i]);",
         "        float old = master[i];\n        adam_one(&hp, g, &master[i], &m[i], &v[i]);\n        if (param_out)\n"
         "            param_out[i] = narrow(old);"),
    ],
}


@pytest.fixture(scope="module")
def c_mutant_dir():
    with tempfile.TemporaryDirectory(prefix="oracle_mutants_") as d:
        yield d


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_mutant_is_caught(name, c_mutant_dir, monkeypatch):
    src = open(OB.SRC).read()
    for old, new in C_MUTANTS[name]:
        assert old in src, f"mutant '{name}' no longer applies to oracle/step.c"
        src = src.replace(old, new)
    tag = str(abs(hash(name)))
    path = os.path.join(c_mutant_dir, f"step_{tag}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = OB.build(src=path, out=os.path.join(c_mutant_dir, f"lib_{tag}.so"), werror=False)
    monkeypatch.setattr(ON, "_lib", ON.load(lib))
    assert _caught(_numeric_pins()), f"no pin catches the planted mistake: {name}"


def test_c_harness_without_mutation_passes(c_mutant_dir, monkeypatch):
    lib = OB.build(src=OB.SRC, out=os.path.join(c_mutant_dir, "lib_none.so"), werror=False)
    monkeypatch.setattr(ON, "_lib", ON.load(lib))
    assert _caught(_numeric_pins()) == []


def test_unmutated_oracle_passes_every_pin():
    assert _caught(_numeric_pins()) == []
    assert _caught(_layout_pins()) == []


# ---- the layout and the rank composition ---------------------------------------------------------

PY_MUTANTS = {
    "rank range not shifted by the bucket offset": ("layout", [
        ("return Range(bucket.offset + rank * shard, bucket.offset + (rank + 1) * shard)",
         "return Range(rank * shard, (rank + 1) * shard)")]),
    "param range measured from the rank's range": ("layout", [
        ("param=world.shift(-pr.start),", "param=world.shift(-mine.start),")]),
    "shard views packed without the phase gap": ("layout", [
        ("base = end + (start - end) % SHARD_PHASE", "base = end")]),
    "bucket closes only above bucket_numel": ("layout", [
        ("if filled >= bucket_numel or i == len(sizes) - 1:", "if filled > bucket_numel or i == len(sizes) - 1:")]),
    "padding placed before the parameters": ("layout", [
        ("    return Layout(sizes, bucket_numel, dp_size, tuple(buckets), tuple(param_world))",
         "    head = {p: b.padded_numel - b.numel for b in buckets for p in b.params}\n"
         "    param_world = [r.shift(head[i]) for i, r in enumerate(param_world)]\n"
         "    return Layout(sizes, bucket_numel, dp_size, tuple(buckets), tuple(param_world))")]),
    "odd ranks skip the first element of their range": ("layout", [
        ("lo, hi = max(pr.start, mine.start), min(pr.end, mine.end)",
         "lo, hi = max(pr.start, mine.start + rank % 2), min(pr.end, mine.end)")]),
    "piece's shard slot from gbuf_local only": ("step", [
        ("k0 = pc.shard_offset\n        k1 = k0 + pc.gbuf_world.size\n        g0, g1 = _span(grad_coords",
         "k0 = pc.gbuf_local.start\n        k1 = k0 + pc.gbuf_world.size\n        g0, g1 = _span(grad_coords")]),
    "all-gather takes every range from the first rank's buffer": ("step", [
        ("            out[r.start:r.end] = params[j][r.start:r.end]",
         "            out[r.start:r.end] = params[0][r.start:r.end]")]),
    "all-gather leaves the padding out": ("step", [
        ("            r = L.rank_range(b, layout.dp_size, j)\n            out[r.start:r.end]",
         "            r = L.rank_range(b, layout.dp_size, j)\n            r = L.Range(r.start, min(r.end, b.offset + b.numel))\n"
         "            out[r.start:r.end]")]),
    "squared norm read at the bucket-local offset": ("step", [
        ("        g0, g1 = _span(grad_coords, pc.gbuf_world, pc.shard_offset)\n        total",
         "        g0, g1 = _span(grad_coords, pc.gbuf_world, pc.gbuf_local.start)\n        total")]),
    "squared norm over the whole rank range, padding included": ("step", [
        ("    for pc in L.rank_pieces(layout, rank):\n        g0, g1 = _span(grad_coords, pc.gbuf_world, pc.shard_offset)\n"
         "        total",
         "    for world, base in L.rank_ranges(layout, rank):\n        g0, g1 = _span(grad_coords, world, base)\n"
         "        total")]),
    "shard views a whole line further apart than the phase needs": ("layout", [
        ("base = end + (start - end) % SHARD_PHASE", "base = end + (start - end) % SHARD_PHASE + SHARD_PHASE")]),
    "owned elements counted over the whole ranges, padding included": ("layout", [
        ("    return sum(p.gbuf_world.size for p in rank_pieces(layout, rank))",
         "    return sum(r.size for r, _ in rank_ranges(layout, rank))")]),
    "reduce-scatter over the parameter pieces only": ("step", [
        ("    for b, (world, base) in enumerate(L.rank_ranges(layout, rank)):",
         "    for b, (world, base) in enumerate([(pc.gbuf_world, pc.shard_offset)\n"
         "                                        for pc in L.rank_pieces(layout, rank)]):")]),
}


def _install_python_mutant(which, edits, monkeypatch, label):
    """Execute the edited source as a fresh module and put its functions in
    place of the real module's; classes stay the real ones."""
    real = {"layout": OL, "step": OS}[which]
    src = open(real.__file__).read()
    for old, new in edits:
        assert old in src, f"mutant '{label}' no longer applies to {real.__file__}"
        src = src.replace(old, new)
    mod = types.ModuleType(f"oracle.mutant_{which}")
    mod.__dict__["__package__"] = "oracle"
    monkeypatch.setitem(sys.modules, mod.__name__, mod)
    exec(compile(src, f"<mutant {label}>", "exec"), mod.__dict__)
    for attr, val in list(mod.__dict__.items()):
        if isinstance(val, type) and getattr(real, attr, None) is not None:
            mod.__dict__[attr] = getattr(real, attr)
    for attr, val in mod.__dict__.items():
        if isinstance(val, types.FunctionType) and hasattr(real, attr):
            monkeypatch.setattr(real, attr, val)


@pytest.mark.parametrize("which", ["layout", "step"])
def test_python_harness_without_mutation_passes(which, monkeypatch):
    _install_python_mutant(which, [], monkeypatch, "none")
    assert _caught(_layout_pins()) == []


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(name, monkeypatch):
    which, edits = PY_MUTANTS[name]
    _install_python_mutant(which, edits, monkeypatch, name)
    assert _caught(_layout_pins()), f"no pin catches the planted mistake: {name}"
