"""The oracle's pins must catch plausible mistakes.  Each case compiles a copy
of oracle/ring_oracle.c with one mistake planted (a wrong index, a wrong
neighbour, a dropped term, a wrong sign, a wrong rounding, a missing round),
loads it in place of the real one, and runs the pin suite's checks: at least
one must fail.  The unmodified source must pass them all."""
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle_bidir_pins as bidir
import test_oracle_pins as pins
import test_oracle_psum_circ_pins as psum

SRC = os.path.join(os.path.dirname(oracle.__file__), "ring_oracle.c")

MUTANTS = {
    "rs chunk off by one": ("return (r - s - 2 + 2 * P) % P;", "return (r - s - 1 + 2 * P) % P;"),
    "right neighbour instead of left": ("return (r - 1 + P) % P;", "return (r + 1) % P;"),
    "all-gather chunk off by one": ("return (r - t - 1 + P) % P;", "return (r - t + P) % P;"),
    "fp32 add drops own term": ("tmp[(size_t)r * C + i] = own[i] + recv[i];",
                                "tmp[(size_t)r * C + i] = recv[i];"),
    "fp32 reads neighbour input instead of partial":
        ("const float *recv = state + (size_t)left_of(r, P) * n + (size_t)c * C;",
         "const float *recv = src + (size_t)left_of(r, P) * n + (size_t)c * C;"),
    "int32 wrong sign": ("(uint32_t)own[i] + (uint32_t)recv[i]", "(uint32_t)own[i] - (uint32_t)recv[i]"),
    "bf16 rounds half up": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    "bf16 carry rounded every hop": ("tmp[(size_t)r * C + i] = bf16_to_f32(own[i]) + recv[i];",
                                     "tmp[(size_t)r * C + i] = bf16_to_f32(oracle_bf16_from_f32(bf16_to_f32(own[i]) + recv[i]));"),
    "ppermute does not shift": ("s + (size_t)left_of(r, P) * bytes_per_rank, bytes_per_rank);",
                                "s + (size_t)r * bytes_per_rank, bytes_per_rank);"),
    "all-reduce misses a gather round": ("return oracle_all_gather(state, P, n, sizeof(float), P - 1);",
                                         "return oracle_all_gather(state, P, n, sizeof(float), P - 2);"),
    "all-gather places pieces at the wrong chunk":
        ("memcpy((uint8_t *)state + (size_t)r * nb + (size_t)r * Cb,",
         "memcpy((uint8_t *)state + (size_t)r * nb + (size_t)((r + 1) % P) * Cb,"),
    "bidir top half pulled from the left":
        ("const float *from_right = top + (size_t)mod_p(d + 1, P) * h;",
         "const float *from_right = top + (size_t)mod_p(d - 1, P) * h;"),
    "bidir block index off by one":
        ("const float *xt = src + (size_t)d * n + (size_t)mod_p(d + s + 1, P) * C;",
         "const float *xt = src + (size_t)d * n + (size_t)mod_p(d + s, P) * C;"),
    "bidir last step adds again":
        ("ntop[(size_t)d * h + i] = last ? from_right[i] : from_right[i] + xt[i];",
         "ntop[(size_t)d * h + i] = from_right[i] + xt[i];"),
    "bidir halves split at the wrong place": ("static size_t bidir_top_len(size_t C) { return C - C / 2; }",
                                              "static size_t bidir_top_len(size_t C) { return C / 2 + 1; }"),
    "bidir bf16 rounds every step":
        ("ntop[(size_t)d * h + i] = last ? from_right[i] : from_right[i] + bf16_to_f32(xt[i]);",
         "ntop[(size_t)d * h + i] = last ? from_right[i] : bf16_to_f32(oracle_bf16_from_f32(from_right[i] + bf16_to_f32(xt[i])));"),
    "psum forwards to the left":
        ("memcpy(slots + ((size_t)((d + 1) % P) * 2 + (1 - w)) * n, item + (size_t)d * n,\n                   sizeof(float) * n);",
         "memcpy(slots + ((size_t)((d + P - 1) % P) * 2 + (1 - w)) * n, item + (size_t)d * n,\n                   sizeof(float) * n);"),
    "psum adds the receiving slot": ("const float *in = slots + ((size_t)d * 2 + w) * n;",
                                     "const float *in = slots + ((size_t)d * 2 + (1 - w)) * n;"),
    "psum first send into slot 1":
        ("memcpy(slots + ((size_t)((d + 1) % P) * 2 + 0) * n, src + (size_t)d * n, sizeof(float) * n);",
         "memcpy(slots + ((size_t)((d + 1) % P) * 2 + 1) * n, src + (size_t)d * n, sizeof(float) * n);"),
    "psum bf16 items in the wrong order": ("const uint16_t *in = src + (size_t)(((d - s - 1) % P + P) % P) * n;",
                                           "const uint16_t *in = src + (size_t)(((d + s + 1) % P + P) % P) * n;"),
    "magnitude sum without abs": ("            m += fabs(x);\n        }\n        sum[i] = a;\n        if (abssum) abssum[i] = m;\n    }\n    return 0;\n}\n\nint oracle_rank_sum_f64_bf16",
                                  "            m += x;\n        }\n        sum[i] = a;\n        if (abssum) abssum[i] = m;\n    }\n    return 0;\n}\n\nint oracle_rank_sum_f64_bf16"),
}


def _checks():
    yield "ppermute table", pins.test_ppermute_matches_page_table
    yield "all-gather table", pins.test_all_gather_matches_page_slot_table
    for P in (2, 3, 4, 8):
        yield "psum_scatter P=%d" % P, lambda P=P: pins.test_reduce_scatter_is_psum_scatter_int32(P)
        yield "contributors P=%d" % P, lambda P=P: pins.test_reduce_scatter_contributor_sets(P)
        yield "int32 all-reduce P=%d" % P, lambda P=P: pins.test_all_reduce_int32_brute_force(P)
    yield "owner last", pins.test_fp32_association_order_owner_last
    yield "chain direction", pins.test_fp32_association_order_chain_direction
    yield "p2", pins.test_p2_single_round
    for P in (2, 4):
        yield "fp32 bound P=%d" % P, lambda P=P: pins.test_all_reduce_fp32_within_recursive_sum_bound(P)
        yield "int fp32 exact P=%d" % P, lambda P=P: pins.test_all_reduce_int_valued_fp32_exact(P)
    for bits, want in [(0x3F808000, 0x3F80), (0x3F818000, 0x3F82), (0x00008000, 0x0000)]:
        yield "bf16 %#x" % bits, lambda b=bits, w=want: pins.test_bf16_rne_hand_cases(b, w)
    yield "bf16 vs torch", pins.test_bf16_rne_matches_torch
    yield "bf16 nan", pins.test_bf16_rne_nan_stays_nan
    yield "all-gather concat", lambda: pins.test_all_gather_is_concatenation(4)
    yield "rank sum", lambda: pins.test_rank_sum_f64_matches_numpy(3)
    yield "bf16 carry", pins.test_bf16_carry_is_fp32_until_owner
    yield "bf16 bound", lambda: pins.test_bf16_all_reduce_one_rounding_bound(4)
    yield "bidir page trace", bidir.test_bidir_matches_page_trace_in_fp32_order
    for P in (2, 3, 4):
        yield "bidir psum_scatter P=%d" % P, lambda P=P: bidir.test_bidir_is_psum_scatter_int32(P)
        yield "bidir contributors P=%d" % P, lambda P=P: bidir.test_bidir_contributor_sets(P)
    yield "bidir odd chunks", lambda: bidir.test_bidir_odd_chunks(3, 5)
    yield "bidir p1 p2", bidir.test_bidir_p1_identity_and_p2
    yield "bidir bf16", lambda: bidir.test_bidir_bf16_one_rounding(4)
    yield "psum page trace", psum.test_psum_matches_page_trace
    for P in (2, 3, 4):
        yield "psum sum P=%d" % P, lambda P=P: psum.test_psum_is_sum_over_devices_int32(P)
        yield "psum visits P=%d" % P, lambda P=P: psum.test_psum_every_item_visits_every_device(P)
    yield "psum bf16", lambda: psum.test_psum_fp32_bound_and_bf16_one_rounding(4)
    yield "psum bf16 order", psum.test_psum_bf16_follows_page_order


def _load_variant(tmp_path, text, name):
    c = tmp_path / ("%s.c" % name)
    so = tmp_path / ("%s.so" % name)
    c.write_text(text)
    subprocess.check_call(["gcc", *oracle._CFLAGS, str(c), "-o", str(so), "-lm"])
    lib = ctypes.CDLL(str(so))
    return lib


def _run_checks_with(lib, monkeypatch):
    real = oracle._load()
    for fname in ("oracle_ppermute", "oracle_reduce_scatter_f32", "oracle_reduce_scatter_i32",
                  "oracle_all_gather", "oracle_all_gather_place", "oracle_all_reduce_f32",
                  "oracle_all_reduce_i32", "oracle_reduce_scatter_bf16", "oracle_all_reduce_bf16",
                  "oracle_bf16_from_f32_array", "oracle_rank_sum_f64_f32", "oracle_rank_sum_f64_bf16",
                  "oracle_reduce_scatter_bidir_f32", "oracle_reduce_scatter_bidir_i32",
                  "oracle_reduce_scatter_bidir_bf16", "oracle_psum_circ_f32", "oracle_psum_circ_i32",
                  "oracle_psum_circ_bf16"):
        f, g = getattr(lib, fname), getattr(real, fname)
        f.argtypes, f.restype = g.argtypes, g.restype
    monkeypatch.setattr(oracle, "_lib", lib)
    failed = []
    for label, check in _checks():
        try:
            check()
        except (AssertionError, ValueError):
            failed.append(label)
    return failed


def test_unmodified_source_passes(tmp_path, monkeypatch):
    lib = _load_variant(tmp_path, open(SRC).read(), "clean")
    assert _run_checks_with(lib, monkeypatch) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert old in text, "mutation site not found: %s" % name
    lib = _load_variant(tmp_path, text.replace(old, new, 1), "mutant")
    failed = _run_checks_with(lib, monkeypatch)
    assert failed, "no pin caught the planted mistake '%s'" % name


# ---------------------------------------------------------------- the MLP layer
# The MLP part of the oracle is Python; a mutant is a copy of the package
# source with one mistake planted, executed as a module of its own and put in
# place of `oracle` for the MLP pins.
import importlib.util
import types

import test_oracle_mlp_pins as mlp

PY_SRC = os.path.join(os.path.dirname(oracle.__file__), "__init__.py")

PY_MUTANTS = {
    "gelu cubic coefficient": ("t = 2.0 * _GELU_C * (x + 0.044715 * x * x * x)\n    with",
                               "t = 2.0 * _GELU_C * (x + 0.04471 * x * x * x)\n    with"),
    "gelu argument not doubled": ("t = 2.0 * _GELU_C * (x + 0.044715 * x * x * x)\n    with",
                                  "t = _GELU_C * (x + 0.044715 * x * x * x)\n    with"),
    "gelu cancels in the tail": ("return x / (1.0 + np.exp(-t))",
                                 "return 0.5 * x * (1.0 + np.tanh(t / 2.0))"),
    "product not rounded before gelu": ("h[q] = bf16_from_f64(gelu_tanh(_f64(local0)))",
                                        "h[q] = bf16_from_f64(gelu_tanh(_f64(full[q]) @ _f64(W1[q])))"),
    "wrong column block of W1": ("local0 = bf16_from_f64(_f64(full[q]) @ _f64(W1[q]))",
                                 "local0 = bf16_from_f64(_f64(full[q]) @ _f64(W1[(q + 1) % P]))"),
    "rank keeps the wrong row block": ("[r * Mq:(r + 1) * Mq]) for r in range(P)])",
                                       "[((r + 1) % P) * Mq:((r + 1) % P + 1) * Mq]) for r in range(P)])"),
    "bf16 rounding truncates": ("r = _bf16_grid(v, np.rint).astype(np.float32)",
                                "r = _bf16_grid(v, np.trunc).astype(np.float32)"),
    "bf16 subnormal spacing": ("e = np.maximum(e, -125)", "e = np.maximum(e, -126)"),
}


def _mlp_checks():
    yield "gelu torch", mlp.test_gelu_matches_torch_tanh_form
    for x in (-12.0, -10.0, -6.0, -0.75, 1.0, 3.0):
        yield "gelu decimal %g" % x, lambda x=x: mlp.test_gelu_against_decimal_literal_formula(x)
    yield "gelu identities", mlp.test_gelu_identities
    yield "bf16 vs torch", mlp.test_bf16_from_f64_matches_torch_on_fp32_values
    yield "bf16 one rounding", mlp.test_bf16_from_f64_is_one_rounding
    yield "bf16 nearest", mlp.test_nearest_is_monotone_and_within_half_a_step
    for P in (1, 2, 3, 4):
        yield "unsharded P=%d" % P, lambda P=P: mlp.test_layer_equals_unsharded_computation(P)
    yield "brute force", mlp.test_layer_brute_force_tiny


def _py_variant(text):
    spec = importlib.util.spec_from_loader("oracle_mutant", loader=None)
    mod = types.ModuleType(spec.name)
    mod.__file__ = PY_SRC   # the C library is found next to it, as for the real package
    exec(compile(text, "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _run_mlp_checks_with(mod, monkeypatch):
    monkeypatch.setattr(mlp, "oracle", mod)
    failed = []
    for label, check in _mlp_checks():
        try:
            check()
        except (AssertionError, ValueError):
            failed.append(label)
    return failed


def test_unmodified_python_source_passes(monkeypatch):
    assert _run_mlp_checks_with(_py_variant(open(PY_SRC).read()), monkeypatch) == []


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(name, monkeypatch):
    old, new = PY_MUTANTS[name]
    text = open(PY_SRC).read()
    assert old in text, "mutation site not found: %s" % name
    failed = _run_mlp_checks_with(_py_variant(text.replace(old, new, 1)), monkeypatch)
    assert failed, "no pin caught the planted mistake '%s'" % name
