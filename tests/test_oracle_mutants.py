"""The pins have teeth: plant one plausible mistake at a time in a copy of the
oracle's C source (on the CPU), rebuild it, and check that at least one pin
in test_oracle_pins.py fails against the planted mistake.

Each mutation is a textual replacement that must match the source exactly
once, so a refactor of the oracle that silently disables a mutation fails
here too.
"""
import ctypes
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = oracle._SRC.read_text()

MUTATIONS = {
    # the two maps added instead of subtracted
    "combine_sign": ("a1[c] = a1[c] - lam * a2[c];", "a1[c] = a1[c] + lam * a2[c];"),
    # lambda_init dropped from lambda
    "lambda_no_init": ("exp(dot(d, lq1, lk1)) - exp(dot(d, lq2, lk2)) +\n           da_oracle_lambda_init(layer)",
                       "exp(dot(d, lq1, lk1)) - exp(dot(d, lq2, lk2))"),
    # second exponential added
    "lambda_sign": ("exp(dot(d, lq1, lk1)) - exp(dot(d, lq2, lk2))", "exp(dot(d, lq1, lk1)) + exp(dot(d, lq2, lk2))"),
    # lambda_init constant garbled
    "lambda_init_rate": ("0.6 * exp(-0.3 * (double)layer)", "0.6 * exp(-0.03 * (double)layer)"),
    # softmax scale over the V width instead of the q/k width
    "scale_2d": ("1.0 / sqrt((double)d)", "1.0 / sqrt(2.0 * (double)d)"),
    # causal mask one past the diagonal (V1)
    "mask_off_by_one": ("softmax_attention_row(d, dv, i + 1, q1i", "softmax_attention_row(d, dv, (i + 2 < T ? i + 2 : T), q1i"),
    # eps outside the root
    "eps_outside": ("1.0 / sqrt(ms + 1e-5)", "1.0 / (sqrt(ms) + 1e-5)"),
    # RMS mean over d instead of 2d
    "rms_over_d": ("ms /= dv;", "ms /= d;"),
    # output scale (1 - lambda_init) dropped
    "no_out_scale": ("dst[c] = a1[c] * r * (1.0 - lam_init);", "dst[c] = a1[c] * r;"),
    # V rows read in reverse (a transposed / mis-indexed operand)
    "v_reversed": ("const double* vj = v + (int64_t)j * vstride;",
                   "const double* vj = v + (int64_t)(nkeys - 1 - j) * vstride;"),
    # V2: odd and even heads swapped
    "pair_swap": ("dst[c] = a_even[c] - s * a_odd[c];", "dst[c] = a_odd[c] - s * a_even[c];"),
    # V2: gate not passed through the sigmoid's sign convention
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-x));", "return 1.0 / (1.0 + exp(x));"),
    # V2: head -> kv-group mapping interleaved instead of contiguous
    "gqa_mod": ("const int ge = he / group, go = ho / group;", "const int ge = he % Hkv, go = ho % Hkv;"),
    # decode: the newest cache entry is not seen
    "decode_drops_last": ("v2_row(Hq, Hkv, d, L, qrow", "v2_row(Hq, Hkv, d, L - 1, qrow"),
    # off-by-one softmax: the extra exp(0) term dropped
    "softmax1_ignored": ("double z = softmax1 ? exp(0.0 - m) : 0.0;", "double z = 0.0;"),
    # off-by-one softmax: the extra term added without the max shift
    "softmax1_unshifted": ("double z = softmax1 ? exp(0.0 - m) : 0.0;", "double z = softmax1 ? 1.0 : 0.0;"),
}

PINS = [
    pins.test_lambda_init_special_values,
    pins.test_lambda_init_geometric_gap_decimal,
    pins.test_v1_lambda_special_cases,
    lambda: [pins.test_v1_lambda_zero_is_plain_attention(l) for l in (0, 3, 14)],
    pins.test_v1_identical_branches,
    pins.test_v2_sigmoid_zero_is_plain_gqa_attention,
    pins.test_v2_identical_heads_and_full_gate,
    pins.test_t1_closed_forms,
    pins.test_uniform_attention_prefix_mean,
    lambda: pins.test_needle_on_and_past_the_diagonal(0, True),
    lambda: pins.test_needle_on_and_past_the_diagonal(1, False),
    pins.test_v2_gqa_group_mapping,
    # one fixed brute-force draw per path (hypothesis is not re-run here)
    lambda: pins.test_v1_matches_bruteforce.hypothesis.inner_test(B=2, H=2, T=16, d=8, layer=5, seed=1),
    lambda: pins.test_v2_matches_bruteforce.hypothesis.inner_test(B=1, T=16, Hkv=2, G=4, d=8, seed=2),
    lambda: pins.test_decode_matches_bruteforce.hypothesis.inner_test(B=2, L=9, Hkv=2, G=4, d=4, seed=3),
    lambda: pins.test_softmax1_is_an_extra_zero_key(0),
    lambda: [pins.test_softmax1_equal_scores_closed_form(s) for s in (-2.0, 1.5)],
]


def _failing_pins():
    failed = 0
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            failed += 1
    return failed


@pytest.fixture(scope="module")
def restore_oracle():
    saved = oracle._load()
    yield
    oracle._lib = saved


def test_pins_pass_on_the_real_oracle(restore_oracle):
    assert _failing_pins() == 0


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name, tmp_path, restore_oracle):
    old, new = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation {name} no longer matches the oracle source"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    (tmp_path / "diffattn_oracle.h").write_text((oracle._HERE / "diffattn_oracle.h").read_text())
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", str(src), "-o", str(so), "-lm"],
                   check=True)
    saved = oracle._lib
    oracle._lib = oracle._configure(ctypes.CDLL(str(so)))
    try:
        failed = _failing_pins()
    finally:
        oracle._lib = saved
    assert failed >= 1, f"no pin catches mutation {name}"


# --------------------------------------------------------------------------
# The paged decode's gather is Python (oracle.v2_decode_paged): its mutants
# are textual replacements in that function's source, re-executed in the
# oracle module's namespace.
# --------------------------------------------------------------------------

import inspect  # noqa: E402

PAGED_SRC = inspect.getsource(oracle.v2_decode_paged)

PAGED_MUTATIONS = {
    # page and row swapped
    "paged_page_row_swap": ("k = kp[pg, t % page]", "k = kp[t % page, pg % page]"),
    # every sequence read through the first sequence's table row
    "paged_first_row_only": ("pg = table[b, t // page]", "pg = table[0, t // page]"),
    # the sequence's own length ignored (the table's full width used)
    "paged_full_width": ("L = int(lens[b])", "L = int(lens.max())"),
    # the newest entry of each sequence dropped
    "paged_drops_last": ("t = np.arange(L)", "t = np.arange(max(L - 1, 1))"),
    # V read from the K pool
    "paged_v_from_k": ("v = vp[pg, t % page]", "v = kp[pg, t % page]"),
}

PAGED_PINS = [
    lambda: pins.test_paged_decode_matches_bruteforce.hypothesis.inner_test(
        lens=[5, 33, 1], page=4, Hkv=2, G=2, d=4, seed=4),
    pins.test_paged_identity_table_is_the_dense_cache,
    pins.test_paged_pool_permutation_invariance,
    pins.test_paged_ragged_lengths_are_dense_prefixes,
]


def _failing_paged_pins():
    failed = 0
    for pin in PAGED_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, IndexError, ValueError):
            failed += 1
    return failed


def test_paged_pins_pass_on_the_real_oracle():
    assert _failing_paged_pins() == 0


@pytest.mark.parametrize("name", sorted(PAGED_MUTATIONS))
def test_paged_mutant_is_caught(name, monkeypatch):
    old, new = PAGED_MUTATIONS[name]
    assert PAGED_SRC.count(old) == 1, f"mutation {name} no longer matches the oracle source"
    ns = dict(vars(oracle))
    exec(compile(PAGED_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "v2_decode_paged", ns["v2_decode_paged"])
    assert _failing_paged_pins() >= 1, f"no pin catches mutation {name}"


MULTI_SRC = inspect.getsource(oracle.v2_decode_multi)

MULTI_MUTATIONS = {
    # every new token sees the whole cache (no causality among the new tokens)
    "multi_sees_all": ("n = L - nq + i + 1  # visible entries of new token i", "n = L"),
    # each new token also sees the next one
    "multi_one_ahead": ("n = L - nq + i + 1  # visible entries of new token i", "n = min(L, L - nq + i + 2)"),
    # queries matched to the wrong positions
    "multi_reversed": ("out[:, i] = v2_decode(q[:, i],", "out[:, i] = v2_decode(q[:, nq - 1 - i],"),
}

MULTI_PINS = [
    lambda: pins.test_multi_decode_is_the_last_prefill_rows_bruteforce.hypothesis.inner_test(
        B=1, L=17, nq=4, Hkv=1, G=2, d=4, seed=5),
    pins.test_multi_decode_matches_prefill_oracle_and_single_token,
]


@pytest.mark.parametrize("name", sorted(MULTI_MUTATIONS))
def test_multi_mutant_is_caught(name, monkeypatch):
    old, new = MULTI_MUTATIONS[name]
    assert MULTI_SRC.count(old) == 1, f"mutation {name} no longer matches the oracle source"
    ns = dict(vars(oracle))
    exec(compile(MULTI_SRC.replace(old, new), "<mutant>", "exec"), ns)
    monkeypatch.setattr(oracle, "v2_decode_multi", ns["v2_decode_multi"])
    failed = 0
    for pin in MULTI_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except (AssertionError, IndexError, ValueError):
            failed += 1
    assert failed >= 1, f"no pin catches mutation {name}"


def test_multi_pins_pass_on_the_real_oracle():
    for pin in MULTI_PINS:
        pin()
