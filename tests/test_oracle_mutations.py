"""The pins have teeth: copies of ep_oracle.c with one plausible mistake
each -- a wrong tie rule, a dropped term, a wrong index, order or starting
value -- are built, and the pins that cover that step must fail on every one.

Each mutant runs the named pin tests in a child pytest process with
EP_ORACLE_LIB pointing at the mutant's library; exit status 1 means that
tests ran and failed.  The unmutated source, built the same way, passes
them all (the control).
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "ep_oracle.c")
F = "tests/test_oracle_formats.py::"
R = "tests/test_oracle_route.py::"
L = "tests/test_oracle_layout.py::"

# (name, text in ep_oracle.c, replacement (every occurrence), pins that must fail)
MUTANTS = [
    ("bf16 ties round away from zero",
     "return (uint16_t)(((lo >> 16) & 1u) ? (hi >> 16) : (lo >> 16));",
     "return (uint16_t)(hi >> 16);",
     [F + "test_bf16_ties_to_even"]),
    ("bf16 saturates instead of overflowing",
     "hi_mag = ldexp(1.0, 128);", "hi_mag = INFINITY;",
     [F + "test_bf16_rounding_at_overflow_matches_torch"]),
    ("E4M3 ties go to the lower code",
     "else code = (lo & 1) ? hi : lo;", "else code = lo;",
     [F + "test_e4m3_encode_boundaries_match_torch"]),
    ("E4M3 saturates at 240 (the FNUZ maximum)",
     "if (a >= 448.0) return sign | 0x7E;", "if (a >= 240.0) return sign | 0x77;",
     [F + "test_e4m3_encode_strided_sweep_matches_torch"]),
    ("quotient through the reciprocal scale",
     "float v = orc_bf16_to_f32(x[b * 128 + j]) / scale;",
     "float v = orc_bf16_to_f32(x[b * 128 + j]) * (448.0f / amax);",
     [F + "test_quantize_matches_torch_blockwise"]),
    ("node score drops its second term",
     "for (int j = 0; j < J; ++j) {", "for (int j = 0; j < (J > 1 ? J - 1 : 1); ++j) {",
     [R + "test_c_oracle_matches_page_study"]),
    ("node score takes floor(K/M) terms",
     "const int J = limited ? (K + M - 1) / M : 0;", "const int J = limited ? (K / M > 0 ? K / M : 1) : 0;",
     [R + "test_brute_force_tiny"]),
    ("one node fewer is kept",
     "for (int m = 0; m < M; ++m) {", "for (int m = 0; m < M - 1; ++m) {",
     [R + "test_brute_force_tiny"]),
    ("repeated entries get a slot",
     "if (row[j] == e) { *err |= ORC_ERR_DUP_INDEX; return 0; }",
     "if (row[j] == e) { *err |= ORC_ERR_DUP_INDEX; return 1; }",
     [L + "test_ll_brute_force_tiny"]),
    ("expert ties go to the higher index",
     "if (allowed[e] && !taken[e] && (best < 0 || s[e] > s[best])) best = e;",
     "if (allowed[e] && !taken[e] && (best < 0 || s[e] >= s[best])) best = e;",
     [R + "test_forced_ties_follow_lower_index"]),
    ("LL slots counted across sources",
     "const int slot = counts[e * S + s]++;", "const int slot = counts[e * S]++;",
     [L + "test_ll_brute_force_tiny"]),
    ("same-position rank from s / G",
     "n * G + s % G", "n * G + s / G",
     [L + "test_ht_brute_force_tiny"]),
    ("combine rounds the product before the add",
     "acc = fmaf(w[i * K + k], orc_bf16_to_f32(Y[(int64_t)r * ld_y + h]), acc);",
     "acc = acc + w[i * K + k] * orc_bf16_to_f32(Y[(int64_t)r * ld_y + h]);",
     [F + "test_combine_is_a_fused_multiply_add_chain"]),
    ("combine in reverse k order",
     "            for (int k = 0; k < K; ++k) {\n                const int32_t r = loc[i * K + k];\n"
     "                if (r < 0) continue;\n                acc = fmaf(",
     "            for (int k = K - 1; k >= 0; --k) {\n                const int32_t r = loc[i * K + k];\n"
     "                if (r < 0) continue;\n                acc = fmaf(",
     [F + "test_combine_accumulates_in_k_order"]),
    ("combine starts from -0",
     "            float acc = 0.0f;\n            for (int k = 0; k < K; ++k) {\n"
     "                const int32_t r = loc[i * K + k];\n                if (r < 0) continue;\n"
     "                acc = fmaf(",
     "            float acc = -0.0f;\n            for (int k = 0; k < K; ++k) {\n"
     "                const int32_t r = loc[i * K + k];\n                if (r < 0) continue;\n"
     "                acc = fmaf(",
     [F + "test_combine_starts_from_plus_zero"]),
    ("node ties go to the higher index",
     "node_score[n] > node_score[best]", "node_score[n] >= node_score[best]",
     [R + "test_forced_ties_follow_lower_index"]),
    ("amax misses a block's last element",
     "for (int j = 0; j < 128; ++j) {\n            float a = fabsf",
     "for (int j = 0; j < 127; ++j) {\n            float a = fabsf",
     [F + "test_quantize_matches_torch_blockwise"]),
    ("the inverse scale is stored",
     "scales[b] = scale;", "scales[b] = 1.0f / scale;",
     [F + "test_quantize_matches_torch_blockwise"]),
    ("LL header fields swapped",
     "int32_t hdr[4] = {(int32_t)(i % T), (int32_t)(i / T), k, 0};",
     "int32_t hdr[4] = {(int32_t)(i / T), (int32_t)(i % T), k, 0};",
     [L + "test_pack_roundtrip_headers"]),
    ("stage-1 metadata names the global token index",
     "meta1_tok[r] = t;", "meta1_tok[r] = (int32_t)i;",
     [L + "test_ht_pack_rows_and_metadata_roundtrip"]),
    ("stage-1 weights not forwarded",
     "if (w) meta1_w[(int64_t)r * K + k] = w[i * K + k];", "if (w) meta1_w[(int64_t)r * K + k] = 0.0f;",
     [L + "test_ht_pack_rows_and_metadata_roundtrip"]),
    ("stage-2 metadata source and token swapped",
     "meta2_src[r] = s;\n            meta2_tok[r] = t;", "meta2_src[r] = t;\n            meta2_tok[r] = s;",
     [L + "test_ht_pack_rows_and_metadata_roundtrip"]),
    ("stage-2 k off by one",
     "meta2_k[r] = k;", "meta2_k[r] = k + 1;",
     [L + "test_ht_pack_rows_and_metadata_roundtrip"]),
    ("row gradient drops the weight",
     "const float prod = w[t * K + k] * gv;", "const float prod = gv;",
     ["tests/test_oracle_backward.py::test_row_gradient_rounding_matches_torch"]),
    ("weight gradient drops a term",
     "for (int h = 0; h < H; ++h) {\n                    const float gv",
     "for (int h = 0; h < H - 1; ++h) {\n                    const float gv",
     ["tests/test_oracle_backward.py::test_weight_gradient_is_the_derivative"]),
    ("E4M3 drops the sign of zero",
     "uint8_t sign = signbit(v) ? 0x80 : 0x00;", "uint8_t sign = (v < 0) ? 0x80 : 0x00;",
     [F + "test_e4m3_signed_zero_and_saturation"]),
    ("an all-zero block gets codes 0x80",
     "            memset(q + b * 128, 0, 128);", "            memset(q + b * 128, 0x80, 128);",
     [F + "test_quantize_matches_torch_blockwise"]),
    ("a row's scales in reverse block order",
     "memcpy(dst + H, sc, sizeof(float) * (size_t)(H / 128));",
     "for (int b_ = 0; b_ < H / 128; ++b_) memcpy(dst + H + 4 * b_, &sc[H / 128 - 1 - b_], 4);",
     [F + "test_row_image_layout"]),
    ("combine reads row 0 for an invalid entry",
     "                if (r < 0) continue;\n                acc = fmaf(",
     "                const int32_t rr = r < 0 ? 0 : r;\n"
     "                acc = fmaf(w[i * K + k], orc_bf16_to_f32(Y[(int64_t)rr * ld_y + h]), acc); continue;\n"
     "                acc = fmaf(",
     [F + "test_combine_skips_invalid_and_k1_copy"]),
    ("a per-rank row belongs to the token's last entry on the rank",
     "            if (hit[r]) continue;\n            hit[r] = 1;",
     "            if (hit[r]) { for (int q_ = 0; q_ < k; ++q_) if (row2[i*K+q_] >= 0 && row[q_] / L == r)"
     " { row2[i*K+k] = row2[i*K+q_]; row2[i*K+q_] = -1; } continue; }\n            hit[r] = 1;",
     ["tests/test_oracle_rank_dedup.py::test_brute_force_rows"]),
    ("identity expert reads the wrong block's scale",
     "memcpy(&sc, src + H + 4 * (h / 128), 4);", "memcpy(&sc, src + H + 4 * ((h / 128) ^ 1), 4);",
     [F + "test_dequant_matches_torch"]),
]


def _build(d, name, text):
    c = os.path.join(d, f"{name}.c")
    with open(c, "w") as f:
        f.write(text)
    so = os.path.join(d, f"{name}.so")
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-shared", "-fPIC", c, "-o", so, "-lm"],
                   check=True, capture_output=True)
    return so


def _run_pins(lib, pins):
    env = dict(os.environ, EP_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", *pins],
                          cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Every mutant (and the control) built and run, a few at a time."""
    d = str(tmp_path_factory.mktemp("mutants"))
    src = open(SRC).read()
    jobs = {"control": (src, sorted({p for m in MUTANTS for p in m[3]}))}
    for name, old, new, pins in MUTANTS:
        jobs[name] = (src.replace(old, new) if old in src else None, pins)

    def run(item):
        idx, (key, (text, pins)) = item
        if text is None:
            return key, None
        return key, _run_pins(_build(d, f"m{idx}", text), pins)

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(6, os.cpu_count() or 1)) as ex:
        return dict(ex.map(run, enumerate(jobs.items())))


def test_control_passes(outcomes):
    r = outcomes["control"]
    assert r.returncode == 0, r.stdout[-3000:]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(outcomes, name, old, new, pins):
    r = outcomes[name]
    assert r is not None, "the mutated text must exist in the oracle"
    assert r.returncode == 1, f"pins {pins} did not catch: {name}\n{r.stdout[-2000:]}"
