"""Mutation check of the oracle's pins.

Each case plants one plausible mistake in a copy of oracle/oracle.c.  Examples
are a dropped term, a wrong sign or index, swapped operands, an off-by-one
bound, or the wrong Philox word.  The case compiles the copy, loads it in a
fresh pytest process through SV_ORACLE_LIB, and runs the pins named for it.
At least one of them must fail.  An unmutated copy built the same way must
pass every named pin, so a broken harness cannot pass the check.

CPU only: gcc plus subprocesses, eight at a time.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

P = "tests/test_oracle_pins.py::"
X = "tests/test_oracle_pins_ext.py::"
M = "tests/test_oracle_margins.py::"
D = "tests/test_oracle_pins_draft.py::"
L = "tests/test_oracle_pins_lmhead.py::"

# (name, text to replace, replacement, occurrence (0-based), pins that must catch it)
MUTATIONS = [
    ("philox: wrong product in the first word", "uint32_t y0 = hi_b ^ x1 ^ k0;", "uint32_t y0 = hi_a ^ x1 ^ k0;", 0,
     [P + "test_philox_known_answer_vectors"]),
    ("philox: one Weyl constant for both key words", "k1 += PHILOX_WEYL_B;", "k1 += PHILOX_WEYL_A;", 0,
     [P + "test_philox_known_answer_vectors"]),
    ("counter layout: row and tag swapped", "uint32_t ctr[4] = {idx >> 2, g, tag, offset};",
     "uint32_t ctr[4] = {idx >> 2, tag, g, offset};", 0, [P + "test_counter_layout_selects_word"]),
    ("accept uniform may be 0", "ldexp((double)((w >> 8) + 1u), -24)", "ldexp((double)(w >> 8), -24)", 0,
     [P + "test_uniform_grid_endpoints"]),
    ("race noise from 1 - U", "return -log(u);", "return -log1p(-u);", 0,
     [M + "test_exp_noise_is_minus_log_of_the_race_uniform"]),
    ("bf16 widened by 15 bits", "uint32_t u = (uint32_t)bits << 16;", "uint32_t u = (uint32_t)bits << 15;", 0,
     [P + "test_bf16_conversion_bit_patterns"]),
    ("softmax multiplies by the temperature", "p[x] = exp((double)z[x] / T - m);",
     "p[x] = exp((double)z[x] * T - m);", 0, [P + "test_softmax_matches_library_and_closed_forms"]),
    ("repetition penalty: divide and multiply swapped", "        z[x] = z[x] / theta;", "        z[x] = z[x] * theta;", 0,
     [P + "test_repetition_penalty_reading"]),
    ("frequency penalty ignores the count", "float t = freq * (float)counts[x];", "float t = freq;", 0,
     [X + "test_frequency_penalty_page_example"]),
    ("top-k drops the ties at the k-th value", "if (z[x] < tau) z[x] = -INFINITY;", "if (z[x] <= tau) z[x] = -INFINITY;",
     0, [P + "test_top_k_threshold_and_ties"]),
    ("argmax keeps the last maximum", "if (z[x] > z[best]) best = x;", "if (z[x] >= z[best]) best = x;", 0,
     [P + "test_argmax_lowest_index_wins_ties"]),
    ("accept test strict at the boundary", "if (!(p >= uq)) {", "if (!(p > uq)) {", 0,
     [M + "test_accept_margin_exact_tie_is_zero_and_accepted"]),
    ("accept margin over the smaller side", "(p > uq ? p : uq)", "(p < uq ? p : uq)", 0,
     [M + "test_accept_margins_by_construction_no_draft"]),
    ("accept uniform of position 0 for every position",
     "double u = orc_uniform_accept(orc_word(seed, offset, g0 + (uint32_t)i, ORC_TAG_ACCEPT, 0));\n    if (syn_rates) {",
     "double u = orc_uniform_accept(orc_word(seed, offset, g0, ORC_TAG_ACCEPT, 0));\n    if (syn_rates) {", 0,
     [M + "test_accept_margin_uses_each_positions_own_uniform"]),
    ("race margin inverted", "return 1.0 - b2 / b1;", "return 1.0 - b1 / b2;", 0,
     [M + "test_flat_race_margin_and_winner"]),
    ("race levels combined with max", "if (margin) *margin = m1 < m2 ? m1 : m2;",
     "if (margin) *margin = m1 > m2 ? m1 : m2;", 0, [M + "test_two_level_race_margin"]),
    ("token-level margin against the chunk level's second score", "double m2 = level_margin(t1, t2, tcand > 1);",
     "double m2 = level_margin(t1, b2, tcand > 1);", 0, [M + "test_two_level_race_margin"]),
    ("second-best score not demoted on a new best", "if (*i1 >= 0) *b2 = *b1;", "if (*i1 < 0) *b2 = *b1;", 0,
     [M + "test_flat_race_margin_and_winner"]),
    ("race chunks one token short", "int32_t lo = c * C, hi = lo + C < V ? lo + C : V;",
     "int32_t lo = c * C, hi = lo + C - 1 < V ? lo + C - 1 : V;", 0,
     [P + "test_race_chunk_boundaries", P + "test_race_levels_are_exact_for_one_chunk"]),
    ("sampled row one before the reject", "const double *pj = P + (int64_t)j * V;",
     "const double *pj = P + (int64_t)(j > 0 ? j - 1 : j) * V;", 0,
     [P + "test_rows_of_a_request_are_used_in_place"]),
    ("residual q - p instead of p - q", "double r = pj[x] - draft_q(draft_probs, dstride, Q, V, j, x);",
     "double r = draft_q(draft_probs, dstride, Q, V, j, x) - pj[x];", 0,
     [P + "test_three_token_example_accept_mass_and_residual"]),
    ("no-draft mode keeps the rejected draft", "if (d >= 0 && d < V) w[d] = 0.0;",
     "if (d >= 0 && d < V) w[d] = w[d];", 0, [P + "test_four_token_no_draft_probs_example"]),
    ("greedy bonus from the last draft row", "    tokens[K] = amax[K];\n    *num_sampled = K + 1;",
     "    tokens[K] = amax[K > 0 ? K - 1 : 0];\n    *num_sampled = K + 1;", 0, [P + "test_greedy_rule"]),
    ("synthetic rate taken as conditional", "return u * prev <= (double)a[i];", "return u <= (double)a[i];", 0,
     [X + "test_synthetic_acceptance_law"]),
    ("top-p keeps the boundary value", "above < top_p + shift", "above <= top_p + shift", 0,
     [X + "test_top_p_keeps_ties_at_the_boundary"]),
    ("draft sampler on the verifier's tags", "ORC_TAG_DRAFT_CHUNK, ORC_TAG_DRAFT_TOKEN, &mg",
     "ORC_TAG_CHUNK, ORC_TAG_TOKEN, &mg", 0, [D + "test_draft_noise_is_not_the_verifiers"]),
    ("LM-head product with a shuffled weight row", "acc += hd[k] * (double)orc_bf16_to_f32(w[k]);",
     "acc += hd[k] * (double)orc_bf16_to_f32(w[k ^ 1]);", 0, [L + "test_logits_small_integers_brute_force"]),
    ("post_update adds num_rejected", "num_computed[s] += query_len[r] - num_rejected[r];",
     "num_computed[s] += query_len[r] + num_rejected[r];", 0, [P + "test_post_update_example_and_rollback_rule"]),
    ("post_update records the first token", "last_sampled[s] = tok[n - 1];", "last_sampled[s] = tok[0];", 0,
     [P + "test_post_update_example_and_rollback_rule"]),
]


def replace_nth(text, old, new, n):
    at = -1
    for _ in range(n + 1):
        at = text.find(old, at + 1)
        assert at >= 0, f"mutation target not found: {old!r}"
    return text[:at] + new + text[at + len(old):]


def run_pins(so, pins):
    env = dict(os.environ, SV_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", *pins],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


def build_and_run(tmp, i, text, pins):
    d = os.path.join(tmp, f"m{i}")
    os.makedirs(d, exist_ok=True)
    src = os.path.join(d, "oracle.c")
    shutil.copy(os.path.join(ROOT, "oracle", "oracle.h"), d)
    with open(src, "w") as f:
        f.write(text)
    so = oracle.compile_to(src, os.path.join(d, "liborc.so"))
    return run_pins(so, pins)


def test_every_planted_mistake_fails_a_pin(tmp_path):
    base = open(SRC).read()
    jobs = [(i, replace_nth(base, old, new, n), pins) for i, (_, old, new, n, pins) in enumerate(MUTATIONS)]
    for _, text, _ in jobs:
        assert text != base
    all_pins = sorted({p for *_, pins in MUTATIONS for p in pins})
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        clean = ex.submit(build_and_run, str(tmp_path), "clean", base, all_pins)
        res = list(ex.map(lambda j: build_and_run(str(tmp_path), *j), jobs))
    rc, out = clean.result()
    assert rc == 0, f"unmutated oracle fails its pins:\n{out}"
    survived = [(MUTATIONS[i][0], out) for i, (rc, out) in enumerate(res) if rc != 1]
    assert not survived, "mutations no pin caught:\n" + "\n".join(f"{n}: {o[-400:]}" for n, o in survived)
