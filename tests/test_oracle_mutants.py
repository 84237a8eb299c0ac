"""Mutation check of the oracle pins (CPU only).

Each mutant is a copy of the oracle source with one plausible mistake planted in it (a dropped
term, a wrong sign, a wrong index, a swapped operand), compiled to a temporary library.  The
pins of tests/oracle_pins.py must reject every mutant; a mutant that passes them all means a
class of mistakes the pins cannot see.

Every mutant runs in a child process of its own: a planted index mistake can write outside an
array (a sequence reading another sequence's block table reaches an unallocated -1 entry), and
the heap it corrupts must not be the test runner's.  A child that dies of a signal has been
caught too: the mistake is loud.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "qdec_oracle.c")

# (name, [(old, new), ...]): every `old` must occur exactly once in the oracle source
MUTANTS = [
    ("f16_rebias", [("(e + 112u)", "(e + 111u)")]),
    ("bf16_truncate", [("b += 0x7FFFu + lsb;", "b += 0u * lsb;")]),
    ("int4_zero_point", [("(float)(nib - 8)", "(float)(nib - 7)")]),
    ("int4_nibble_order", [("(k % 2 == 0) ? (byte & 0x0F) : (byte >> 4)",
                            "(k % 2 == 0) ? (byte >> 4) : (byte & 0x0F)")]),
    ("int4_group_index", [("orc_f16_to_f32(sc[g])", "orc_f16_to_f32(sc[g / 2])")]),
    ("int8_row_scale", [("float s = ((const float *)S)[row];", "float s = ((const float *)S)[0];")]),
    ("gemv_drop_bias", [("if (bias) acc += (double)bias[n];", "")]),
    ("rms_drop_eps", [("sqrt(ss / dim + eps)", "sqrt(ss / dim)")]),
    ("rms_sum_not_mean", [("sqrt(ss / dim + eps)", "sqrt(ss + eps)")]),
    ("rms_drop_gain", [("double g = gamma ? (double)gamma[i] : 1.0;", "double g = 1.0;")]),
    ("rope_sign", [("xr[i] = (float)(a * c - b * s);", "xr[i] = (float)(a * c + b * s);")]),
    ("rope_schedule", [("pow(base, -2.0 * (double)i / (double)dim)",
                        "pow(base, -1.0 * (double)i / (double)dim)")]),
    ("rope_pairing", [("int half = dim / 2;", "int half = dim / 4;")]),
    ("swiglu_sign", [("z / (1.0 + exp(-z))", "z / (1.0 + exp(z))")]),
    ("swiglu_swap", [("double z = g[i];", "double z = u[i];"), ("(double)u[i]", "(double)g[i]")]),
    ("attn_drop_scale", [("s[t] = acc * scale;", "s[t] = acc;")]),
    ("attn_head_map", [("int j = h / G;", "int j = h % Hkv;")]),
    ("attn_page_table", [("int64_t page = page_table[t / page_size];",
                          "int64_t page = t / page_size;")]),
    ("step_exclude_new_token", [("T = pos + 1;", "T = pos;")]),
    ("step_v_from_k", [("Hkv, D, pos, v);", "Hkv, D, pos, k);")]),
    ("step_drop_o_residual", [("att, NULL, h, h, H, qd", "att, NULL, NULL, h, H, qd")]),
    ("step_drop_down_residual", [("m, NULL, h, h, H, I", "m, NULL, NULL, h, H, I")]),
    ("step_ffn_uses_attn_gain", [("orc_rmsnorm(h, L->g_ffn, a, 1, H, c->eps);",
                                  "orc_rmsnorm(h, L->g_attn, a, 1, H, c->eps);")]),
    ("step_drop_qk_norm", [("orc_rmsnorm(q, L->g_q, q, Hq, D, c->eps);", "")]),
    ("step_drop_final_norm", [("orc_rmsnorm(h, head->g_out, a, 1, H, c->eps);",
                               "memcpy(a, h, sizeof(float) * (size_t)H);")]),
    ("step_embed_row", [("head->embed[(int64_t)token * H + i]",
                         "head->embed[(int64_t)token * H + (H - 1 - i)]")]),
    ("argmax_last_tie", [("v[i] > v[best]", "v[i] >= v[best]")]),
    ("a8_round_trunc", [("float r = rintf(t);", "float r = truncf(t);")]),
    ("a8_round_half_away", [("float r = rintf(t);", "float r = roundf(t);")]),
    ("a8_signed_amax", [("const float a = fabsf(xg[i]);", "const float a = xg[i];")]),
    ("a8_scale_128", [("sx[g] = amax / 127.0f;", "sx[g] = amax / 128.0f;")]),
    ("a8_first_group_scale", [("acc += ws * (double)sx[g] * (double)isum;",
                               "acc += ws * (double)sx[0] * (double)isum;")]),
    ("a8_zero_point", [("isum += (int64_t)(nib - 8) * q[k];", "isum += (int64_t)(nib - 7) * q[k];")]),
    ("a8_nibble_order", [("(k % 2 == 0) ? (b[k / 2] & 0x0F) : (b[k / 2] >> 4);",
                          "(k % 2 == 0) ? (b[k / 2] >> 4) : (b[k / 2] & 0x0F);")]),
    ("a8_drop_residual", [("if (residual != NULL) acc += (double)residual[n];", "")]),
    ("a8_drop_bias", [("if (bias != NULL) acc += (double)bias[n];", "")]),
    ("philox_multiplier", [("0xCA5A826395121157ull", "0xCA5A826395121155ull")]),
    ("philox_nine_rounds", [("for (int r = 0; r < 10; ++r) {\n    const unsigned __int128",
                             "for (int r = 0; r < 9; ++r) {\n    const unsigned __int128")]),
    ("uniform_word", [("return ((double)(w[i & 3] >> 11)", "return ((double)(w[0] >> 11)")]),
    ("uniform_counter_order", [("{(uint64_t)i >> 2, (uint64_t)step, 0, 0}", "{(uint64_t)step, (uint64_t)i >> 2, 0, 0}")]),
    ("sample_temperature_mul", [("(float)((double)logits[i] / temperature + g)", "(float)((double)logits[i] * temperature + g)")]),
    ("sample_gumbel_sign", [("const double g = -log(-log(", "const double g = log(-log(")]),
    ("sample_topp_strict", [("if (cum >= top_p * tot) {", "if (cum > top_p * tot) {")]),
    ("sample_topk_tie_order", [("  return x->i - y->i;", "  return y->i - x->i;")]),
    ("sample_greedy_threshold", [("if (!(temperature > 0.0)) return orc_argmax", "if (!(temperature > 1.0)) return orc_argmax")]),
    ("sample_topk_off_by_one", [("if (filt_k) n = top_k;", "if (filt_k) n = top_k + 1;")]),
    ("batch_first_table", [("block_tables + (int64_t)b * max_blocks, pos[b]", "block_tables, pos[b]")]),
    ("batch_shared_hidden", [("h + (int64_t)b * c->hidden, NULL,", "h, NULL,")]),
    ("batch_shared_logits", [("logits ? logits + (int64_t)b * c->vocab : NULL", "logits")]),
    ("prefill_fixed_position", [("page_table, pos0 + t, tokens[t], h, NULL", "page_table, pos0, tokens[t], h, NULL")]),
    ("prefill_first_logits", [("t == T - 1 ? logits : NULL", "t == 0 ? logits : NULL"),
                              ("t == T - 1 ? c : &body", "t == 0 ? c : &body")]),
]


_CHILD = r"""
import sys
sys.path[:0] = sys.argv[2:]
import oracle as O
import oracle_pins as P
O.use_library(sys.argv[1])
for chk in P.ALL_CHECKS:
    try:
        chk()
    except AssertionError:
        print("caught by", chk.__name__)
        break
else:
    print("passed every pin")
"""


def _run_mutant(name, edits, source, work):
    src = source
    for old, new in edits:
        if src.count(old) != 1:
            return None, f"mutation site for {name} not unique: {old!r}", ""
        src = src.replace(old, new)
    c = os.path.join(work, name + ".c")
    with open(c, "w") as f:
        f.write(src)
    so = os.path.join(work, "lib" + name + ".so")
    subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                           "-I", os.path.dirname(SRC), c, "-o", so, "-lm"])
    tests = os.path.dirname(os.path.abspath(__file__))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", _CHILD, so, tests, os.path.dirname(tests)],
                       capture_output=True, text=True, env=env, timeout=600)
    return r.returncode, r.stdout, r.stderr


@pytest.fixture(scope="module")
def verdicts(tmp_path_factory):
    with open(SRC) as f:
        source = f.read()
    work = str(tmp_path_factory.mktemp("mutants"))
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {name: ex.submit(_run_mutant, name, edits, source, work) for name, edits in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, verdicts):
    rc, out, err = verdicts[name]
    assert rc is not None, out
    if rc < 0:
        return  # the planted mistake crashed the oracle (e.g. an out-of-bounds write)
    assert rc == 0, f"mutant {name}: child failed\n{err[-2000:]}"
    assert "caught by" in out, f"mutant {name} passed every pin"
