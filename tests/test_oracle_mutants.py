"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them."""
import os

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "gqa_oracle.c")

# (name, exact text in gqa_oracle.c, replacement)
MUTANTS = [
    ("interleaved_groups", "const int g = h / r;", "const int g = h % J->G;"),
    ("dropped_scale", "s[t] = J->scale * acc;", "s[t] = acc;"),
    ("keys_from_values", "acc += widen(J->q, q_off + i, J->elem) * widen(J->k,",
     "acc += widen(J->q, q_off + i, J->elem) * widen(J->v,"),
    ("reversed_query", "widen(J->q, q_off + i, J->elem)", "widen(J->q, q_off + (d - 1 - i), J->elem)"),
    ("flipped_exponent", "s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    ("no_max_shift", "s[t] = exp(s[t] - m);", "s[t] = exp(s[t]);"),
    ("no_normalisation", "const double p = s[t] / Z;", "const double p = s[t];"),
    ("ignores_lengths", "long n = J->seq_lens[b];", "long n = J->Lmax;"),
    ("off_by_one_length", "long n = J->seq_lens[b];", "long n = J->seq_lens[b] - 1;"),
    ("no_max", "if (s[t] > m) m = s[t];", "if (s[t] < m) m = s[t];"),
    ("window_one_short", "lo = n - J->window;", "lo = n - J->window + 1;"),
    ("window_one_long", "lo = n - J->window;", "lo = n - J->window - 1;"),
    ("window_ignored", "if (J->window > 0 && n > J->window)", "if (0)"),
    ("append_wrong_row", "(size_t)Lmax + (size_t)(n - 1)) * d;", "(size_t)Lmax + (size_t)(n > 1 ? n - 2 : 0)) * d;"),
    ("append_value_from_key", "(const char *)v_new + src * es", "(const char *)k_new + src * es"),
    ("append_skipped", "memcpy((char *)k_cache + dst * es", "if (0) memcpy((char *)k_cache + dst * es"),
    ("matmul_transposed_w", "widen(w, (size_t)k * N + n, elem)", "widen(w, (size_t)n * K + k, elem)"),
    ("matmul_drops_last_k", "for (int k = 0; k < K; ++k)\n        acc +=", "for (int k = 0; k < K - 1; ++k)\n        acc +="),
    ("pool_divides_by_G", "(float)(acc / (double)r)", "(float)(acc / (double)G)"),
    ("pool_interleaved_columns", "acc += (double)wr[(size_t)i * h + c];", "acc += (double)wr[(size_t)c * H + i];"),
    ("pool_float_accumulator", "double acc = (double)wr[(size_t)(g * r) * h + c];",
     "float acc = wr[(size_t)(g * r) * h + c];"),
    ("pool_skips_first", "for (int i = g * r + 1; i < g * r + r; ++i)", "for (int i = g * r + 2; i < g * r + r; ++i)"),
    ("pool_wrong_group_base", "double acc = (double)wr[(size_t)(g * r) * h + c];",
     "double acc = (double)wr[(size_t)(g) * h + c];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) >= 1, "mutation site vanished: " + old
    src = tmp_path / ("mutant_%s.c" % name)
    src.write_text(text.replace(old, new))
    lib = oracle.build(str(src), str(tmp_path / ("mutant_%s.so" % name)))
    mut = oracle.Oracle(lib)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, "no pin caught mutant %s" % name
