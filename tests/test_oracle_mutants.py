"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins reject every one of them.  The mutated sources live only in a
temporary directory; the real oracle is untouched."""
import json
import os
import subprocess
import sys
import tempfile

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# (name, original text, mutated text)
MUTANTS = [
    ("tie_goes_left", "const int bit = !(left > m) && right != 0.0f;",
     "const int bit = !(left >= m) && right != 0.0f;"),
    ("no_zero_guard", "const int bit = !(left > m) && right != 0.0f;",
     "const int bit = !(left > m);"),
    ("children_swapped", "const float left = sum[2 * node], right = sum[2 * node + 1];",
     "const float left = sum[2 * node + 1], right = sum[2 * node];"),
    ("mass_added", "if (bit) m -= left;", "if (bit) m += left;"),
    ("mass_not_reduced", "if (bit) m -= left;", "if (bit) m -= 0.0f;"),
    ("sum_drops_right", "t->sum[i] = l + r;", "t->sum[i] = l;"),
    ("sum_wrong_index", "float l = t->sum[2 * i], r = t->sum[2 * i + 1];",
     "float l = t->sum[2 * i], r = t->sum[2 * i];"),
    ("min_is_max", "t->mn[i] = (b < a) ? b : a;", "t->mn[i] = (b < a) ? a : b;"),
    ("walk_skips_root", "for (i >>= 1; i >= 1; i >>= 1)", "for (i >>= 1; i > 1; i >>= 1)"),
    ("is_sign", "pow(N * P_i, -beta) / pow(N * P_min, -beta)",
     "pow(N * P_i, beta) / pow(N * P_min, beta)"),
    ("is_unnormalised", "double P_min = (double)pmin / (double)total;", "double P_min = 1.0;"),
    ("is_drops_N", "pow(N * P_i, -beta) /", "pow(P_i, -beta) /"),
    ("prio_eps_outside", "(float)pow((double)x + t->eps, t->alpha)",
     "(float)(pow((double)x, t->alpha) + t->eps)"),
    ("prio_in_f32", "(float)pow((double)x + t->eps, t->alpha)",
     "powf(x + (float)t->eps, (float)t->alpha)"),
    ("prio_no_abs", "float x = fabsf(td);", "float x = td;"),
    ("nan_to_max", "if (isnan(x)) return (float)pow(t->eps, t->alpha);",
     "if (isnan(x)) return max_at_start;"),
    ("inf_to_current_max", "if (isinf(x)) return max_at_start;", "if (isinf(x)) return t->maxp;"),
    ("first_position_wins", "for (int64_t b = 0; b < B; ++b) {\n        int64_t slot = idx[b];",
     "for (int64_t b = B - 1; b >= 0; --b) {\n        int64_t slot = idx[b];"),
    ("skip_off_by_one", "slot >= t->size", "slot > t->size"),
    ("intake_at_one", "p = t->maxp;", "p = 1.0f;"),
    ("cursor_no_wrap", "t->cursor = (t->cursor + count) % t->n;",
     "t->cursor = (t->cursor + count);"),
    ("size_no_cap", "t->size = (t->size + count < t->n) ? t->size + count : t->n;",
     "t->size = t->size + count;"),
    ("given_prio_not_raising_max", "if (p > t->maxp) t->maxp = p;\n        } else {",
     "} else {"),
    ("negative_zero_kept", "p = prio[j] + 0.0f;", "p = prio[j];"),
    ("pad_not_zero", "(c < D) ? t->states[slot * D + c] : 0.0f;",
     "(c < D) ? t->states[slot * D + c] : t->states[slot * D];"),
    ("pad_stride_ignored", "next_states_out[b * out_stride + c] =",
     "next_states_out[b * D + c] ="),
    ("dones_as_bool", "dones_out[b] = (float)t->dones[slot];",
     "dones_out[b] = t->dones[slot] ? 1.0f : 0.0f;"),
    ("pad_accepts_short_stride", "if (out_stride < D) return -1;", "if (out_stride < 0) return -1;"),
    ("philox_round_constant", "0xD2E7470EE14C6C93ull", "0xD2E7470EE14C6C95ull"),
    ("philox_no_key_bump", "            k1 += 0xBB67AE8584CAA73Bull;\n", ""),
    ("philox_nine_rounds", "for (int r = 0; r < 10; ++r)", "for (int r = 0; r < 9; ++r)"),
    ("stream_word_order", "return out[j % 4];", "return out[3 - j % 4];"),
    ("mass_wrong_bits", ">> 40) * 0x1p-24f", ">> 41) * 0x1p-24f"),
    ("rank_ties_by_slot_desc", "return (x->slot < y->slot) ? -1 : (x->slot > y->slot);",
     "return (x->slot > y->slot) ? -1 : (x->slot < y->slot);"),
    ("rank_ascending", "if (x->p > y->p) return -1;\n    if (x->p < y->p) return 1;",
     "if (x->p > y->p) return 1;\n    if (x->p < y->p) return -1;"),
    ("rank_weight_off_by_one", "pow((double)(r + 1), -t->alpha)", "pow((double)(r + 2), -t->alpha)"),
    ("rank_weight_sign", "pow((double)(r + 1), -t->alpha)", "pow((double)(r + 1), t->alpha)"),
    ("rank_descends_priorities", "descend_tree(t->rsum, t->n, m)", "descend_tree(t->sum, t->n, m)"),
    ("rank_slot_not_through_order", "const int64_t slot = t->order[r];", "const int64_t slot = r;"),
    ("uniform_modulo", "(int64_t)((hi * (uint64_t)t->size) >> 32)", "(int64_t)(hi % (uint64_t)t->size)"),
]

_RUNNER = r"""
import json, sys
sys.path.insert(0, %(root)r)
sys.path.insert(0, %(tests)r)
import oracle, pins
lib = oracle.load(%(lib)r)
failed = []
for pin in pins.ALL_PINS:
    try:
        pin(lib)
    except Exception as e:
        failed.append(pin.__name__)
print(json.dumps(failed))
"""


def _build_mutant(src: str, tmp: str) -> str:
    c = os.path.join(tmp, "pero.c")
    with open(c, "w") as f:
        f.write(src)
    with open(os.path.join(os.path.dirname(oracle.__file__), "pero.h")) as f:
        hdr = f.read()
    with open(os.path.join(tmp, "pero.h"), "w") as f:
        f.write(hdr)
    so = os.path.join(tmp, "libpero_mutant.so")
    subprocess.check_call(["gcc", *oracle.CFLAGS, "-o", so, c, "-lm"])
    return so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new):
    with open(os.path.join(os.path.dirname(oracle.__file__), "pero.c")) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation site not found exactly once: %s" % name
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(src.replace(old, new), tmp)
        code = _RUNNER % dict(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=so)
        r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                           timeout=600)
        if r.returncode != 0:
            # a crash of the mutant also counts as rejected
            return
        failed = json.loads(r.stdout.strip().splitlines()[-1])
        assert failed, "no pin caught mutant %s" % name
