"""Plants plausible mistakes in copies of the oracle (on the CPU) and checks that the pin tests
catch every one of them. The real oracle source is never modified."""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mx_oracle.c")
PIN_TESTS = [os.path.join(ROOT, "tests", "test_oracle_codec.py"),
             os.path.join(ROOT, "tests", "test_oracle_path.py"),
             os.path.join(ROOT, "tests", "test_oracle_fragile.py"),
             os.path.join(ROOT, "tests", "test_oracle_operand.py"),
             os.path.join(ROOT, "tests", "test_oracle_act.py")]

# (name, exact text in mx_oracle.c, replacement)
MUTANTS = [
    ("tie-to-odd", "(d == best_d && (c & 1) == 0)", "(d == best_d && (c & 1) == 1)"),
    ("scale-minus-1", "s = (q - 1) - 2;", "s = (q - 1) - 1;"),
    ("scale-ceil", "s = (q - 1) - 2;", "s = q - 2;"),
    ("no-lower-clamp", "if (s < -127) s = -127;", ";"),
    ("nibble-order-pack", "codes[2 * j] | (codes[2 * j + 1] << 4)",
     "codes[2 * j + 1] | (codes[2 * j] << 4)"),
    ("nibble-order-decode", "(k & 1) ? (byte >> 4) : (byte & 0xfu)",
     "(k & 1) ? (byte & 0xfu) : (byte >> 4)"),
    ("negative-zero-sign", "(signbit(x[i]) ? 8 : 0)", "(x[i] < 0 ? 8 : 0)"),
    ("e2m1-bias", "ldexp(1.0 + 0.5 * (double)m, (int)e - 1)", "ldexp(1.0 + 0.5 * (double)m, (int)e - 2)"),
    ("e8m0-bias", "ldexp(1.0, (int)b - 127)", "ldexp(1.0, (int)b - 128)"),
    ("nonfinite-not-flagged", "*scale = 255;", "*scale = 254;"),
    ("topk-tie-high-index", "if (best < 0 || l[e] > l[best]) best = e;",
     "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("softmax-denominator", "(float)(exp(sel[j] - mx) / sum)", "(float)(exp(sel[j] - mx) / (sum + 1e-3))"),
    ("router-no-bias", "if (br) acc += (double)br[e];", ";"),
    ("permute-unstable", "int32_t row = offsets[e] + fill[e]++;",
     "int32_t row = offsets[e + 1] - 1 - fill[e]++;"),
    ("swiglu-gate-up-swapped", "double g = a[gi], u = a[ui];\n        if (limit > 0.0) {",
     "double g = a[ui], u = a[gi];\n        if (limit > 0.0) {"),
    ("silu-sign", "hv[f] = g / (1.0 + exp(-alpha * g)) * (u + shift);",
     "hv[f] = g / (1.0 + exp(alpha * g)) * (u + shift);"),
    ("routing-weight-dropped", "o[m] += wt * acc;", "o[m] += acc;"),
    ("down-expert-stride", "prow = dn_packed + ((int64_t)e * H + m) * dn_row",
     "prow = dn_packed + ((int64_t)e * F + m) * dn_row"),
    ("mx-act-h-skipped", "activation_row(hb, F, mx_act, h);", "activation_row(hb, F, 0, h);"),
    ("bf16-truncates", "nearbyint(a / quantum)", "floor(a / quantum)"),
    # the weight operand of the products (bf16 operand on the bf16 path, exact on the FP4 path)
    ("bf16-operand-skipped", "return bf16_operand ? g_dq_bf16[b][c] : g_dq_exact[b][c];",
     "return g_dq_exact[b][c];"),
    ("bf16-operand-in-fp4-linear", "acc += xr[kk] * weight_elem(prow, srow, kk, !mx_act);",
     "acc += xr[kk] * weight_elem(prow, srow, kk, 1);"),
    ("gate-up-exact-operand", "const double term = xr[kk] * weight_elem(prow, srow, kk, !mx_act);",
     "const double term = xr[kk] * decode_elem(prow, srow, kk);"),
    ("down-exact-operand", "acc += h[f] * weight_elem(prow, srow, f, !mx_act);",
     "acc += h[f] * decode_elem(prow, srow, f);"),
    ("tables-subnormal-flush", "g_dq_bf16[b][c] = mxo_double_from_bf16(mxo_bf16_from_double(g_dq_exact[b][c]));",
     "g_dq_bf16[b][c] = fabs(g_dq_exact[b][c]) < 0x1p-126 ? 0.0 : mxo_double_from_bf16(mxo_bf16_from_double(g_dq_exact[b][c]));"),
    # the parameterised expert activation
    ("act-gate-clamped-below", "g = fmin(g, limit);", "g = fmax(fmin(g, limit), -limit);"),
    ("act-up-not-clamped", "u = fmax(fmin(u, limit), -limit);", ";"),
    ("act-alpha-ignored", "hv[f] = g / (1.0 + exp(-alpha * g)) * (u + shift);",
     "hv[f] = g / (1.0 + exp(-g)) * (u + shift);"),
    ("act-shift-dropped", "hv[f] = g / (1.0 + exp(-alpha * g)) * (u + shift);",
     "hv[f] = g / (1.0 + exp(-alpha * g)) * u;"),
    ("act-interleave-ignored",
     "const int gi = interleaved ? 2 * f : f, ui = interleaved ? 2 * f + 1 : F + f;\n        double g",
     "const int gi = f, ui = F + f;\n        double g"),
    ("act-gate-up-bias-dropped", "if (gu_bias) acc += (double)gu_bias[(int64_t)e * 2 * F + n];", ";"),
    ("act-down-bias-unweighted",
     "if (dn_bias) acc += (double)dn_bias[(int64_t)e * H + m];\n        o[m] += wt * acc;",
     "o[m] += wt * acc;\n        if (dn_bias) o[m] += (double)dn_bias[(int64_t)e * H + m];"),
    # the fragile-decision aid of the activation variant
    ("fragile-slack-unweighted", "sl[m] += wt * d;", "sl[m] += d;"),
    ("fragile-alt-two-steps", "if (up != neg) return (uint16_t)(b + 1);",
     "if (up != neg) return (uint16_t)(b + 2);"),
    ("fragile-no-block-check", "if (!differs) continue;", ";"),
    ("fragile-slack-wrong-weight-row", "wrow = dn_packed + ((int64_t)e * H + m) * dn_row",
     "wrow = dn_packed + ((int64_t)e * H + (m + 1) % H) * dn_row"),
]


def _run_mutant(args):
    name, old, new, tmp = args
    with open(SRC) as f:
        src = f.read()
    assert old is None or src.count(old) == 1, "mutation site for %s not found once" % name
    if old is None:  # the unmodified source, built the same way: must pass
        old = new = ""
    msrc = os.path.join(tmp, "mut_%s.c" % name)
    with open(msrc, "w") as f:
        f.write(src.replace(old, new) if old else src)
    mlib = os.path.join(tmp, "libmut_%s.so" % name)
    oracle.build(src=msrc, out=mlib)
    env = dict(os.environ, MXO_ORACLE_LIB=mlib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PIN_TESTS], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return name, r.returncode


@pytest.mark.timeout(900)
def test_every_planted_mistake_is_caught():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(4) as ex:
            results = list(ex.map(_run_mutant, [("unmodified", None, None, tmp)] +
                                  [(n, o, w, tmp) for n, o, w in MUTANTS]))
    assert results[0] == ("unmodified", 0), "the harness fails even without a planted mistake"
    results = results[1:]
    survivors = [n for n, rc in results if rc == 0]
    assert not survivors, "planted mistakes not caught by the pins: %s" % survivors
