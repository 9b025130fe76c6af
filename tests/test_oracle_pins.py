"""The fp64 oracle against its pins (CPU only).

Every pin in ``oracle_pins`` must hold for the real oracle, and every planted
mistake in a copy of the oracle's C source (a dropped term, a wrong sign, a
wrong index, a transposed operand) must break at least one pin.  Mistakes are
planted only in a temporary copy of the oracle, on the CPU.
"""
import os

import pytest

import oracle
import oracle_pins

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.default())


# (description, exact text in msda_oracle.c, replacement)
MUTANTS = [
    ("pixel centre offset dropped", "double x = u * (double)W - 0.5;",
     "double x = u * (double)W;"),
    ("y scaled by W (transposed shape)", "double y = v * (double)H - 0.5;",
     "double y = v * (double)W - 0.5;"),
    ("corner 01 weight transposed", "cs->w[1] = lx * (1.0 - ly);",
     "cs->w[1] = ly * (1.0 - lx);"),
    ("corner 11 weight wrong", "cs->w[3] = lx * ly;", "cs->w[3] = lx * lx;"),
    ("row stride H instead of W", "cs->row[c] = start + (int64_t)cy[c] * W + (int64_t)cx[c];",
     "cs->row[c] = start + (int64_t)cy[c] * H + (int64_t)cx[c];"),
    ("level start ignored", "cs->row[c] = start + (int64_t)cy[c] * W + (int64_t)cx[c];",
     "cs->row[c] = (int64_t)cy[c] * W + (int64_t)cx[c];"),
    ("x bound off by one", "cx[c] < (double)W", "cx[c] <= (double)W"),
    ("corner x0+1 swapped to x0-1", "double cx[4] = {x0, x0 + 1.0, x0, x0 + 1.0};",
     "double cx[4] = {x0, x0 - 1.0, x0, x0 - 1.0};"),
    ("attention weight dropped in forward", "o[d] += a * cs.w[c] * vr[d];",
     "o[d] += cs.w[c] * vr[d];"),
    ("value and head index transposed", "const double *vr = value + ((b * S + cs.row[c]) * M + m) * D;\n"
     "                            for (int64_t d = 0; d < D; ++d)\n"
     "                                o[d]",
     "const double *vr = value + ((b * S + cs.row[c]) * M + (M - 1 - m)) * D;\n"
     "                            for (int64_t d = 0; d < D; ++d)\n"
     "                                o[d]"),
    ("grad_out dropped from p_c", "p[c] += g[d] * vr[d];", "p[c] += vr[d];"),
    ("grad_attn uses wrong corner", "cs.w[1] * p[1] + cs.w[2] * p[2]",
     "cs.w[1] * p[2] + cs.w[2] * p[2]"),
    ("grad_loc_x sign flipped", "((1.0 - ly) * (p[1] - p[0]) + ly * (p[3] - p[2]))",
     "((1.0 - ly) * (p[0] - p[1]) + ly * (p[3] - p[2]))"),
    ("grad_loc_x second term wrong corner", "ly * (p[3] - p[2])", "ly * (p[3] - p[1])"),
    ("grad_loc_y chain factor W", "a * (double)H * ((1.0 - lx)", "a * (double)W * ((1.0 - lx)"),
    ("grad_loc_y lx and ly transposed", "((1.0 - lx) * (p[2] - p[0]) + lx * (p[3] - p[1]))",
     "((1.0 - ly) * (p[2] - p[0]) + ly * (p[3] - p[1]))"),
    ("grad_loc attention weight dropped", "a * (double)W * ((1.0 - ly)", "(double)W * ((1.0 - ly)"),
    ("grad_value corner weight dropped", "double aw = a * cs.w[c];", "double aw = a;"),
    ("grad_value not zeroed", "memset(grad_value, 0, (size_t)(B * S * M * D) * sizeof(double));",
     "grad_value[0] += 0.0;"),
    ("empty-sample gradient not cleared", "grad_loc[2 * s] = 0.0;\n", "grad_loc[2 * s] = 1.0;\n"),
    ("softmax not normalised", "a[j] = a[j] / sum;", "a[j] = a[j] / (sum + 1e-3);"),
    ("softmax sum drops the last term", "sum += a[j];", "sum += (j + 1 < lk) ? a[j] : 0.0;"),
    ("softmax derivative sign", "a[j] * (ga[j] - dot)", "a[j] * (ga[j] + dot)"),
    ("softmax derivative drops the weights in the sum", "dot += a[i] * ga[i];", "dot += ga[i];"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(desc, old, new, tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation site for {desc!r} must occur exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(str(mutant_src), str(tmp_path / "libmutant.so"))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except AssertionError as e:
            caught.append(f"{pin.__name__}: {e}")
            break
    assert caught, f"no pin catches the planted mistake: {desc}"


def test_oracle_source_has_no_gpu_dependency():
    """The oracle shares nothing with the GPU library: it includes no header of it."""
    src = open(oracle.SOURCE).read()
    assert "#include \"" not in src and "hip" not in src.lower()
    here = os.path.dirname(oracle.SOURCE)
    assert not [f for f in os.listdir(here) if f.endswith((".h", ".hip", ".cpp"))]
