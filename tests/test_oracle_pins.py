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
    ("pixel centre offset dropped", "double x = u * (double)W - 0.5;\n                        double y = v * (double)H - 0.5;\n                        cell_taps t;\n                        cell_of(x, y, H, W, &t);\n                        double *dst",
     "double x = u * (double)W;\n                        double y = v * (double)H - 0.5;\n                        cell_taps t;\n                        cell_of(x, y, H, W, &t);\n                        double *dst"),
    ("y scaled by W (transposed shape)", "double y = v * (double)H - 0.5;\n                        cell_taps t;\n                        cell_of(x, y, H, W, &t);\n                        double *dst",
     "double y = v * (double)W - 0.5;\n                        cell_taps t;\n                        cell_of(x, y, H, W, &t);\n                        double *dst"),
    ("tent kernel of the wrong shape", "return a < 1.0 ? 1.0 - a : 0.0;",
     "return a < 1.0 ? 1.0 - a * a : 0.0;"),
    ("tent factors use one axis twice", "t->wy[t->n] = tent(y - py);", "t->wy[t->n] = tent(x - px);"),
    ("row stride H instead of W", "t->pix[t->n] = (int64_t)py * W + (int64_t)px;",
     "t->pix[t->n] = (int64_t)py * H + (int64_t)px;"),
    ("level start ignored", "const double *img = value + ((b * S + level_start_index[l]) * M + m) * D;",
     "const double *img = value + ((b * S) * M + m) * D;"),
    ("x bound off by one", "px < (double)W", "px <= (double)W"),
    ("second column swapped to x0-1", "double px = xc + (double)dx;", "double px = xc - (double)dx;"),
    ("attention weight dropped in forward", "o[d] += a * smp[j][d];", "o[d] += smp[j][d];"),
    ("value and head index transposed",
     "const double *img = value + ((b * S + level_start_index[l]) * M + m) * D;",
     "const double *img = value + ((b * S + level_start_index[l]) * M + (M - 1 - m)) * D;"),
    ("grad_out dropped from grad_attn", "ga += g[d] * smp[d];", "ga += smp[d];"),
    ("grad_attn takes the x-derivative", "grad_attn[s] = ga;", "grad_attn[s] = gx;"),
    ("left-column slope sign flipped", "t->sx[t->n] = (px == xc) ? -1.0 : 1.0;",
     "t->sx[t->n] = (px == xc) ? 1.0 : -1.0;"),
    ("x-derivative drops the y factor", "dsx[d] += t.sx[c] * t.wy[c] * vr[d];",
     "dsx[d] += t.sx[c] * vr[d];"),
    ("grad_loc_y chain factor W", "a * (double)H * gy", "a * (double)W * gy"),
    ("grad_loc_y takes the x-slopes", "dsy[d] += t.wx[c] * t.sy[c] * vr[d];",
     "dsy[d] += t.sx[c] * t.wy[c] * vr[d];"),
    ("grad_loc attention weight dropped", "a * (double)W * gx", "(double)W * gx"),
    ("grad_value tent weights dropped", "double aw = a * t.wx[c] * t.wy[c];", "double aw = a;"),
    ("grad_value not zeroed", "memset(grad_value, 0, (size_t)(B * S * M * D) * sizeof(double));",
     "grad_value[0] += 0.0;"),
    ("grad_value row of the wrong level", "const int64_t row0 = b * S + level_start_index[l];",
     "const int64_t row0 = b * S + level_start_index[0];"),
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
