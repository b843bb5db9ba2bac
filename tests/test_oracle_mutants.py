"""The oracle's pins are sharp enough: each plausible mistake planted in a copy
of the oracle source (on the CPU) makes at least one pin fail."""
import ctypes
import os
import subprocess
import tempfile

import pytest

from oracle import oracle
from tests import oracle_pins_lib as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "rnn_oracle.c")

# (name, original text, planted mistake)
MUTANTS = [
    ("lstm gate blocks o/f swapped", "double pi = pre[0] + (Pd ? Pd[j] * c[j] : 0.0);\n        double pf = pre[2]",
     "double pi = pre[0] + (Pd ? Pd[j] * c[j] : 0.0);\n        double pf = pre[1]"),
    ("peephole P order f<->o", "Pd[2 * H + j] * c[j]", "Pd[H + j] * c[j]"),
    ("peephole o uses previous c", "Pd[H + j] * cnew", "Pd[H + j] * c[j]"),
    ("gru lbr0 as r(R.h)", "const double rech = dot(Rd + nh * H, rh, H);",
     "const double rech = gr[j] * dot(Rd + nh * H, h, H);"),
    ("gru update gate swapped", "hn[j] = (1.0 - gz[j]) * hh + gz[j] * h[j];",
     "hn[j] = gz[j] * hh + (1.0 - gz[j]) * h[j];"),
    ("gru lbr1 Rb outside r", "ph = (xw[nh] + gr[j] * (rec[nh] + rbh)) + wbh;",
     "ph = (xw[nh] + gr[j] * rec[nh] + rbh) + wbh;"),
    ("gru z/r blocks swapped", "const int64_t nz = j, nr = H + j;", "const int64_t nz = H + j, nr = j;"),
    ("reverse starts at Seq-1", "const int64_t t = reverse ? L - 1 - s : s;",
     "const int64_t t = reverse ? S - 1 - s : s;"),
    ("layout 1 X read as layout 0", "(p->layout == 0 ? (t * B + b) * I : (b * S + t) * I)",
     "((t * B + b) * I)"),
    ("layout 1 states read as layout 0", "p->layout == 0 ? (d * B + b) * H : (b * D + d) * H",
     "(d * B + b) * H"),
    ("output gate not clipped", "po = clipv(po, p->clip);", ""),
    ("input_forget f = i", "p->input_forget ? 1.0 - ig :", "p->input_forget ? ig :"),
    ("len 0 keeps state", "Y_h[sidx + j] = L == 0 ? 0.0 : h[j];", "Y_h[sidx + j] = h[j];"),
    ("bias stride per direction", "Bias + d * 2 * (int64_t)G * H", "Bias + d * (int64_t)G * H"),
    ("reverse uses forward activations", "const int* ak = p->act_kind + d * ns;", "const int* ak = p->act_kind;"),
    ("elu form", "alpha * (exp(x) - 1.0)", "alpha * exp(x) - 1.0"),
    ("hardsigmoid no upper clamp", "if (v > 1.0) v = 1.0;", ""),
    ("softplus form", "log1p(exp(x))", "log(2.0 + exp(x))"),
    ("lstm h uses g slot", "hn[j] = og * oracle_activation(ak[2], aa[2], ab[2], cnew);",
     "hn[j] = og * oracle_activation(ak[1], aa[1], ab[1], cnew);"),
    ("recurrence reads R transposed", "rec[n] = dot(Rd + n * H, h, H);",
     "rec[n] = 0.0; for (int64_t k = 0; k < H; ++k) rec[n] += Rd[k * G * H + n] * h[k];"),
    ("Y zero past len dropped", "for (int64_t j = 0; j < H; ++j) y[j] = 0.0;", ""),
    ("bias Wb/Rb added twice Wb", "(Rb ? Rb[n] : 0.0);\n        }", "(Wb ? Wb[n] : 0.0);\n        }"),
    ("clip bound sign", "if (x < -clip) return -clip;", "if (x < -clip) return clip;"),
    ("max_length ignored", "if (p->max_length > 0 && L > p->max_length) L = p->max_length;", ""),
    ("max_length only with lengths", "if (p->max_length > 0 && L > p->max_length) L = p->max_length;",
     "if (lens && p->max_length > 0 && L > p->max_length) L = p->max_length;"),
    ("half ties away from zero", "const double q = rint(a / ldexp(1.0, -24));",
     "const double q = round(a / ldexp(1.0, -24));"),
    ("half normal ties away", "double q = rint(a / ldexp(1.0, e - 10));", "double q = round(a / ldexp(1.0, e - 10));"),
    ("half overflow at the largest value", "if (a >= 65520.0)", "if (a > 65504.0)"),
    ("half truncates", "double q = rint(a / ldexp(1.0, e - 10));", "double q = floor(a / ldexp(1.0, e - 10));"),
]


def _build_mutant(tmp, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique for {name!r}"
    path_c = os.path.join(tmp, "m.c")
    path_so = os.path.join(tmp, "m_%d.so" % abs(hash(name)))
    open(path_c, "w").write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", path_so, path_c, "-lm"])
    return path_so


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new):
    saved = oracle._load()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(tmp, name, old, new)
        lib = ctypes.CDLL(so)
        lib.oracle_rnn.restype = saved.oracle_rnn.restype
        lib.oracle_rnn.argtypes = saved.oracle_rnn.argtypes
        lib.oracle_projection.argtypes = saved.oracle_projection.argtypes
        lib.oracle_activation.restype = saved.oracle_activation.restype
        lib.oracle_activation.argtypes = saved.oracle_activation.argtypes
        lib.oracle_round_half.restype = saved.oracle_round_half.restype
        lib.oracle_round_half.argtypes = saved.oracle_round_half.argtypes
        oracle._lib = lib
        try:
            caught = None
            for pin_name, check in pins.all_pins(oracle.run, oracle.round_half):
                try:
                    check()
                except AssertionError:
                    caught = pin_name
                    break
            assert caught is not None, f"no pin caught the planted mistake {name!r}"
        finally:
            oracle._lib = saved


BRUTE_MUTANTS = [m for m in MUTANTS if not m[0].startswith("half ")]


@pytest.mark.parametrize("name,old,new", BRUTE_MUTANTS, ids=[m[0] for m in BRUTE_MUTANTS])
def test_brute_force_alone_catches_planted_mistake(name, old, new):
    """The 50-digit brute force is a pin of its own: each planted mistake in
    the layer arithmetic makes at least one brute-force case fail."""
    from tests import test_oracle_brute as brute
    saved = oracle._load()
    with tempfile.TemporaryDirectory() as tmp:
        so = _build_mutant(tmp, name, old, new)
        lib = ctypes.CDLL(so)
        lib.oracle_rnn.restype = saved.oracle_rnn.restype
        lib.oracle_rnn.argtypes = saved.oracle_rnn.argtypes
        oracle._lib = lib
        try:
            caught = None
            for case in brute.CASES:
                try:
                    brute.test_oracle_matches_brute_force(*case)
                except AssertionError:
                    caught = case[0]
                    break
            if caught is None:
                for cell in ("RNN", "GRU", "LSTM"):
                    try:
                        brute.test_edge_lengths_and_max_length_brute_force(cell)
                    except AssertionError:
                        caught = f"edges {cell}"
                        break
            assert caught is not None, f"the brute force missed the planted mistake {name!r}"
        finally:
            oracle._lib = saved
