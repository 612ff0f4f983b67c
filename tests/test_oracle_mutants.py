"""Plants plausible mistakes in copies of the oracle's C source (on the CPU) and checks that the
pin set rejects every one of them: evidence that the pins would catch such a mistake in the
oracle itself."""
import os
import tempfile

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "conv_oracle.c")

# (name, exact source text, replacement); each text must occur in the source.
MUTANTS = [
    ("kernel flipped in rows", "const int ih = stride * oh - 1 + ky;", "const int ih = stride * oh + 1 - ky;"),
    ("padding offset dropped", "const int iw = stride * ow - 1 + kx;", "const int iw = stride * ow + kx;"),
    ("temporal tap flipped", "const int id = od - 1 + kd;", "const int id = od + 1 - kd;"),
    ("stride ignored in 2D", "const int ih = stride * oh - 1 + ky;\n                        if (ih < 0 || ih >= H) continue; /* zero padding */",
     "const int ih = oh - 1 + ky;\n                        if (ih < 0 || ih >= H) continue; /* zero padding */"),
    ("bias dropped", "double acc = b ? tab[b[co]] : 0.0;", "double acc = 0.0;"),
    ("ReLU keeps negatives", "if (epi == OR_EPI_RELU) return v < 0.0 ? 0.0 : v;", "if (epi == OR_EPI_RELU) return v;"),
    ("clamp bound wrong", "return fmin(1.0, fmax(-1.0, v));", "return fmin(1.0, fmax(0.0, v));"),
    ("weight ky/kx transposed", "tab[w[((((int64_t)co * C_in + ci) * 3 + kd) * 3 + ky) * 3 + kx]];",
     "tab[w[((((int64_t)co * C_in + ci) * 3 + kd) * 3 + kx) * 3 + ky]];"),
    ("split tap channel transposed", "* GC + (ky * 3 + kx) * C_out + co] = acc;", "* GC + (kx * 3 + ky) * C_out + co] = acc;"),
    ("f16 exponent bias off by one", "v = ldexp((double)(1024 + m), e - 25);", "v = ldexp((double)(1024 + m), e - 24);"),
    ("bf16 subnormal scale wrong", "v = ldexp((double)m, -133);", "v = ldexp((double)m, -126);"),
    ("rounding truncates", "double n = rint(a / q);", "double n = floor(a / q);"),
    ("channels-last offset wrong", "return (((n * D + d) * H + h) * W + w) * C + c;", "return (((n * D + d) * W + w) * H + h) * C + c;"),
    ("one C_in channel skipped", "for (int ci = 0; ci < C_in; ++ci) {\n                                const double wv",
     "for (int ci = 1; ci < C_in; ++ci) {\n                                const double wv"),
]


def _failing_pins(orc):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # noqa: BLE001 - any failure counts as a rejection
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, tmp_path):
    with open(SRC) as fh:
        src = fh.read()
    assert src.count(old) >= 1, "mutation site not found: " + name
    mutated = src.replace(old, new)
    cfile = tmp_path / "mutant.c"
    cfile.write_text(mutated)
    lib = oracle.build(force=True, src=str(cfile), out=str(tmp_path / "libmutant.so"))
    failed = _failing_pins(oracle.Oracle(lib))
    assert failed, "no pin rejects the mutant: " + name
