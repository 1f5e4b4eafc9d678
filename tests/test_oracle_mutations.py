"""The oracle's pins catch plausible mistakes.  Each case plants one mistake
in a copy of moe_oracle.c (a textual replacement), builds it, and runs the
oracle's pin tests against that build (BEF_ORACLE_LIB): at least one pin must
fail.  The pin that compares a second compiler's build of the pristine source
is left out, since it would flag any change at all."""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "moe_oracle.c")

MUTANTS = {
    "nibble order swapped": (
        "unsigned nib = (col % 2 == 0) ? (byte & 0xFu) : (byte >> 4);",
        "unsigned nib = (col % 2 == 0) ? (byte >> 4) : (byte & 0xFu);"),
    "shared expert dropped": (
        "for (int32_t m = 0; m < H; ++m) o[m] = y[m];",
        "for (int32_t m = 0; m < H; ++m) o[m] = 0.0 * y[m];"),
    "sigmoid sign flipped": (
        "double sg = 1.0 / (1.0 + exp(-zz));",
        "double sg = 1.0 / (1.0 + exp(zz));"),
    "activation scale dropped (gate)": (
        "gs += (double)xs[kb] * gb;",
        "gs += gb;"),
    "ties to the higher id": (
        "return a > b;",
        "return a >= b;"),
    "reciprocal instead of division": (
        "float t = xb[i] / sc;",
        "float t = xb[i] * (1.0f / sc);"),
    "down operand indices exchanged": (
        "orc_weight(w, 2, e, m, n);",
        "orc_weight(w, 2, e, n, m % w->I);"),
    "rounding ties away from zero": (
        "return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;",
        "return fl + 1.0;"),
    "neighbouring scale block": (
        "int64_t si = ((int64_t)e * rows + row) * (cols / 32) + col / 32;",
        "int64_t si = ((int64_t)e * rows + row) * (cols / 32) + (col / 32 + 1) % (cols / 32);"),
    "router chunk summed in descending h": (
        "for (int32_t h = 64 * c; h < 64 * c + 64; ++h) {",
        "for (int32_t h = 64 * c + 63; h >= 64 * c; --h) {"),
    "SiLU left out": (
        "h[i] = (float)(sv * u[i]);",
        "h[i] = (float)(g[i] * u[i]);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_a_planted_mistake_fails_a_pin(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mut = tmp_path / "moe_oracle.c"
    mut.write_text(src.replace(old, new))
    so = str(tmp_path / "libmutant.so")
    oracle.build(out=so, src=str(mut))
    env = dict(os.environ, BEF_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-k", "not second_compiler",
                        os.path.join(ROOT, "tests", "test_oracle_codecs.py"),
                        os.path.join(ROOT, "tests", "test_oracle_layer.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    caught = [ln for ln in r.stdout.splitlines() if ln.startswith("FAILED")]
    print(name, "->", caught[:1], flush=True)
    assert r.returncode != 0, f"no pin caught: {name}"
