"""Planted mistakes: each test copies the oracle's C source, plants one
plausible slip (a wrong sign, a dropped term or factor, swapped operands,
read-before-write, a wrong group index), compiles the copy on the CPU and
checks that the pins reject it.  This shows the pins are strong enough to
catch such a slip in the oracle itself.  Nothing here touches the GPU or the
HIP library, and the real oracle is left as it is."""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest

import oracle
import ssd_synth as syn
from oracle import quadratic

from test_oracle_pins import _case_arrays, _cases

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

WRITE = ("        /* write: h = exp(dt A) h + dt B x^T */\n"
         "        for (int64_t i = 0; i < n; ++i) {\n"
         "            const double wb = d * ld(J->B, (row * g + gi) * n + i, J->io);\n"
         "            double *Hi = H + i * p;\n"
         "            for (int64_t j = 0; j < p; ++j)\n"
         "                Hi[j] = decay * Hi[j] + wb * xv[j];\n"
         "        }\n")
READ_START = "        /* read: y = C^T h + D x */\n"
READ_END = "                yt[j] += ci * Hi[j];\n        }\n"


def _read_before_write(src):
    """Move the read block in front of the write block."""
    assert WRITE in src and READ_START in src
    a = src.index(READ_START)
    b = src.index(READ_END, a) + len(READ_END)
    read = src[a:b]
    src = src[:a] + src[b:]
    return src.replace(WRITE, read + WRITE)


MUTANTS = {
    "decay_sign": lambda s: s.replace("const double decay = exp(Ah * d);",
                                      "const double decay = exp(-Ah * d);"),
    "decay_without_dt": lambda s: s.replace("const double decay = exp(Ah * d);",
                                            "const double decay = exp(Ah);"),
    "write_without_dt": lambda s: s.replace("const double wb = d * ld(J->B,",
                                            "const double wb = ld(J->B,"),
    "dropped_skip": lambda s: s.replace("yt[j] = Dh * xv[j];", "yt[j] = 0.0;"),
    "B_for_C": lambda s: s.replace("const double ci = ld(J->C,", "const double ci = ld(J->B,"),
    "group_index": lambda s: s.replace("const int64_t gi = hh / (h / g);",
                                       "const int64_t gi = hh % g;"),
    "read_before_write": _read_before_write,
    "softplus_sign": lambda s: s.replace("return fmax(z, 0.0) + log1p(exp(-fabs(z)));",
                                         "return fmax(z, 0.0) - log1p(exp(-fabs(z)));"),
}


def _build_mutant(name, tmp_path):
    src = open(SRC).read()
    mutated = MUTANTS[name](src)
    assert mutated != src, "mutation %s did not apply" % name
    c = tmp_path / ("%s.c" % name)
    so = tmp_path / ("%s.so" % name)
    c.write_text(mutated)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", "-D_GNU_SOURCE",
                           "-o", str(so), str(c), "-lm", "-lpthread"])
    return oracle._bind(ctypes.CDLL(str(so)))


def _pins_pass():
    """Run the independent pins against whatever oracle library is loaded;
    True if every one of them holds."""
    for case in _cases():
        a = _case_arrays(case)
        y, fin = oracle.scan(**a, io="f32")
        if not (np.allclose(y.reshape(-1), case["y"], rtol=1e-12, atol=1e-15)
                and np.allclose(fin.reshape(-1), case["final"], rtol=1e-12, atol=1e-15)):
            return False
    inp = syn.random_case(11, 2, 37, 4, 5, 6, 2, io="f32", init_std=0.3)
    kw = dict(x=inp["x"], dt=inp["dt"], A=inp["A"], B=inp["B"], C=inp["C"], D=inp["D"],
              dt_bias=inp["dt_bias"], init_state=inp["init_state"], io="f32")
    y, fin = oracle.scan(**kw)
    yq, fq = quadratic.dual_form(**kw)
    scale = max(np.abs(yq).max(), 1e-300)
    if np.abs(y - yq).max() > 1e-12 * scale:
        return False
    if np.abs(fin - fq).max() > 1e-12 * max(np.abs(fq).max(), 1e-300):
        return False
    return True


def test_pins_accept_the_real_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_planted_mistake(name, tmp_path):
    lib = _build_mutant(name, tmp_path)
    saved = oracle._lib
    oracle._lib = lib
    try:
        assert not _pins_pass(), "planted mistake %s went undetected" % name
    finally:
        oracle._lib = saved
