"""The conv1d + SiLU oracle against its pins, and the pins against planted mistakes."""
import importlib.util
import os
import tempfile

import pytest

import conv_pins
from oracle import conv_oracle

SRC = conv_oracle.__file__


@pytest.mark.parametrize("pin", conv_pins.ALL_PINS, ids=[p.__name__ for p in conv_pins.ALL_PINS])
def test_conv_oracle_pin(pin):
    pin(conv_oracle)


# (name, text in the oracle, replacement)
MUTANTS = [
    ("tap_reversed", "shift = W - 1 - i  # tap i", "shift = i  # tap i"),
    ("bias_dropped", "        pre += np.asarray(bias, dtype=np.float64)", "        pass"),
    ("crosses_documents", "            if shift < L:\n                pre[s + shift:e] += w[:, i] * xs[:L - shift]",
     "            lo = max(0, s - shift)\n            pre[lo + shift:e] += w[:, i] * x[lo:e - shift]"),
    ("silu_derivative_missing_term", "dpre = dy * s * (1.0 + pre * (1.0 - s))", "dpre = dy * s"),
    ("dx_wrong_direction", "dx[s0:e - shift] += w[:, i] * ds[shift:]", "dx[s0 + shift:e] += w[:, i] * ds[:L - shift]"),
    ("dweight_unshifted", "dw[:, i] += np.sum(ds[shift:] * xs[:L - shift], axis=0)",
     "dw[:, i] += np.sum(ds * xs, axis=0)"),
    ("dbias_from_dy", "return dict(dx=dx, dweight=dw, dbias=dpre.sum(axis=0))",
     "return dict(dx=dx, dweight=dw, dbias=dy.sum(axis=0))"),
]


def _load(path):
    spec = importlib.util.spec_from_file_location("conv_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,find,repl", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_conv_pins_catch_mutant(name, find, repl):
    src = open(SRC).read()
    assert src.count(find) == 1, "mutation anchor not found: %r" % find
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "conv_mutant.py")
        with open(path, "w") as f:
            f.write(src.replace(find, repl))
        mod = _load(path)
        caught = []
        for pin in conv_pins.ALL_PINS:
            try:
                pin(mod)
            except (AssertionError, ValueError, IndexError):
                caught.append(pin.__name__)
        assert caught, "no pin catches the planted mistake %s" % name
