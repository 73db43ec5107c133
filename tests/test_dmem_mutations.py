"""The delta-mem oracle's pins are sharp: a plausible mistake planted in a copy of
oracle/dmem.py makes at least one pin in tests/test_dmem_oracle.py fail.  Mistakes
are planted on the CPU, in a module built from the mutated text; the real oracle is
untouched."""
import importlib.util
import inspect
import os

import pytest

import tests.test_dmem_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "dmem.py")

# (name, [(text in oracle/dmem.py, replacement), ...])
MUTATIONS = [
    ("segment_sum_not_mean",
     [("kb = ks / n\n", "kb = ks\n"), ("vb = vs / n\n", "vb = vs\n")]),
    ("read_after_the_write",
     [("                reads[b, t, h] = Mh @ q[b, t, h]          # before this token's segment is written\n", ""),
      ("                    n = 0\n            M[b, h] = Mh\n",
       "                    n = 0\n                reads[b, t, h] = Mh @ q[b, t, h]\n            M[b, h] = Mh\n")]),
    ("sub_state_reads_averaged",
     [(".sum(axis=3)", ".mean(axis=3)")]),
    ("gates_of_the_first_token_of_the_segment",
     [("lam[b, t, h], beta[b, t, h])", "lam[b, t - n + 1, h], beta[b, t - n + 1, h])")]),
    ("prediction_from_the_decayed_memory",
     [("lam * M + beta * np.outer(v - M @ k, k)", "lam * M + beta * np.outer(v - lam * M @ k, k)")]),
    ("outer_product_transposed",
     [("lam * M + beta * np.outer(v - M @ k, k)", "lam * M + beta * np.outer(k, v - M @ k)")]),
    ("last_token_does_not_close",
     [(" or t == T - 1", "")]),
    ("segment_sums_not_reset",
     [("                    ks = np.zeros(r)\n                    vs = np.zeros(r)\n                    n = 0\n",
       "                    n = 0\n")]),
]


def _mutated_module(text, name):
    spec = importlib.util.spec_from_loader(f"dmem_mut_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text, f"<mutated dmem {name}>", "exec"), mod.__dict__)
    return mod


def _failing_pins():
    failed = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        cases = [{}]
        for mark in getattr(fn, "pytestmark", []):
            if mark.name == "parametrize":
                cases = [{mark.args[0]: v} for v in mark.args[1]]
        for c in cases:
            try:
                fn(**c)
            except Exception:
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("name,edits", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, edits, monkeypatch):
    with open(SRC) as f:
        text = f.read()
    for old, new in edits:
        assert old in text, f"mutation {name} no longer applies"
        text = text.replace(old, new, 1)
    monkeypatch.setattr(pins, "dmem", _mutated_module(text, name))
    assert _failing_pins(), f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []
