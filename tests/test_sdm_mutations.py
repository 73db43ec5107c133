"""The Sparse Delta Memory oracle's pins are sharp: a plausible mistake planted in a
copy of oracle/sdm.py (the slot weight dropped, the softmax taken over every slot,
the read weights reused for the write, the gate applied after the delta, the read
taken before the write) makes at least one pin in tests/test_sdm_oracle.py fail.
Mistakes are planted on the CPU, in a module built from the mutated text; the real
oracle is untouched."""
import importlib.util
import inspect
import os

import pytest

import tests.test_sdm_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "sdm.py")

# (name, text in oracle/sdm.py, replacement)
MUTATIONS = [
    ("slot_weight_dropped",
     "Mh[i] = mt + be * w * (v[b, t, h] - mt)",
     "Mh[i] = mt + be * (v[b, t, h] - mt)"),
    ("softmax_over_all_slots",
     "wk = softmax(sc)",
     "wk = softmax((ks[b, t, h, 0][:, None] + ks[b, t, h, 1][None, :]).reshape(-1).astype(np.float32))[slots]"),
    ("read_weights_used_for_the_write",
     "wk = softmax(sc)",
     "wk = softmax(select(qs[b, t, h, 0], qs[b, t, h, 1], W)[1])"),
    ("gate_after_the_delta",
     "Mh[i] = mt + be * w * (v[b, t, h] - mt)",
     "Mh[i] = a * (Mh[i] + be * w * (v[b, t, h] - Mh[i]))"),
    ("read_before_the_write",
     "                rs, rsc = select(qs[b, t, h, 0], qs[b, t, h, 1], R)\n"
     "                o[b, t, h] = softmax(rsc) @ Mh[rs]\n",
     "                rs, rsc = select(qs[b, t, h, 0], qs[b, t, h, 1], R)\n"
     "                o[b, t, h] = softmax(rsc) @ M0h[rs]\n"),
    ("read_weights_uniform",
     "o[b, t, h] = softmax(rsc) @ Mh[rs]",
     "o[b, t, h] = Mh[rs].mean(axis=0)"),
]


def _mutated_module(text, name):
    spec = importlib.util.spec_from_loader(f"sdm_mut_{name}", loader=None)
    mod = importlib.util.module_from_spec(spec)
    exec(compile(text, f"<mutated sdm {name}>", "exec"), mod.__dict__)
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


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, monkeypatch):
    with open(SRC) as f:
        src = f.read()
    assert old in src, f"mutation {name} no longer applies"
    text = src.replace(old, new, 1)
    if name == "read_before_the_write":
        # keep a copy of the table as it was before the token's write
        text = text.replace("                slots, sc = select(ks[b, t, h, 0], ks[b, t, h, 1], W)\n",
                            "                M0h = Mh.copy()\n"
                            "                slots, sc = select(ks[b, t, h, 0], ks[b, t, h, 1], W)\n", 1)
    monkeypatch.setattr(pins, "sdm", _mutated_module(text, name))
    assert _failing_pins(), f"no pin caught the planted mistake {name}"


def test_unmutated_oracle_passes_every_pin():
    assert _failing_pins() == []
