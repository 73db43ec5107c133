"""The oracle's pins are sharp: a plausible mistake planted in a temporary copy of
the oracle source (a dropped term, a wrong sign, a transposed index, a gate
applied at the wrong point) makes at least one pin fail.  Mistakes are planted
only on the CPU, in a scratch build; the real oracle is untouched."""
import os

import pytest

import oracle
import tests.test_oracle_pins as pins
import tests.test_chunked_ref as chunked

# (name, text in gdr_ref.c, replacement)
MUTATIONS = [
    ("forget_gate_dropped",
     "    /* forget gate */\n    for (i = 0; i < dk; ++i) {",
     "    /* forget gate */\n    for (i = 0; i < dk && 0; ++i) {"),
    ("transposed_state_in_prediction",
     "                s += S[(size_t)i * dv + j] * k[i];\n            pred[j] = s;",
     "                s += S[(size_t)(i % dv) * dv + (j % dk)] * k[i] * (i < dv && j < dk);\n            pred[j] = s;"),
    ("dropped_prediction_term",
     "S[(size_t)i * dv + j] += b * kw[i] * (v[j] - pred[j]);",
     "S[(size_t)i * dv + j] += b * kw[i] * (v[j]);"),
    ("wrong_sign_in_write",
     "S[(size_t)i * dv + j] += b * kw[i] * (v[j] - pred[j]);",
     "S[(size_t)i * dv + j] -= b * kw[i] * (v[j] - pred[j]);"),
    ("erase_with_write_key",
     "                s += S[(size_t)i * dv + j] * k[i];\n            pred[j] = s;",
     "                s += S[(size_t)i * dv + j] * kw[i];\n            pred[j] = s;"),
    ("beta_not_square_rooted",
     "            kt[i] = sqrt(bk[i]) * k[i];",
     "            kt[i] = bk[i] * k[i];"),
    ("beta_v_ignored",
     "            vt[j] = sqrt(bvv[j]) * v[j];",
     "            vt[j] = sqrt(bk[j % dk]) * v[j];"),
    ("readout_before_write",
     "            ref_readout(dk, dv, S, q + tok * dk, o + tok * dv);",
     "            ;"),
    ("channel_gate_index_by_value_dim",
     "        const double ai = channel_alpha ? a[i] : a[0];\n        for (j = 0; j < dv; ++j)\n            S[(size_t)i * dv + j] *= ai;",
     "        for (j = 0; j < dv; ++j)\n            S[(size_t)i * dv + j] *= channel_alpha ? a[j % dk] : a[0];"),
    ("readout_transposed",
     "            s += S[(size_t)i * dv + j] * q[i];\n        o[j] = s;",
     "            s += S[(size_t)(j % dk) * dv + (i % dv)] * q[i];\n        o[j] = s;"),
]


def _all_pins():
    """Run every pin; return the names of those that failed."""
    import glob
    import inspect

    failed = []
    for name, fn in list(inspect.getmembers(pins, inspect.isfunction)) + \
            list(inspect.getmembers(chunked, inspect.isfunction)):
        if not name.startswith("test_"):
            continue
        params = getattr(fn, "pytestmark", [])
        cases = [{}]
        for mark in params:
            if mark.name == "parametrize":
                argnames = [a.strip() for a in mark.args[0].split(",")]
                new = []
                for c in cases:
                    for val in mark.args[1]:
                        vals = val if len(argnames) > 1 else (val,)
                        d = dict(c)
                        d.update(zip(argnames, vals))
                        new.append(d)
                cases = new
        for c in cases:
            try:
                fn(**c)
            except Exception:  # assertion or rejected arguments
                failed.append(name)
                break
    return failed


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = oracle.source()
    assert old in src, f"mutation {name} no longer applies"
    mutated = src.replace(old, new, 1)
    if name == "readout_before_write":
        # ... and read out before the step instead
        mutated = mutated.replace(
            "            ref_step(dk, dv, S, alpha + tok * a_n,",
            "            ref_readout(dk, dv, S, q + tok * dk, o + tok * dv);\n            ref_step(dk, dv, S, alpha + tok * a_n,", 1)
    lib = oracle.build_variant(mutated, str(tmp_path / f"libmut_{name}.so"))
    with oracle.use_library(lib):
        failed = _all_pins()
    assert failed, f"no pin caught the planted mistake {name}"
