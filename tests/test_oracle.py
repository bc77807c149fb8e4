"""The CPU oracle against its pins, and the pins against planted mistakes."""
import os
import re
import subprocess
import sys

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.load_library())


# Each mutant plants one plausible mistake in a copy of the oracle source; at least
# one pin must reject every mutant, so the battery above is not vacuous.
MUTANTS = {
    "no_decay": ("const double a = (j == 0) ? exp(g[t * Hv + h]) : 1.0;",
                 "const double a = 1.0;"),
    "delta_sign": ("S[i * K + j] - beta * Sk[i] * k[j]", "S[i * K + j] + beta * Sk[i] * k[j]"),
    "decay_after_write": ("a * (S[i * K + j] - beta * Sk[i] * k[j]) + beta * v[i] * k[j]",
                          "a * (S[i * K + j] - beta * Sk[i] * k[j] + beta * v[i] * k[j])"),
    "no_beta_on_write": ("+ beta * v[i] * k[j]", "+ v[i] * k[j]"),
    "transposed_readout": ("acc += S[i * K + j] * q[j]", "acc += S[j * K + i] * q[j]"),
    "state_layout_transposed": ("S[j * K + i] = src[i * V + j]", "S[i * K + j] = src[i * V + j]"),
    "decay_every_substep": ("(j == 0) ? exp(g[t * Hv + h]) : 1.0", "exp(g[t * Hv + h])"),
    "head_group_mapping": ("hk = h / group", "hk = h % Hk"),
    "no_scale": ("o[i] = scale * acc", "o[i] = acc"),
    "q_not_normalised": ("maybe_l2norm(q + (t * Hk + hk) * K, K, use_qk_l2norm, qn)",
                         "maybe_l2norm(q + (t * Hk + hk) * K, K, 0, qn)"),
    "prefill_padding_writes": ("if (state_indices[n] < 0) continue; /* padding writes nothing */",
                               "if (state_indices[n] < 0) { store_state(states + p * SS, K, V, final_state + h * SS); continue; }"),
    "decode_padding_writes": ("if (slot < 0) continue; /* padding writes nothing */",
                              "if (slot < 0) { store_state(states + p * SS, K, V, cache + h * SS); continue; }"),
    "l2norm_eps_outside_sqrt": ("1.0 / sqrt(ss + 1e-6)", "1.0 / (sqrt(ss) + 1e-6)"),
    "l2norm_no_eps": ("1.0 / sqrt(ss + 1e-6)", "1.0 / sqrt(ss)"),
    "no_sequence_reset": ("double *S = states + p * SS;\n    double *buf",
                          "double *S = states + (p % Hv) * SS;\n    double *buf"),
}

_RUN_PINS = r"""
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle
from oracle_pins import ALL_PINS
lib = oracle.load_library({lib!r})
failed = []
for pin in ALL_PINS:
    try:
        pin(lib)
    except AssertionError as e:
        failed.append(pin.__name__)
print("FAILED:" + ",".join(failed))
"""


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mutated = tmp_path / "gdr_oracle_mutant.c"
    mutated.write_text(src.replace(old, new, 1))
    lib = str(tmp_path / "libmutant.so")
    # build with -Wno-error: some mutants leave variables unused
    oracle.build(out_path=lib, src=str(mutated), extra_flags=("-Wno-error",))
    root = os.path.dirname(os.path.dirname(os.path.abspath(oracle.__file__)))
    code = _RUN_PINS.format(root=root, tests=os.path.dirname(__file__), lib=lib)
    # a separate process: a broken oracle must not take the test run down with it
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         timeout=300)
    m = re.search(r"FAILED:(.*)", res.stdout)
    failed = [x for x in (m.group(1).split(",") if m else []) if x]
    assert res.returncode != 0 or failed, f"mutant {name} passed every pin"
