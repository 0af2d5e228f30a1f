"""Each planted mistake in the oracle must fail at least one oracle pin.

The mistakes are the plausible ones: a wrong sign, a dropped term, a wrong
index or stride, a wrong decoder constant, a node range read one past its
end.  Mistakes in oracle.c are planted in temporary copies of the source,
compiled with gcc; mistakes in the Python side (which keys a generated step's
sequence attends) are planted in a rewritten copy of that function swapped in
for the duration of the test.  Everything runs on the CPU.
"""
import inspect
import os
import textwrap

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

MUTANTS = {
    "lse_sign": ("*lse = m + log(l);", "*lse = m - log(l);"),
    "lse_drop_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "no_normalise": ("o[c] = acc[c] / l;", "o[c] = acc[c];"),
    "no_scale": ("sc[j++] = scale * dot;", "sc[j++] = dot;"),
    "gqa_index": ("g = h / (p->Hq / p->Hkv);", "g = h % p->Hkv;"),
    "v_head_stride": ("acc[c] += e * elem(sg->v, base + c, p->dtype);",
                      "acc[c] += e * elem(sg->v, t * sg->stride_tok + c, p->dtype);"),
    "k_transposed": ("dot += qd[c] * elem(sg->k, base + c, p->dtype);",
                     "dot += qd[c] * elem(sg->k, t * sg->stride_tok + c * sg->stride_head + g, p->dtype);"),
    "no_max_shift": ("const double e = exp(sc[j++] - m);", "const double e = exp(sc[j++]);"),
    "f16_subnormal": ("v = ldexp((double)m, -24);", "v = ldexp((double)m, -25);"),
    "f16_bias": ("v = ldexp((double)(m | 0x400), e - 25);", "v = ldexp((double)(m | 0x400), e - 24);"),
    "bf16_shift": ("uint32_t w = (uint32_t)h << 16;", "uint32_t w = (uint32_t)h << 15;"),
    "merge_lse_drop": ("cur_lse = mx + log(w1 + w2);", "cur_lse = mx;"),
    "merge_weight_swap": ("cur_o[c] = (w1 * cur_o[c] + w2 * o2[c]) / (w1 + w2);",
                          "cur_o[c] = (w2 * cur_o[c] + w1 * o2[c]) / (w1 + w2);"),
    "rows_ignored": ("const int64_t r = p->rows ? p->rows[i] : i;", "const int64_t r = i;"),
    "max_skips_first": ("for (j = 0; j < n; j++)\n        if (sc[j] > m) m = sc[j];",
                        "for (j = 1; j < n; j++)\n        if (sc[j] > m) m = sc[j];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for {name} not found exactly once"
    src = tmp_path / f"oracle_{name}.c"
    src.write_text(text.replace(old, new))
    lib = oracle.load(oracle.compile_source(str(src), str(tmp_path / f"lib_{name}.so")))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"mutant {name} passed every pin"


# Mistakes in oracle.step_segments: which prefix nodes a sequence attends.
PY_MUTANTS = {
    "node_end_inclusive": ("node.seq_begin <= b < node.seq_end",
                           "node.seq_begin <= b <= node.seq_end"),
    "node_begin_exclusive": ("node.seq_begin <= b < node.seq_end",
                             "node.seq_begin < b < node.seq_end"),
    "first_level_only": ("for li, level in enumerate(step.levels):",
                         "for li, level in enumerate(step.levels[:1]):"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_python_mutant_is_caught(name, monkeypatch):
    old, new = PY_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.step_segments))
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), ns)
    monkeypatch.setattr(oracle, "step_segments", ns["step_segments"])
    lib = oracle._get()
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, FloatingPointError) as e:
            caught.append((pin.__name__, str(e)[:80]))
    assert caught, f"mutant {name} passed every pin"
