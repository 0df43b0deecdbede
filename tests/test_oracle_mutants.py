"""Planted mistakes in the oracle must each fail at least one pin.

Every mutant is a copy of oracle/pod_oracle.c with one textual change,
compiled with gcc into a temporary library and run against all pins in a
child process (a mutant that crashes counts as caught).  The real oracle is
never modified.
"""
import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    "mask_off_by_one": ("!(j <= limit)", "!(j < limit)"),
    "decode_context_plus_one": ("int64_t L = context_lens[req];", "int64_t L = context_lens[req] + 1;"),
    "gqa_interleaved_decode": ("int h = g * G + hh;", "int h = hh * hkv + g;"),
    "gqa_interleaved_prefill": ("int h = g * G + (int)(w % G);", "int h = (int)(w % G) * hkv + g;"),
    "slot_reversed": ("int64_t slot = j % page_size;", "int64_t slot = page_size - 1 - j % page_size;"),
    "scale_dropped": ("s *= scale;", ""),
    "no_max_shift": ("double e = exp(scores[j] - m);", "double e = exp(scores[j]);"),
    "count_not_weight": ("l += e;", "l += 1.0;"),
    "value_row_reversed": ("out[k] += e * V[j * d + k];", "out[k] += e * V[(n_keys - 1 - j) * d + k];"),
    "key_elem_reversed": ("s += q[k] * K[j * d + k];", "s += q[k] * K[j * d + (d - 1 - k)];"),
    "q_row_head_swapped": ("qd[k] = elem(q, dtype, ((size_t)row * hq + h) * d + k);",
                           "qd[k] = elem(q, dtype, ((size_t)h * chunk_len + row) * d + k);"),
    "bf16_upcast_shift": ("<< 16;", "<< 15;"),
    "normalise_dropped": ("out[k] /= l;", ""),
}

RUNNER = textwrap.dedent("""
    import sys
    sys.path[:0] = [{root!r}, {tests!r}]
    import oracle, oracle_pins
    lib = oracle.load({lib!r})
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except Exception as e:
            failed.append(pin.__name__)
    print("FAILED_PINS", failed)
    sys.exit(1 if failed else 0)
""")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "pod_oracle.c")).read()
    assert src.count(old) >= 1, f"mutation anchor for {name} missing"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    oracle.build(str(mutated), str(lib))
    code = RUNNER.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=str(lib))
    env = dict(os.environ, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode != 0, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr}"
