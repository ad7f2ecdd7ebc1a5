"""The oracle's pins must fail when a plausible mistake is planted in it.

Each case copies the oracle source, applies one textual mutation (a dropped
fusion term, swapped sources, a wrong GQA index, a transposed weight index, a
wrong scale, an off-by-one causal mask, log base 2 instead of natural log),
builds it on the CPU into a temporary directory, and runs the pin tests
against that build in a subprocess.  The mistakes live only in the temporary
copy; the committed oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fkv_oracle.c")

MUTATIONS = {
    "drop_second_source": ("return (double)w1[(int64_t)g * D + d] * x1 + (double)wn[(int64_t)g * D + d] * xn;",
                           "return (double)w1[(int64_t)g * D + d] * x1;"),
    "swap_source_weights": ("return (double)w1[(int64_t)g * D + d] * x1 + (double)wn[(int64_t)g * D + d] * xn;",
                            "return (double)wn[(int64_t)g * D + d] * x1 + (double)w1[(int64_t)g * D + d] * xn;"),
    "gqa_modulo_index": ("const int g = h / G;", "const int g = h % Hkv;"),
    "transposed_weight": ("return (double)w1[(int64_t)g * D + d] * x1 + (double)wn[(int64_t)g * D + d] * xn;",
                          "return (double)w1[(int64_t)d * Hkv_ + g] * x1 + (double)wn[(int64_t)d * Hkv_ + g] * xn;"),
    "sign_flip_second_term": ("* x1 + (double)wn", "* x1 - (double)wn"),
    "causal_off_by_one": ("last = p + (len - Sq);", "last = p + (len - Sq) - 1;"),
    "lse_log2": ("lse[i] = m + log(l);", "lse[i] = m + log2(l);"),
    "scale_dropped": ("s[t] = shape->scale * dot;", "s[t] = dot;"),
    "value_from_key": ("acc[d] += e * reconstructed(&v1, &vn, vw1, vwn,", "acc[d] += e * reconstructed(&k1, &kn, vw1, vwn,"),
}


def _mutate(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC, encoding="utf-8").read()
    assert src.count(old) >= 1, name
    src = src.replace(old, new)
    if name == "transposed_weight":   # needs the KV-head count in scope
        src = src.replace("static double reconstructed(", "static int Hkv_ = 1;\nstatic double reconstructed(")
        src = src.replace("const int G = Hq / Hkv;", "const int G = Hq / Hkv;\n    Hkv_ = Hkv;")
    path = tmp_path / ("fkv_oracle_%s.c" % name)
    path.write_text(src, encoding="utf-8")
    return str(path)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    sys.path.insert(0, ROOT)
    from oracle import oracle as orc_mod
    so = orc_mod.build_from(_mutate(name, tmp_path), str(tmp_path / "liboracle_mut.so"))
    env = dict(os.environ, FKV_ORACLE_SO=so, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_rope_and_counts.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "pins did not catch mutation %s:\n%s" % (name, r.stdout[-2000:])
