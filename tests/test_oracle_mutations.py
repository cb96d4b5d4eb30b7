"""The n-gram oracle's pins catch plausible mistakes: each case plants one
mistake in a copy of oracle/ngram_oracle.c (a one-line substitution), builds
that copy, and runs the pins it should trip against it in a subprocess (the
oracle module loads the copy through NGRAM_ORACLE_LIB).  The committed oracle
itself holds no mistake; the regular pins check it as it is."""
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "ngram_oracle.c")

MUTATIONS = [
    ("seed added instead of xored", "(key ^ seed) + UINT64_C(0x9E3779B97F4A7C15)",
     "(key + seed) + UINT64_C(0x9E3779B97F4A7C15)", ["test_oracle_hash.py"]),
    ("first shift of the finaliser", "z = (z ^ (z >> 30))", "z = (z ^ (z >> 31))", ["test_oracle_hash.py"]),
    ("sign from bit 1", "neg_b[i] = (uint8_t)(zb & 1u);", "neg_b[i] = (uint8_t)((zb >> 1) & 1u);",
     ["test_oracle_hash.py"]),
    ("trigram context crosses an EoS", "p2[i] = (i >= 2 && !opens_doc && tok[i - 1] != eos)",
     "p2[i] = (i >= 2 && !opens_doc)", ["test_oracle_hash.py"]),
    ("trigram key order", "*kt = ((uint64_t)p2 * B + (uint64_t)p1) * B + tt;",
     "*kt = ((uint64_t)p1 * B + (uint64_t)p2) * B + tt;", ["test_oracle_hash.py"]),
    ("trigram sign ignored in the forward", "            if (neg_t[i])\n                b = -b;\n", "",
     ["test_oracle_forward.py"]),
    ("sign ignored in the window gradient", "double s = neg[e[k].pos] ? -1.0 : 1.0;", "double s = 1.0;",
     ["test_oracle_grad.py"]),
    ("eps inside the root", "sqrt((double)v32) + (double)eps", "sqrt((double)v32 + (double)eps)",
     ["test_oracle_step.py"]),
    ("missing (1 - beta2)", "+ (1.0 - (double)beta2) * m;", "+ m;", ["test_oracle_step.py"]),
    ("decay exponent off by one", "return pow(beta2, (double)k);", "return pow(beta2, (double)(k + 1));",
     ["test_oracle_step.py"]),
    ("sum instead of mean of G^2", "        m /= (double)dim;\n", "", ["test_oracle_step.py"]),
    ("bf16 by truncation", "double r = nearbyint(ldexp(x, -q));", "double r = trunc(ldexp(x, -q));",
     ["test_oracle_forward.py"]),
    ("t_last not updated", "        t_last[u] = t;\n", "", ["test_oracle_step.py"]),
]


@pytest.mark.parametrize("desc,old,new,files", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_a_planted_mistake_fails_a_pin(tmp_path, desc, old, new, files):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found: {desc}"
    mut = tmp_path / "ngram_oracle.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "libngram_oracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", str(mut), "-o", str(so),
                           "-lm"], stderr=subprocess.DEVNULL)
    env = dict(os.environ, NGRAM_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                        *[os.path.join(HERE, f) for f in files]],
                       env=env, capture_output=True, text=True, timeout=600, cwd=os.path.dirname(HERE))
    assert r.returncode == 1, f"{desc} went unnoticed:\n{r.stdout[-2000:]}"
