"""Plant plausible mistakes in a copy of the oracle's C source, rebuild it on
the CPU, and check that the pins catch every one of them (CPU only).

This shows the pins are sharp enough: a dropped term, a wrong sign or index,
a transposed operand or an off-by-one mask in the oracle fails at least one
of them. The real oracle is never modified."""
import os
import subprocess

import pytest

import oracle
from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# (id, text in oracle.c, replacement)
MUTATIONS = [
    ("alpha_sign", "exp(m[ri] - m_new)", "exp(m_new - m[ri])"),
    ("alpha_dropped_on_numerator", "acc[ri * d + c] *= alpha;", ";"),
    ("alpha_dropped_on_denominator", "l[ri] = alpha * l[ri] + psum;", "l[ri] = l[ri] + psum;"),
    ("tile_scale_dropped", "*s = scale * dot;", "*s = dot;"),
    ("tile_max_not_running", "const double m_new = (tmax > m[ri]) ? tmax : m[ri];",
     "const double m_new = (tmax != -INFINITY) ? tmax : m[ri];"),
    ("dense_wrong_operand", "s += qi[c] * k[j * d + c];", "s += qi[c] * v[j * d + c];"),
    ("dense_denominator_unshifted", "if (z[j] != -INFINITY) l += exp(z[j] - m);",
     "if (z[j] != -INFINITY) l += exp(z[j]);"),
    ("lse_drops_max", "if (lse_out) *lse_out = m + log(l);", "if (lse_out) *lse_out = log(l);"),
    ("causal_off_by_one", "if (mask == OR_MASK_CAUSAL) return j <= i;",
     "if (mask == OR_MASK_CAUSAL) return j < i + 1 && j != i;"),
    ("band_asymmetric", "(j - i <= window)", "(j - i <= window + 1)"),
    ("bwd_ds_sign", "dS[i * N + j] = Pi[j] * (dp - Di);", "dS[i * N + j] = Pi[j] * (dp + Di);"),
    ("bwd_dk_scale_dropped", "dk[off + j * d + c] = scale * skj[c];",
     "dk[off + j * d + c] = skj[c];"),
    ("bwd_dv_transposed", "const double p_ij = P[i * N + j];", "const double p_ij = P[j * N + i];"),
    ("bwd_dq_wrong_operand", "acc[c] += ds_ij * K[j * d + c];", "acc[c] += ds_ij * V[j * d + c];"),
    ("bwd_o_wrong_operand", "Oi[c] += p * V[j * d + c];", "Oi[c] += p * K[j * d + c];"),
]


@pytest.mark.parametrize("mid,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(tmp_path, mid, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {mid} not unique/present"
    mutated = tmp_path / f"oracle_{mid}.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / f"liboracle_{mid}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", str(mutated), "-o", str(lib),
                    "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught planted mistake {mid}"
