"""Plant plausible mistakes in copies of the oracle's C source (on the CPU)
and check that the pin battery catches every one of them. This shows the pins
constrain each part of the oracle: a dropped term, a wrong sign, a transposed
operand, a wrong window or a wrong membership test all fail some pin."""
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "na_oracle.c")

MUTATIONS = {
    "softmax_grad_sign_dq": ("double dS = w[j] * (dP - delta);", "double dS = w[j] * (dP + delta);", 0),
    "softmax_grad_sign_dk": ("double dS = w[j] * (dP - delta);", "double dS = w[j] * (dP + delta);", 1),
    "dq_drops_scale": ("g[c] += p->scale * dS * ky[c];", "g[c] += dS * ky[c];", 0),
    "dk_wrong_operand": ("gk[c] += p->scale * dS * qx[c];", "gk[c] += p->scale * dS * dox[c];", 0),
    "dv_drops_weight": ("gv[c] += w[j] * dox[c];", "gv[c] += dox[c];", 0),
    "lse_drops_max": ("double lse = m + log(sum);", "double lse = log(sum);", 0),
    "no_high_border_shift": ("if (s + k > n) s = n - k;", "", 0),
    "off_center_even": ("int64_t s = i - k / 2;", "int64_t s = i - (k - 1) / 2;", 0),
    "ignores_residue": ("int64_t r = x % d;", "int64_t r = 0;", 0),
    "short_membership_reach": ("reach[a] = (p->kernel[a] - 1) * p->dilation[a];",
                               "reach[a] = (p->kernel[a] / 2) * p->dilation[a];", 0),
    "delta_dropped": ("return dot(vec(p, dout, b, tok, h), o, p->head_dim);", "return 0.0;", 0),
    "scores_unscaled": ("w[j] = p->scale * dot(qv, vec(p, k, b, keys[j], h), D);",
                        "w[j] = dot(qv, vec(p, k, b, keys[j], h), D);", 0),
    "values_from_keys": ("const double *vv = vec(p, v, b, keys[j], h);",
                         "const double *vv = vec(p, k, b, keys[j], h);", 0),
    "qk_drops_alpha": ("attn[s * K + j] = alpha * dot(", "attn[s * K + j] = dot(", 0),
    "qk_wrong_operand": ("dot(ax, vec(p, b, bb, keys[j], h), D)", "dot(ax, vec(p, a, bb, keys[j], h), D)", 0),
    "av_transposed_index": ("o[c] += attn[u * K + j] * bv[c];", "o[c] += attn[j * K + u] * bv[c];", 0),
    "av_drops_alpha": ("o[c] *= alpha;", "o[c] *= 1.0;", 0),
    "inverse_drops_alpha": ("o[c] *= alpha;", "o[c] *= 1.0;", 1),
    "inverse_wrong_operand": ("const double *ax = vec(p, a, bb, xtok, h);",
                              "const double *ax = vec(p, a, bb, tok, h);", 0),
    "inverse_own_row": ("o[c] += attn[xu * K + j] * ax[c];",
                        "o[c] += attn[((bb * tokens(p) + tok) * p->heads + h) * K + j] * ax[c];", 0),
    "inverse_short_reach": ("lo[ax] = ctr[ax] - (p->kernel[ax] - 1) * p->dilation[ax];",
                            "lo[ax] = ctr[ax] - (p->kernel[ax] / 2) * p->dilation[ax];", 0),
    "rpb_offset_sign": ("int64_t delta = (yc[a] - xc[a]) / p->dilation[a];",
                        "int64_t delta = (xc[a] - yc[a]) / p->dilation[a];", 0),
    "rpb_ignores_dilation": ("int64_t delta = (yc[a] - xc[a]) / p->dilation[a];",
                             "int64_t delta = (yc[a] - xc[a]);", 0),
    "rpb_off_center": ("idx = idx * (2 * p->kernel[a] - 1) + delta + p->kernel[a] - 1;",
                       "idx = idx * (2 * p->kernel[a] - 1) + delta + p->kernel[a] / 2;", 0),
    "rpb_grad_wrong_head": ("drpb[h * R + rpb_index(p, tok, keys[j])] += dattn[u * K + j];",
                            "drpb[rpb_index(p, tok, keys[j])] += dattn[u * K + j];", 0),
}


def _mutate(text, old, new, nth):
    pos = -1
    for _ in range(nth + 1):
        pos = text.index(old, pos + 1)
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new, nth = MUTATIONS[name]
    text = open(SRC).read()
    assert text.count(old) > nth, f"mutation anchor missing: {old!r}"
    src = tmp_path / "mutant.c"
    src.write_text(_mutate(text, old, new, nth))
    lib = oracle.build(str(src), str(tmp_path / "libmutant.so"))
    # A mutant may read out of bounds, so its battery runs in a child process;
    # a crash there also counts as caught.
    here = os.path.dirname(os.path.abspath(__file__))
    code = ("import sys; sys.path[:0] = [%r, %r]; import oracle, oracle_pins as P; "
            "print(','.join(P.failing_checks(oracle.Bound(%r), first_only=True)))"
            % (here, os.path.dirname(here), lib))
    # the battery's problems are tiny: one OpenMP thread avoids waking a team
    # for each of the finite-difference evaluations
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300,
                       env=env)
    caught = r.returncode != 0 or r.stdout.strip() != ""
    assert caught, f"no pin catches the planted mistake {name}"
