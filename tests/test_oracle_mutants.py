"""Plant mistakes in copies of the oracle and check that the pins catch each one.

Every mutation is a plausible slip (a dropped term, a wrong sign or index, a
transposed operand, a forgotten rescale) and keeps all memory accesses in
bounds.  A mutant that passes every pin would mean the pins cannot tell that
mistake from the definition.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = [
    ("drop_scale", "s[j] = c->scale * acc;", "s[j] = acc;"),
    ("causal_off_by_one", "return causal ? i + 1 : n;", "return causal ? i : n;"),
    ("causal_ignored", "return causal ? i + 1 : n;", "return causal ? n : n;"),
    ("transposed_scores", "const double* qi = c->q + i * c->d;", "const double* qi = c->k + i * c->d;"),
    ("reversed_values", "const double* vj = c->v + j * c->d;", "const double* vj = c->v + (nvis - 1 - j) * c->d;"),
    ("sum_without_max", "    l += exp(s[j] - m);", "    l += exp(s[j]);"),
    ("lse_without_max", "c->lse[r] = m + log(l);", "c->lse[r] = log(l);"),
    ("p_wrong_sign", "double pij = exp(s[j] - m) / l;", "double pij = exp(m - s[j]) / l;"),
    ("p_not_normalised", "double pij = exp(s[j] - m) / l;", "double pij = exp(s[j] - m);"),
    ("softmax_not_normalised", "y[j] = exp(x[j] - m) / l;", "y[j] = exp(x[j] - m);"),
    ("softmax_min_not_max", "if (x[j] > m) m = x[j];", "if (x[j] < m) m = x[j];"),
    ("softmax_sum_unshifted", "    l += exp(x[j] - m);", "    l += exp(x[j]);"),
    ("online_no_rescale", "dsum = dsum * exp(m - m_next) + exp(x[j] - m_next);", "dsum = dsum + exp(x[j] - m_next);"),
    ("online_rescale_sign", "dsum = dsum * exp(m - m_next)", "dsum = dsum * exp(m_next - m)"),
    ("tiled_no_o_rescale", "o[e] = o[e] * alpha;", "o[e] = o[e];"),
    ("tiled_no_l_rescale", "l = l * alpha + psum;", "l = l + psum;"),
    ("tiled_tile_max_weights", "psum += exp(s[j] - m_new);", "psum += exp(s[j] - rowmax);"),
    ("tiled_no_final_divide", "o[e] = o[e] / l;", "o[e] = o[e];"),
    ("probs_not_normalised", "p[j] = exp(p[j] - m) / l;", "p[j] = exp(p[j] - m);"),
    ("bwd_row_drop_d", "const double ds = exp(s[j] - m) / l * (dp[j] - di);",
     "const double ds = exp(s[j] - m) / l * dp[j];"),
    ("bwd_col_drop_d", "const double ds = pij * (dpij - c->dd[i]);", "const double ds = pij * dpij;"),
    ("bwd_d_sign", "di += exp(s[j] - m) / l * dp[j];", "di -= exp(s[j] - m) / l * dp[j];"),
    ("bwd_dq_no_scale", "dqi[e] += c->scale * ds * kj[e];", "dqi[e] += ds * kj[e];"),
    ("bwd_dk_transposed", "dkj[e] += c->scale * ds * qi[e];", "dkj[e] += c->scale * ds * kj[e];"),
    ("bwd_dv_uses_v", "dvj[e] += pij * doi[e];", "dvj[e] += pij * vj[e];"),
    ("bwd_col_unnormalised", "const double pij = exp(c->scale * sij - c->lse[i]);",
     "const double pij = exp(c->scale * sij);"),
    ("bwd_col_causal_off_by_one", "for (long i = c->causal ? j : 0; i < n; ++i) {",
     "for (long i = c->causal ? j + 1 : 0; i < n; ++i) {"),
    ("bwd_dp_uses_k", "    const double* vj = c->v + j * d;\n    double acc = 0.0;",
     "    const double* vj = c->k + j * d;\n    double acc = 0.0;"),
    ("bwd_given_o_ignored", "for (long e = 0; e < d; ++e) di += doi[e] * oi[e];",
     "for (long e = 0; e < d; ++e) di += doi[e] * doi[e];"),
    ("bwd_magnitude_signed", "mvj[e] += fabs(pij * doi[e]);", "mvj[e] += pij * doi[e];"),
    ("bwd_magnitude_wrong_operand", "mqi[e] += c->scale * fabs(ds * kj[e]);",
     "mqi[e] += c->scale * fabs(ds * c->q[i * d + e]);"),
    ("ranged_hi_exclusive", "const long i = c->rows[r], j0 = c->lo[i], j1 = c->hi[i];",
     "const long i = c->rows[r], j0 = c->lo[i], j1 = c->hi[i] > c->lo[i] ? c->hi[i] - 1 : c->hi[i];"),
    ("ranged_values_unshifted", "const double* vj = c->v + (j0 + t) * c->d;", "const double* vj = c->v + t * c->d;"),
    ("ranged_keys_from_zero", "for (long e = 0; e < c->d; ++e) acc += qrow[e] * kj[e];",
     "for (long e = 0; e < c->d; ++e) acc += qrow[e] * c->k[(j - j0) * c->d + e];"),
    ("ranged_query_is_key", "acc += qrow[e] * kj[e];", "acc += kj[e] * kj[e];"),
    ("keyset_ignores_list", "const double* kk = c->k + c->keys[b0 + t] * c->d;",
     "const double* kk = c->k + t * c->d;"),
    ("keyset_values_misplaced", "const double* vv = c->v + c->keys[b0 + t] * c->d;",
     "const double* vv = c->v + c->keys[b0] * c->d;"),
    ("keyset_sum_unshifted", "den += exp(sc[t] - mx);", "den += exp(sc[t]);"),
    ("keyset_empty_is_nan", "    c->lse[r] = -INFINITY;\n    return;", "    c->lse[r] = NAN;\n    return;"),
    ("partition_drops_rows", "jobs[t].end = (t + 1) * per < nrows ? (t + 1) * per : nrows;",
     "jobs[t].end = (t + 1) * per < nrows ? (t + 1) * per - 1 : nrows;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    mpath = tmp_path / f"mutant_{name}.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.build(str(mpath), str(tmp_path / f"libmutant_{name}.so"))
    orc = oracle.load(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError, ValueError) as e:
            caught.append(pin.__name__)
    assert caught, f"mutation {name} passes every pin"
