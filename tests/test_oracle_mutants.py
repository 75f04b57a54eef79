"""Pin sensitivity: plausible mistakes planted in a copy of the oracle's C
source must each be caught by at least one pin.  The mutants are built with
gcc into a temporary directory; the real oracle is never modified."""
import os
import shutil
import tempfile

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

# (name, original text, mutated text): each replacement must match exactly once.
MUTATIONS = [
    ("f16_exponent_bias", "expo - 25);", "expo - 24);"),
    ("f16_subnormal_scale", "ldexp((double)frac, -24)", "ldexp((double)frac, -23)"),
    ("bf16_exponent_bias", "expo - 134);", "expo - 133);"),
    ("bf16_hidden_bit", "(double)(128 + frac)", "(double)(frac)"),
    ("diagonal_excluded", "return j <= i + c;", "return j < i + c;"),
    ("mask_polarity", "return j <= i + c;", "return j >= i + c;"),
    ("causal_top_left", "if (!visible(i, j, Sk - Sq, causal)) { srow[j] = -INFINITY; continue; }",
     "if (!visible(i, j, 0, causal)) { srow[j] = -INFINITY; continue; }"),
    ("causal_offset_sign", "if (!visible(i, j, Sk - Sq, causal)) { srow[j] = -INFINITY; continue; }",
     "if (!visible(i, j, Sq - Sk, causal)) { srow[j] = -INFINITY; continue; }"),
    ("dropped_feature", "for (int d = 0; d < D; ++d) acc += qrow[d] * kr[d];",
     "for (int d = 0; d < D - 1; ++d) acc += qrow[d] * kr[d];"),
    ("wrong_key_row", "const double* kr = K + j * D;", "const double* kr = K + ((j + 1) % Sk) * D;"),
    ("transposed_scores", "row_attention(Qd + i * D, Kd, Vd,",
     "row_attention(Sq == Sk ? Kd + i * D : Qd + i * D, Sq == Sk ? Qd : Kd, Vd,"),
    ("scale_missing", "        srow[j] = scale * acc;\n    }\n    /* pass 1: row maximum */",
     "        srow[j] = acc;\n    }\n    /* pass 1: row maximum */"),
    ("ext_scale_missing", "        srow[j] = scale * acc;\n    }\n    double m = -INFINITY;",
     "        srow[j] = acc;\n    }\n    double m = -INFINITY;"),
    ("exp_sign", "double p = exp(srow[j] - m);", "double p = exp(m - srow[j]);"),
    ("exp_without_max", "double p = exp(srow[j] - m);", "double p = exp(srow[j]);"),
    ("not_normalised", "for (int64_t j = 0; j < Sk; ++j) srow[j] = srow[j] / l;", ""),
    ("v_rows_reversed", "const double* vr = V + j * D;", "const double* vr = V + (Sk - 1 - j) * D;"),
    ("lse_drops_max", "return m + log(l);", "return log(l);"),
    ("lse_log2", "return m + log(l);", "return m + log2(l);"),
    ("rows_wrong_query", "ora_decode(q + rows[r] * D, Qr, D, dtype);",
     "ora_decode(q + (rows[r] ^ 1) * D, Qr, D, dtype);"),
    # backward
    ("bwd_rowdot_dropped", "for (int64_t j = 0; j < Sk; ++j) srow[j] = prow[j] * (srow[j] - rowdot);",
     "for (int64_t j = 0; j < Sk; ++j) srow[j] = prow[j] * srow[j];"),
    ("bwd_ds_sign", "for (int64_t j = 0; j < Sk; ++j) srow[j] = prow[j] * (srow[j] - rowdot);",
     "for (int64_t j = 0; j < Sk; ++j) srow[j] = prow[j] * (rowdot - srow[j]);"),
    ("bwd_rowdot_unweighted", "            rowdot += prow[j] * dp;\n", "            rowdot += dp;\n"),
    ("bwd_dp_uses_keys", "            const double* vr = Vd + j * D;\n            double dp = 0.0;\n"
     "            for (int d = 0; d < D; ++d) dp += gi[d] * vr[d];\n            srow[j] = dp;",
     "            const double* vr = Kd + j * D;\n            double dp = 0.0;\n"
     "            for (int d = 0; d < D; ++d) dp += gi[d] * vr[d];\n            srow[j] = dp;"),
    ("bwd_dq_scale_missing", "            for (int d = 0; d < D; ++d) gq[d] += srow[j] * kr[d];\n        }\n"
     "        for (int d = 0; d < D; ++d) gq[d] *= sc;",
     "            for (int d = 0; d < D; ++d) gq[d] += srow[j] * kr[d];\n        }\n"),
    ("bwd_dq_uses_values", "            const double* kr = Kd + j * D;\n            for (int d = 0; d < D; ++d) gq[d] += srow[j] * kr[d];",
     "            const double* kr = Vd + j * D;\n            for (int d = 0; d < D; ++d) gq[d] += srow[j] * kr[d];"),
    ("bwd_dq_uses_probs", "for (int d = 0; d < D; ++d) gq[d] += srow[j] * kr[d];",
     "for (int d = 0; d < D; ++d) gq[d] += prow[j] * kr[d];"),
    ("bwd_dk_scale_missing", "        for (int d = 0; d < D; ++d) gk[d] *= sc;\n", ""),
    ("bwd_dv_uses_ds", "gv[d] += pij * gi[d];", "gv[d] += sij * gi[d];"),
    ("bwd_dk_uses_dout", "gk[d] += sij * qr[d];", "gk[d] += sij * gi[d];"),
    ("bwd_dk_uses_probs", "gk[d] += sij * qr[d];", "gk[d] += pij * qr[d];"),
    ("bwd_dk_transposed", "const double pij = P[i * Sk + j], sij = dS[i * Sk + j];",
     "const double pij = P[i * Sk + j], sij = dS[(Sq == Sk ? j * Sk + i : i * Sk + j)];"),
    ("bwd_rows_rowdot_dropped", "const double sij = pij * (dp - rowdot);", "const double sij = pij * dp;"),
    ("bwd_rows_dq_rowdot_dropped", "const double ds = Pr[j] * (Sr[j] - rowdot);", "const double ds = Pr[j] * Sr[j];"),
    ("bwd_rows_dk_scale_missing", "for (int d = 0; d < D; ++d) dk[r * D + d] *= sc;",
     "for (int d = 0; d < D; ++d) dk[r * D + d] *= 1.0;"),
    ("bwd_rows_wrong_key", "const int64_t j = krows[r] % Sk;", "const int64_t j = (krows[r] + 1) % Sk;"),
    # explicit mask and dropout
    ("philox_nine_rounds", "for (int r = 0; r < 10; ++r) {\n        if (r > 0) { k0 += 0x9E3779B9u;",
     "for (int r = 0; r < 9; ++r) {\n        if (r > 0) { k0 += 0x9E3779B9u;"),
    ("philox_multiplier", "(uint64_t)0xD2511F53u * c0", "(uint64_t)0xD2511F57u * c0"),
    ("philox_key_bump", "k1 += 0xBB67AE85u;", "k1 += 0x9E3779B9u;"),
    ("philox_output_order", "out[0] = c0; out[1] = c1;", "out[0] = c1; out[1] = c0;"),
    ("threshold_truncated", "const long t = lrintf(p * 65536.0f);", "const long t = (long)(p * 65536.0f);"),
    ("keep_compare", "return (int)r16 >= t;", "return (int)r16 > t;"),
    ("keep_word", "out[(j & 7) >> 1]", "out[j & 3]"),
    ("keep_half", ">> (16 * (j & 1))) & 0xffffu", ">> (16 * ((j >> 1) & 1))) & 0xffffu"),
    ("keep_counter_swapped", "{(uint32_t)(j >> 3), (uint32_t)i, (uint32_t)bh, offset}",
     "{(uint32_t)i, (uint32_t)(j >> 3), (uint32_t)bh, offset}"),
    ("keep_offset_ignored", "(uint32_t)bh, offset};", "(uint32_t)bh, 0u};"),
    ("keep_head_ignored", "(uint32_t)i, (uint32_t)bh, offset}", "(uint32_t)i, 0u, offset}"),
    ("keep_seed_words_swapped", "{(uint32_t)seed, (uint32_t)(seed >> 32)}",
     "{(uint32_t)(seed >> 32), (uint32_t)seed}"),
    ("ext_mask_polarity", "(!mrow || mrow[j] != 0)", "(!mrow || mrow[j] == 0)"),
    ("ext_mask_head_stride", "mrow = mask + b * mstride[0] + h * mstride[1] + i * mstride[2];",
     "mrow = mask + b * mstride[0] + i * mstride[2];"),
    ("ext_mask_row_stride", "mrow = mask + b * mstride[0] + h * mstride[1] + i * mstride[2];",
     "mrow = mask + b * mstride[0] + h * mstride[1] + i * Sk;"),
    ("dropout_scale_missing", "const double keep_scale = 65536.0 / (65536.0 - (double)t);",
     "const double keep_scale = 1.0;"),
    ("dropout_renormalised", "        srow[j] = e;\n        l += e;",
     "        srow[j] = e;\n        l += (t > 0 && !keep_element(seed, offset, bh, i, j, t)) ? 0.0 : e;"),
    ("bwdx_dv_keep_missing", "const double pz = Pr[j] * Zr[j];", "const double pz = Pr[j];"),
    ("bwdx_dp_keep_missing", "                dPr[j] = Zr[j] * a;", "                dPr[j] = a;"),
    ("bwdx_keep_scale_missing", "const double keep_scale = 65536.0 / (double)(65536 - t);",
     "const double keep_scale = 1.0;"),
    ("bwdx_mask_ignored", "if (!visible(i, j, causal_diag, causal) || (mrow && mrow[j] == 0)) { Pr[j] = -INFINITY; continue; }",
     "if (!visible(i, j, causal_diag, causal)) { Pr[j] = -INFINITY; continue; }"),
    ("bwdx_offset_sign", "if (!visible(i, j, causal_diag, causal) ||", "if (!visible(i, j, -causal_diag, causal) ||"),
    ("bwdx_offset_ignored", "if (!visible(i, j, causal_diag, causal) ||", "if (!visible(i, j, Sk - Sq, causal) ||"),
    ("bwdx_rowdot_undropped", "                rowdot += Pr[j] * dPr[j];", "                rowdot += Pr[j] * a;"),
    ("bwdx_ds_sign", "const double ds = Pr[j] * (dPr[j] - rowdot);\n                    for (int d = 0; d < D; ++d) gq[d] += ds * Kd[j * D + d];",
     "const double ds = Pr[j] * (rowdot - dPr[j]);\n                    for (int d = 0; d < D; ++d) gq[d] += ds * Kd[j * D + d];"),
    ("bwdx_dk_uses_dout", "                    ak[d] += ds * Qr[d];", "                    ak[d] += ds * Gr[d];"),
    ("bwdx_dk_scale_missing", "dk[r * D + d] = sc * dk[r * D + d];", "dk[r * D + d] = dk[r * D + d];"),
    ("bwdx_wrong_key", "const int64_t j = krows[r] - bh * Sk;", "const int64_t j = (krows[r] - bh * Sk + 1) % Sk;"),
    ("ext_causal_ignored", "const int vis = visible(i, j, c, causal) && (!mrow || mrow[j] != 0);",
     "const int vis = (!mrow || mrow[j] != 0);"),
    ("ext_offset_off_by_one", "const int vis = visible(i, j, c, causal) &&", "const int vis = visible(i, j, c + 1, causal) &&"),
    ("ext_offset_ignored", "row_attention_ext(Qr, Kd, Vd, bh, i, causal_diag, Sk,", "row_attention_ext(Qr, Kd, Vd, bh, i, Sk - Sq, Sk,"),
]


def _mutant_source(orig: str, name: str, old: str, new: str) -> str:
    assert orig.count(old) == 1, (name, orig.count(old))
    return orig.replace(old, new)


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutant_is_caught(workdir, name, old, new):
    orig = open(obuild.SRC).read()
    src = os.path.join(workdir, name + ".c")
    with open(src, "w") as f:
        f.write(_mutant_source(orig, name, old, new))
    lib_path = obuild.build(src, os.path.join(workdir, "lib" + name + ".so"),
                            extra_flags=("-Wno-unused-parameter", "-Wno-unused-variable"))
    lib = oracle.load(lib_path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
        except Exception as e:  # a crash inside a pin also counts as detection
            caught.append("%s(%s)" % (pin.__name__, type(e).__name__))
    assert caught, "mutant %s passed every pin" % name
