"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that the
pins catch every one of them.  This is what makes the pins a real check: a pin
set that a dropped term, a wrong sign, a wrong index or a swapped operand could
slip past would not pin anything."""
import functools
import os

import pytest

import oracle
import oracle_pins
from oracle import oracle as oracle_mod

# (name, text in gdn_oracle.c, replacement)
MUTANTS = [
    ("dropped_decay", "S[e] = a * S[e];", "S[e] = S[e];"),
    ("gate_sign", "exp(oracle_load(g, t * hv + h, gate_dtype))", "exp(-oracle_load(g, t * hv + h, gate_dtype))"),
    ("gate_on_key_head", "exp(oracle_load(g, t * hv + h, gate_dtype))", "exp(oracle_load(g, t * hv + kh, gate_dtype))"),
    ("dropped_beta", "const double u = b * (", "const double u = ("),
    ("delta_sign", "(oracle_load(v, v_off + j, v_dtype) - p)", "(oracle_load(v, v_off + j, v_dtype) + p)"),
    ("write_sign", "row[i] += u * oracle_load(k, qk_off + i, qk_dtype);",
     "row[i] -= u * oracle_load(k, qk_off + i, qk_dtype);"),
    ("write_with_query", "row[i] += u * oracle_load(k, qk_off + i, qk_dtype);",
     "row[i] += u * oracle_load(q, qk_off + i, qk_dtype);"),
    ("readout_with_key", "o += row[i] * oracle_load(q, qk_off + i, qk_dtype);",
     "o += row[i] * oracle_load(k, qk_off + i, qk_dtype);"),
    ("readout_before_write", "o += row[i] * oracle_load(q, qk_off + i, qk_dtype);",
     "o += (row[i] - u * oracle_load(k, qk_off + i, qk_dtype)) * oracle_load(q, qk_off + i, qk_dtype);"),
    ("delta_on_undecayed_state", "p += row[i] * oracle_load(k, qk_off + i, qk_dtype);",
     "p += (row[i] / a) * oracle_load(k, qk_off + i, qk_dtype);"),
    ("group_map_modulo", "const int32_t kh = h / group;", "const int32_t kh = h % hk;"),
    ("transposed_state", "double *row = S + (size_t)j * dk;", "double *row = S + (size_t)j;"),
    ("value_index_key_heads", "const int64_t v_off = (t * hv + h) * (int64_t)dv;",
     "const int64_t v_off = (t * hk + h) * (int64_t)dv;"),
    ("dropped_h0", "S[e] = h0 ? h0[state_off + e] : 0.0;", "S[e] = 0.0;"),
    ("query_scaled", "o += row[i] * oracle_load(q, qk_off + i, qk_dtype);",
     "o += row[i] * oracle_load(q, qk_off + i, qk_dtype) / sqrt((double)dk);"),
    ("bf16_low_half", "uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;",
     "uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 15;"),
]


# Mistakes in the fused-path preprocessing, caught by the preprocessing pins.
PRE_MUTANTS = [
    ("norm_without_eps", "const double dq = norm_qk ? sqrt(sq + eps) : 1.0;",
     "const double dq = norm_qk ? sqrt(sq) : 1.0;"),
    ("norm_q_by_k", "const double dq = norm_qk ? sqrt(sq + eps) : 1.0;",
     "const double dq = norm_qk ? sqrt(sk + eps) : 1.0;"),
    ("norm_squared", "qn[off + i] = oracle_load(q, off + i, io_dtype) / dq;",
     "qn[off + i] = oracle_load(q, off + i, io_dtype) / (dq * dq);"),
    ("softplus_as_exp", "log1p(exp(x))", "exp(x)"),
    ("softplus_as_identity", "log1p(exp(x))", "x"),
    ("A_log_not_exponentiated", "g[i] = -exp((double)A_log[h]) * ", "g[i] = -(double)A_log[h] * "),
    ("gate_sign_pre", "g[i] = -exp((double)A_log[h]) * ", "g[i] = exp((double)A_log[h]) * "),
    ("dt_bias_dropped", "(dt_bias ? (double)dt_bias[h] : 0.0)", "0.0"),
    ("A_log_first_head", "exp((double)A_log[h])", "exp((double)A_log[0])"),
    ("sigmoid_sign", "beta[i] = 1.0 / (1.0 + exp(-(double)b[i]));", "beta[i] = 1.0 / (1.0 + exp((double)b[i]));"),
    ("bf16_low_half_pre", "uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 16;",
     "uint32_t bits = ((uint32_t)((const uint16_t *)base)[idx]) << 15;"),
]


# Mistakes in the short convolution, caught by the convolution pins.
CONV_MUTANTS = [
    ("taps_reversed", "z += (double)w[(int64_t)c * K + j] * win[t + j];",
     "z += (double)w[(int64_t)c * K + (K - 1 - j)] * win[t + j];"),
    ("window_off_by_one", "z += (double)w[(int64_t)c * K + j] * win[t + j];",
     "z += (double)w[(int64_t)c * K + j] * win[t + j + 1];"),
    ("bias_dropped", "double z = bias ? (double)bias[c] : 0.0;", "double z = 0.0;"),
    ("silu_as_sigmoid", "y[(tb + t) * C + c] = silu ? z / (1.0 + exp(-z)) : z;",
     "y[(tb + t) * C + c] = silu ? 1.0 / (1.0 + exp(-z)) : z;"),
    ("state_newest_first", "win[m] = state ? state[((int64_t)n * C + c) * M + m] : 0.0;",
     "win[m] = state ? state[((int64_t)n * C + c) * M + (M - 1 - m)] : 0.0;"),
    ("state_ignored", "win[m] = state ? state[((int64_t)n * C + c) * M + m] : 0.0;", "win[m] = 0.0;"),
    ("state_out_first_inputs", "state_out[((int64_t)n * C + c) * M + m] = win[len + m];",
     "state_out[((int64_t)n * C + c) * M + m] = win[m];"),
    ("channel_stride", "win[M + t] = oracle_load(x, (tb + t) * C + c, io_dtype);",
     "win[M + t] = oracle_load(x, (tb + t) * C + (c + 1) % C, io_dtype);"),
]


# Mistakes in the gradients, caught by the gradient pins.
GRAD_MUTANTS = [
    ("dq_from_previous_state", "dq[qk_off + i] += Snew[(size_t)j * dk + i] * dO[j];",
     "dq[qk_off + i] += Sprev[(size_t)j * dk + i] * dO[j];"),
    ("dk_without_readout_term", "dk_out[qk_off + i] += a * Sprev[e] * dp[j];", "(void)0;"),
    ("dk_readout_undecayed", "dk_out[qk_off + i] += a * Sprev[e] * dp[j];",
     "dk_out[qk_off + i] += Sprev[e] * dp[j];"),
    ("dk_without_write_term", "dk_out[qk_off + i] += D[(size_t)j * dk + i] * u;", "(void)u;"),
    ("dp_sign", "dp[j] = -b * du[j];", "dp[j] = b * du[j];"),
    ("dbeta_without_readout", "db += du[j] * (vv[j] - p[j]);", "db += du[j] * vv[j];"),
    ("dv_without_beta", "dv_out[v_off + j] = b * du[j];", "dv_out[v_off + j] = du[j];"),
    ("dg_not_chained", "dg[tt * hv + h] = a * da;", "dg[tt * hv + h] = da;"),
    ("adjoint_not_decayed", "D[e] = a * D[e];", "D[e] = D[e];"),
    ("adjoint_misses_output", "D[(size_t)j * dk + i] += dO[j] * qv[i];", "(void)0;"),
    ("adjoint_misses_readout", "D[e] += dp[j] * kv[i];", "(void)0;"),
    ("recompute_off_by_one", "*Snew = st + (m + 1) * SZ", "*Snew = st + m * SZ"),
    ("dhT_ignored", "D[e] = dhT ? dhT[state_off + e] : 0.0;", "D[e] = 0.0;"),
    ("value_heads_of_next_group", "for (int32_t h = kh * group; h < (kh + 1) * group; ++h) {",
     "for (int32_t h = kh; h < kh + group; ++h) {"),
]


# Mistakes in the gradients of the preprocessing and the conv.
PRE_GRAD_MUTANTS = [
    ("norm_grad_without_projection", "dx[off + i] = dy[off + i] / s - xi * xdy / (s * s * s);",
     "dx[off + i] = dy[off + i] / s;"),
    ("norm_grad_cubed_as_squared", "dx[off + i] = dy[off + i] / s - xi * xdy / (s * s * s);",
     "dx[off + i] = dy[off + i] / s - xi * xdy / (s * s);"),
    ("norm_grad_without_eps", "const double s = sqrt(ss + eps);", "const double s = sqrt(ss);"),
    ("gate_grad_softplus_for_sigmoid", "da[i] = dg[i] * (-e * sig);", "da[i] = dg[i] * (-e * log1p(exp(z)));"),
    ("gate_grad_sign", "da[i] = dg[i] * (-e * sig);", "da[i] = dg[i] * (e * sig);"),
    ("beta_grad_as_beta", "db[i] = dbeta[i] * beta * (1.0 - beta);", "db[i] = dbeta[i] * beta;"),
    ("A_log_grad_missing_g", "dA_log[h] += dg[i] * g;", "dA_log[h] += dg[i];"),
    ("dt_bias_grad_from_dg", "ddt_bias[h] += da[i];", "ddt_bias[h] += dg[i];"),
    ("gate_grad_ignores_dt_bias", "const double z = (double)a[i] + (dt_bias ? (double)dt_bias[h] : 0.0);\n"
     "            const double e", "const double z = (double)a[i];\n            const double e"),
]

CONV_GRAD_MUTANTS = [
    ("silu_grad_as_sigmoid", "dz *= sig * (1.0 + z * (1.0 - sig));", "dz *= sig;"),
    ("conv_grad_taps_reversed", "dwin[t + j] += (double)w[(int64_t)c * K + j] * dz;",
     "dwin[t + j] += (double)w[(int64_t)c * K + (K - 1 - j)] * dz;"),
    ("dw_from_next_token", "dw[(int64_t)c * K + j] += dz * win[t + j];",
     "dw[(int64_t)c * K + j] += dz * win[t + j + 1];"),
    ("dbias_from_dy", "dbias[c] += dz;", "dbias[c] += dy[(tb + t) * C + c];"),
    ("dstate_newest_first", "dstate[((int64_t)n * C + c) * M + m] = dwin[m];",
     "dstate[((int64_t)n * C + c) * M + m] = dwin[M - 1 - m];"),
    ("dx_shifted", "dx[(tb + t) * C + c] = dwin[M + t];", "dx[(tb + t) * C + c] = dwin[M + t - 1];"),
]


@pytest.mark.parametrize("name,old,new", PRE_GRAD_MUTANTS + CONV_GRAD_MUTANTS,
                         ids=[m[0] for m in PRE_GRAD_MUTANTS + CONV_GRAD_MUTANTS])
def test_preprocessing_and_conv_gradient_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation site for %s not found once in the oracle source" % name
    mpath = tmp_path / ("pg_mutant_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / ("libpg_mutant_%s.so" % name))
    oracle.build(str(mpath), lib)
    caught = []
    if any(name == m[0] for m in PRE_GRAD_MUTANTS):
        pb = functools.partial(oracle_mod.preprocess_backward, library=lib)
        pre = functools.partial(oracle_mod.preprocess, library=lib)
        pins = [functools.partial(p, pb, pre) for p in oracle_pins.PRE_GRAD_PINS]
    else:
        cb = functools.partial(oracle_mod.short_conv_backward, library=lib)
        conv = functools.partial(oracle_mod.short_conv, library=lib)
        pins = [functools.partial(p, cb, conv) for p in oracle_pins.CONV_GRAD_PINS]
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError):
            caught.append(pin.func.__name__)
    assert caught, "gradient mutant %s passed every pin" % name


@pytest.mark.parametrize("name,old,new", GRAD_MUTANTS, ids=[m[0] for m in GRAD_MUTANTS])
def test_gradient_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    assert src.count(old) == 1, "mutation site for %s not found once in the oracle source" % name
    mpath = tmp_path / ("grad_mutant_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / ("libgrad_mutant_%s.so" % name))
    oracle.build(str(mpath), lib)
    bwd = functools.partial(oracle_mod.gdn_backward, library=lib)
    fwd = functools.partial(oracle_mod.gdn_forward, library=lib)
    caught = []
    for pin in oracle_pins.GRAD_PINS:
        try:
            pin(bwd, fwd)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "gradient mutant %s passed every pin" % name


@pytest.mark.parametrize("name,old,new", CONV_MUTANTS, ids=[m[0] for m in CONV_MUTANTS])
def test_conv_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    assert old in src, "mutation site for %s not found in the oracle source" % name
    mpath = tmp_path / ("conv_mutant_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / ("libconv_mutant_%s.so" % name))
    oracle.build(str(mpath), lib)
    conv = functools.partial(oracle_mod.short_conv, library=lib)
    caught = []
    for pin in oracle_pins.CONV_PINS:
        try:
            pin(conv)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "convolution mutant %s passed every pin" % name


@pytest.mark.parametrize("name,old,new", PRE_MUTANTS, ids=[m[0] for m in PRE_MUTANTS])
def test_preprocessing_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    assert old in src, "mutation site for %s not found in the oracle source" % name
    mpath = tmp_path / ("pre_mutant_%s.c" % name)
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / ("libpre_mutant_%s.so" % name))
    oracle.build(str(mpath), lib)
    pre = functools.partial(oracle_mod.preprocess, library=lib)
    fwd = functools.partial(oracle_mod.gdn_forward, library=lib)
    caught = []
    for pin in oracle_pins.PRE_PINS:
        try:
            pin(pre, fwd)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "preprocessing mutant %s passed every pin" % name


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    assert old in src, "mutation site for %s not found in the oracle source" % name
    if name == "transposed_state":
        # strided row: element (j, i) read from S[i * dv + j] instead of S[j * dk + i]
        src = src.replace("double *row = S + (size_t)j * dk;", "double *row = S + (size_t)j;")
        src = src.replace("row[i]", "row[(size_t)i * dv]")
    else:
        src = src.replace(old, new)
    mpath = tmp_path / ("mutant_%s.c" % name)
    mpath.write_text(src)
    lib = str(tmp_path / ("libmutant_%s.so" % name))
    oracle.build(str(mpath), lib)
    fwd = functools.partial(oracle_mod.gdn_forward, library=lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(fwd)
        except (AssertionError, ValueError):
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name


def test_unmutated_copy_passes(tmp_path):
    """Control: the same build path on an unmodified copy passes every pin."""
    with open(oracle_mod.SOURCE) as f:
        src = f.read()
    mpath = tmp_path / "copy.c"
    mpath.write_text(src)
    lib = str(tmp_path / "libcopy.so")
    oracle.build(str(mpath), lib)
    fwd = functools.partial(oracle_mod.gdn_forward, library=lib)
    for pin in oracle_pins.ALL_PINS:
        pin(fwd)
    pre = functools.partial(oracle_mod.preprocess, library=lib)
    for pin in oracle_pins.PRE_PINS:
        pin(pre, fwd)
    conv = functools.partial(oracle_mod.short_conv, library=lib)
    for pin in oracle_pins.CONV_PINS:
        pin(conv)
