"""Mutation tests of the pins: each plausible mistake planted in the oracle's
source (on the CPU, in a temporary copy) must make at least one pin fail.

Mutants follow the silent failure modes the correctness section of "colibri
Vulkan compute backend complete guide" names (a mis-decoded nibble, a
reversed group direction, scrambled scale order) plus dropped terms, wrong
signs, swapped operands and transposed indexes.  Every mutant keeps all
memory accesses in bounds.
"""
import os

import pytest

import oracle
from oracle import build as obuild
import pinlib

SRC = open(obuild.SRC).read()

MUTANTS = {
    "nibble_order_swapped": ("    if (k % 2 == 0)\n        return byte & 0x0F;",
                             "    if (k % 2 != 0)\n        return byte & 0x0F;"),
    "int4_offset_dropped": ("return (double)(nibble_at(row, k) - 8);", "return (double)(nibble_at(row, k));"),
    "int4_offset_wrong": ("return (double)(nibble_at(row, k) - 8);", "return (double)(nibble_at(row, k) - 7);"),
    "int4_row_stride": ("        const uint8_t *row = (const uint8_t *)m->q + o * (m->K / 2);\n"
                        "        return (double)(nibble_at(row, k) - 8);",
                        "        const uint8_t *row = (const uint8_t *)m->q + o * (m->K / 4);\n"
                        "        return (double)(nibble_at(row, k) - 8);"),
    "group_direction_reversed": ("return (double)m->scales[o * groups + k / m->gs];",
                                 "return (double)m->scales[o * groups + (m->K - 1 - k) / m->gs];"),
    "scale_index_shifted": ("return (double)m->scales[o * groups + k / m->gs];",
                            "return (double)m->scales[o * groups + (k / m->gs + 1) % groups];"),
    "scale_row_ignored": ("return (double)m->scales[o * groups + k / m->gs];",
                          "return (double)m->scales[k / m->gs];"),
    "e2m1_bias_wrong": ("mag = ldexp(1.0 + 0.5 * mant, expo - 1);", "mag = ldexp(1.0 + 0.5 * mant, expo);"),
    "e2m1_subnormal_wrong": ("mag = 0.5 * mant;", "mag = 1.0 * mant;"),
    "e2m1_sign_ignored": ("    return sign ? -mag : mag;\n}\n\n/* Value of a binary",
                          "    return (void)sign, mag;\n}\n\n/* Value of a binary"),
    "int3_planes_swapped": ("return low | (high << 2);", "return (low << 1) | high;"),
    "int3_offset_wrong": ("return (double)(int3_code(low_row, high_row, k) - 4);",
                          "return (double)(int3_code(low_row, high_row, k) - 3);"),
    "int3_low_bits_reversed": ("(low_row[k / 16] >> (2 * (k % 16)))", "(low_row[k / 16] >> (30 - 2 * (k % 16)))"),
    "int3_high_bits_reversed": ("(high_row[k / 32] >> (k % 32))", "(high_row[k / 32] >> (31 - k % 32))"),
    "int8_unsigned": ("    case 1: {\n        const int8_t *row = (const int8_t *)m->q + o * m->K;\n        return (double)row[k];",
                      "    case 1: {\n        const int8_t *row = (const int8_t *)m->q + o * m->K;\n        return (double)(uint8_t)row[k];"),
    "dot_first_term_dropped": ("        sum += term;", "        sum += (k == 0) ? 0.0 : term;"),
    "dot_sign_flipped": ("        double term = orc_weight(m, o, k) * xk;", "        double term = -orc_weight(m, o, k) * xk;"),
    "normaliser_not_absolute": ("        mag += fabs(term);", "        mag += term;"),
    "gemv_output_transposed": ("row_dot(m, o, x + s * m->K, NULL, &y[s * m->O + o]",
                               "row_dot(m, o, x + s * m->K, NULL, &y[o * S + s]"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "silu_missing_z": ("return z / (1.0 + exp(-z));", "return 1.0 / (1.0 + exp(-z));"),
    "gate_up_swapped": ("h[idx] = orc_silu(gc) * uc;", "h[idx] = orc_silu(uc) * gc;"),
    "clamp_gate_from_below": ("double gc = g > limit ? limit : g;", "double gc = g < limit ? limit : g;"),
    "clamp_up_one_sided": ("double uc = u > limit ? limit : (u < -limit ? -limit : u);",
                           "double uc = u > limit ? limit : u;"),
    "clamp_gate_ignored": ("double gc = g > limit ? limit : g;", "double gc = g;"),
    "clamp_group_ignores_limit": ("mlp_one(&gates[e], &ups[e], &downs[e], x + t * gates[e].K, limit,",
                                  "mlp_one(&gates[e], &ups[e], &downs[e], x + t * gates[e].K, INFINITY,"),
    "clamp_shared_ignores_limit": ("                    limit, h_work, nh_work, dy_work, dabs_work);",
                                   "                    INFINITY, h_work, nh_work, dy_work, dabs_work);"),
    "router_weight_dropped": ("yt[o] += wr * dy_work[o];", "yt[o] += dy_work[o];"),
    "shared_expert_dropped": ("                yt[o] += dy_work[o];", "                yt[o] += 0.0 * dy_work[o];"),
    "down_uses_gate_rows": ("mlp_one(&gates[e], &ups[e], &downs[e],", "mlp_one(&gates[e], &ups[e], &downs[(e + 1) % n_experts],"),
    "route_ties_to_higher_index": ("(best < 0 || key[e] > key[best])", "(best < 0 || key[e] >= key[best])"),
    "route_max_not_subtracted": ("z += exp((double)l[e] - mx);", "z += exp((double)l[e]);"),
    "route_sigmoid_sign": ("p[e] = 1.0 / (1.0 + exp(-(double)l[e]));", "p[e] = 1.0 / (1.0 + exp((double)l[e]));"),
    "route_bias_in_weight": ("w[t * k + r] = p[best];", "w[t * k + r] = bias ? key[best] : p[best];"),
    "route_bias_ignored": ("key[e] = bias ? p[e] + (double)bias[e] : (double)l[e];", "key[e] = (double)l[e];"),
    "route_renorm_ignored": ("            if (renorm)\n                v = v / sum;", "            (void)renorm;"),
    "route_scale_dropped": ("w[t * k + r] = v * w_scale;", "w[t * k + r] = v;"),
    "route_weight_of_wrong_expert": ("w[t * k + r] = p[best];", "w[t * k + r] = p[(best + 1) % E];"),
    "minifloat_bias_off_by_one": ("int bias = (1 << (ebits - 1)) - 1;", "int bias = (1 << (ebits - 1));"),
    "minifloat_subnormal_scale": ("mag = ldexp((double)frac, 1 - bias - mbits);",
                                  "mag = ldexp((double)frac, -bias - mbits);"),
    "minifloat_implicit_one_dropped": ("mag = ldexp((double)((1u << mbits) + frac), (int)expo - bias - mbits);",
                                       "mag = ldexp((double)frac, (int)expo - bias - mbits);"),
    "minifloat_sign_ignored": ("    return sign ? -mag : mag;\n}\n\n/* int3", "    return (void)sign, mag;\n}\n\n/* int3"),
    "e4m3_read_as_ieee": ("return orc_minifloat(row[k], 4, 3, 0);", "return orc_minifloat(row[k], 4, 3, 1);"),
    "e4m3_read_as_e5m2": ("return orc_minifloat(row[k], 4, 3, 0);", "return orc_minifloat(row[k], 5, 2, 0);"),
    "bf16_fields_shifted": ("return orc_minifloat(row[k], 8, 7, 1);", "return orc_minifloat(row[k], 7, 8, 1);"),
    "f16_odd_column_low": ("        return orc_minifloat(row[k], 5, 10, 1);",
                           "        return orc_minifloat(row[k ^ 1], 5, 10, 1);"),
    "f16_read_as_bf16": ("return orc_minifloat(row[k], 5, 10, 1);", "return orc_minifloat(row[k], 8, 7, 1);"),
    "f32_row_stride_halved": ("        const float *row = (const float *)m->q + o * m->K;",
                              "        const float *row = (const float *)m->q + o * (m->K / 2);"),
    "int8_gs_unsigned": ("    case 13: {\n        const int8_t *row = (const int8_t *)m->q + o * m->K;\n        return (double)row[k];",
                         "    case 13: {\n        const int8_t *row = (const int8_t *)m->q + o * m->K;\n        return (double)(uint8_t)row[k];"),
    "fp8_block_row_ignored": ("return (double)m->scales[(o / 128) * blocks + k / 128];",
                              "return (double)m->scales[0 * (o / 128) * blocks + k / 128];"),
    "fp8_block_axes_swapped": ("return (double)m->scales[(o / 128) * blocks + k / 128];",
                               "return (double)m->scales[((k / 128) % ((m->O + 127) / 128)) * blocks + (o / 128) % blocks];"),
    "fp8_block_column_ignored": ("return (double)m->scales[(o / 128) * blocks + k / 128];",
                                 "return (double)m->scales[(o / 128) * blocks];"),
    "no_scale_formats_take_f16_scale": ("if (m->fmt == 10 || m->fmt == 11 || m->fmt == 14)\n        return 1.0;",
                                        "if (m->fmt == 10 || m->fmt == 11 || m->fmt == 14)\n        return m->fmt == 14 ? 0.5 : 1.0;"),
    "v4_ties_away_from_zero": ("return nearbyint(v / quantum) * quantum;", "return round(v / quantum) * quantum;"),
    "v4_round_truncates": ("return nearbyint(v / quantum) * quantum;", "return trunc(v / quantum) * quantum;"),
    "v4_subnormal_quantum": ("int lead = e - 1 < emin ? emin : e - 1;", "int lead = e - 1;"),
    "v4_scale_allows_448": ("while (m / (s / 2.0) < 448.0)", "while (m / (s / 2.0) <= 448.0)"),
    "v4_scale_not_restored": ("e4[j] = orc_round_fmt(e4[j] / s, 3, -6) * s;", "e4[j] = orc_round_fmt(e4[j] / s, 3, -6);"),
    "v4_e4m3_as_e5m2": ("e4[j] = orc_round_fmt(e4[j] / s, 3, -6) * s;", "e4[j] = orc_round_fmt(e4[j] / s, 2, -14) * s;"),
    "v4_block_max_half": ("        for (long j = b0; j < b0 + 128; j++) {\n            if (fabs(e4[j]) > m",
                          "        for (long j = b0; j < b0 + 64; j++) {\n            if (fabs(e4[j]) > m"),
    "v4_weight_dropped": ("double hv = orc_silu(gc) * uc * wr;", "double hv = orc_silu(gc) * uc;"),
    "v4_gate_not_rounded": ("double gb = bf16(g), ub = bf16(u);", "double gb = g, ub = bf16(u);"),
    "v4_clamp_before_rounding": ("double gc = gb > limit ? limit : gb;", "double gc = g > limit ? limit : bf16(g);"),
    "v4_down_not_rounded": ("        d[o] = bf16(sum);", "        d[o] = sum;"),
    "v4_combine_rank_order": ("if (!done[r] && (pick < 0 || ids[r] < ids[pick]))", "if (!done[r] && pick < 0)"),
    "v4_bound_ignores_sign": ("            lo += p < q ? p : q;", "            lo += p;"),
    "group_down_weight_dropped": ("            sum += wr * d;\n            mag += fabs(wr) * a;",
                                  "            sum += d;\n            mag += fabs(wr) * a;"),
    "group_down_slot_by_rank": ("row_dot(&downs[e], o, h + (t * k + r) * I, NULL, &d, &a);",
                                "row_dot(&downs[e], o, h + r * I, NULL, &d, &a);"),
    "group_down_shared_slot_fixed": ("h + (S * k + t) * I", "h + (S * k) * I"),
    "group_down_shared_dropped": ("            sum += ds;", "            sum += 0.0 * ds;"),
    "group_down_norm_signed_weight": ("            mag += fabs(wr) * a;", "            mag += wr * a;"),
    "group_down_bad_id_ignored": ("y[idx] = bad ? NAN : sum;", "y[idx] = sum;"),
    "nh_spare_factor_k": ("nh[idx] = fabs(silu_slope(gc)) * ag * fabs(uc) + fabs(orc_silu(gc)) * au;",
                          "nh[idx] = (fabs(silu_slope(gc)) * ag * fabs(uc) + fabs(orc_silu(gc)) * au) * G->K;"),
    "nh_up_term_dropped": ("nh[idx] = fabs(silu_slope(gc)) * ag * fabs(uc) + fabs(orc_silu(gc)) * au;",
                           "nh[idx] = fabs(silu_slope(gc)) * ag * fabs(uc);"),
    "nh_slope_is_sigmoid": ("return sig * (1.0 + z * (1.0 - sig));", "return sig;"),
    "group_norm_nh_dropped": ("mag += fabs(wk) * (fabs(h[k]) + nh[k]);", "mag += fabs(wk) * fabs(h[k]);"),
    "group_norm_weight_dropped": ("at[o] += fabs(wr) * dabs_work[o];", "at[o] += dabs_work[o];"),
    "token_x_not_advanced": ("mlp_one(&gates[e], &ups[e], &downs[e], x + t * gates[e].K,",
                             "mlp_one(&gates[e], &ups[e], &downs[e], x,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    search, replace = MUTANTS[name]
    assert SRC.count(search) == 1, f"mutant {name}: patch site not unique"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(search, replace))
    lib_path = str(tmp_path / "libmutant.so")
    obuild.build(str(src), lib_path, extra=("-w",))
    lib = oracle.load(lib_path)
    failed = []
    for pin in pinlib.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
            break   # one failing pin is enough
    assert failed, f"mutant {name} passed every pin"


def test_unmutated_copy_passes(tmp_path):
    """The same build route with no patch passes every pin (the harness is fair)."""
    src = tmp_path / "same.c"
    src.write_text(SRC)
    lib_path = str(tmp_path / "libsame.so")
    obuild.build(str(src), lib_path)
    lib = oracle.load(lib_path)
    for pin in pinlib.ALL_PINS:
        pin(lib)
