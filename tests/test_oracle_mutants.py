"""Planted mistakes in a copy of the oracle must each trip at least one pin.

Each mutant is a one-line edit of ``oracle/dsc_oracle.c`` of the kind a
plausible implementation slip would make (a dropped tap, a wrong sign, a
shifted index, a transposed operand).  It is compiled into a temporary
directory on the CPU; the committed oracle is never touched.
"""
import os

import pytest

import oracle
from oracle import build as obuild
from tests import oracle_pins

MUTANTS = {
    "dropped_last_tap": ("for (int k = 0; k < W; ++k) {\n    if (t - k < 0) break;\n    s += wt[k]",
                         "for (int k = 0; k < W - 1; ++k) {\n    if (t - k < 0) break;\n    s += wt[k]"),
    "reversed_taps": ("s += wt[k] * x[IDX3(b, t - k, c, T, D)];",
                      "s += wt[W - 1 - k] * x[IDX3(b, t - k, c, T, D)];"),
    "strided_groups": ("static double conv_at(const double *x, const double *w, int64_t T, int64_t D,\n"
                       "                      int64_t G, int W, int H, int64_t b, int64_t t, int64_t c) {\n"
                       "  int64_t g = c / H;",
                       "static double conv_at(const double *x, const double *w, int64_t T, int64_t D,\n"
                       "                      int64_t G, int W, int H, int64_t b, int64_t t, int64_t c) {\n"
                       "  int64_t g = c % G;"),
    "dx_sign": ("acc += wk * ds_at(", "acc -= wk * ds_at("),
    "dx_no_residual": ("  if (residual) acc += dy[IDX3(b, tau, c, T, D)];\n  return acc;",
                       "  return acc;"),
    "dx_unshifted_weight": ("double wk = w[IDX3(b, t, g, T, G) * W + k];",
                            "double wk = w[IDX3(b, tau, g, T, G) * W + k];"),
    "dw_unshifted_x": ("           x[IDX3(b, t - k, c, T, D)];\n  return acc;",
                       "           x[IDX3(b, t, c, T, D)];\n  return acc;"),
    "U_tap_major": ("for (int r = 0; r < R; ++r) acc += z[n * R + r] * U[(int64_t)r * GW + col];\n"
                    "      w[n * GW + col] = acc;",
                    "for (int r = 0; r < R; ++r) acc += z[n * R + r] * U[(int64_t)r * GW + (col % W) * G + col / W];\n"
                    "      w[n * GW + col] = acc;"),
    "silu_grad_is_sigmoid": ("return sg * (1.0 + s * (1.0 - sg));", "return sg;"),
    "dz_drops_U": ("acc += dw[n * GW + col] * U[(int64_t)r * GW + col];",
                   "acc += dw[n * GW + col];"),
    "dU_drops_z": ("for (int64_t n = 0; n < N; ++n) acc += z[n * R + r] * dw[n * GW + col];",
                   "for (int64_t n = 0; n < N; ++n) acc += dw[n * GW + col];"),
    "decode_tap_order": ("s += w[(b * G + g) * W + k] * state_in[(b * S + (S - k)) * D + c];",
                         "s += w[(b * G + g) * W + k] * state_in[(b * S + (k - 1)) * D + c];"),
    "decode_no_shift": ("state_out[(b * S + j) * D + c] = state_in[(b * S + j + 1) * D + c];",
                        "state_out[(b * S + j) * D + c] = state_in[(b * S + j) * D + c];"),
    "decode_state_offset": ("int64_t t = T - S + j;", "int64_t t = T - S + j - 1;"),
    "static_reversed_taps": ("for (int k = 0; k < W && t - k >= 0; ++k) s += wg[k] * x",
                             "for (int k = 0; k < W && t - k >= 0; ++k) s += wg[W - 1 - k] * x"),
    "static_dw_one_sequence": ("    for (int64_t b = 0; b < B; ++b)\n      for (int64_t t = k; t < T; ++t)",
                               "    for (int64_t b = 0; b < 1; ++b)\n      for (int64_t t = k; t < T; ++t)"),
    "static_dx_unshifted_ds": ("acc += w[(c / H) * W + k] * static_ds(x, w, dy, T, D, W, H, act, b, tau + k, c);",
                               "acc += w[(c / H) * W + k] * static_ds(x, w, dy, T, D, W, H, act, b, tau, c);"),
    "varlen_tap_off_by_one": ("if (k <= pos[n] && t - k >= 0) s += w[(n * G + g) * W + k]",
                              "if (k < pos[n] && t - k >= 0) s += w[(n * G + g) * W + k]"),
    "varlen_dx_mask_own_pos": ("        if (k <= pos[m])\n", "        if (k <= pos[n])\n"),
    "varlen_dw_unmasked": ("        if (k <= pos[n] && tau - k >= 0)\n", "        if (tau - k >= 0)\n"),
    "gen_M_transposed": ("for (int64_t k = 0; k < Dh; ++k) a += xh[n * Dh + k] * M[k * GW + j];",
                         "for (int64_t k = 0; k < Dh; ++k) a += xh[n * Dh + k] * M[(j % Dh) * GW + (k % GW)];"),
    "residual_twice": ("y[n * D + c] = act_fn(s, act) + (residual ? x[n * D + c] : 0.0);\n    }\n  }\n}",
                       "y[n * D + c] = act_fn(s, act) + (residual ? 2.0 * x[n * D + c] : 0.0);\n    }\n  }\n}"),
}


@pytest.fixture(scope="module")
def src():
    return open(obuild.SRC).read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(src, name, tmp_path):
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation anchor for {name} is not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = obuild.build(str(path), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(oracle.load(lib))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
    os.remove(lib)
