"""Planted mistakes in the CPU oracle must be caught by its pins.

Each mutant is a copy of oracle/gdn_oracle.c with one plausible mistake (a dropped term, a
wrong sign, a swapped operand or index, another reduction order), built with gcc into a
temporary directory. Every mutant must fail at least one pin in tests/oracle_pins.py; a
mutant that passes them all would mean the pins cannot tell that mistake from the contract.
Mutations only change arithmetic or in-bounds indices, so no mutant writes out of bounds.
"""

import os

import pytest

import oracle_pins
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                   "gdn_oracle.c")

MUTANTS = {
    "decay_dropped": [("x[e] = a * s[e];", "x[e] = s[e];")],
    "delta_sign_flipped": [("float diff = v_i - u;", "float diff = u - v_i;")],
    "beta_dropped": [("float delta = b * diff;", "float delta = diff;")],
    "readout_before_update": [("return contract_dot(s, q, dk);", "return contract_dot(x, q, dk);")],
    "key_dot_uses_query": [("float u = contract_dot(x, k, dk);", "float u = contract_dot(x, q, dk);")],
    "decay_folded_into_dot": [("float u = contract_dot(x, k, dk);",
                               "float u = a * contract_dot(s, k, dk);")],
    "update_from_undecayed_state": [("s[e] = fmaf(delta, k[e], x[e]);",
                                     "s[e] = fmaf(delta, k[e], s[e]);")],
    "update_unfused": [("s[e] = fmaf(delta, k[e], x[e]);", "s[e] = delta * k[e] + x[e];")],
    "gqa_modulo_mapping": [("int hk = h / group;\n  int dk = J->dk;",
                            "int hk = h % J->Hk;\n  int dk = J->dk;"),
                           ("      int hk = h / group;", "      int hk = h % Hk;")],
    "leaf_chain_unfused": [("acc = fmaf(xl[e], yl[e], acc);", "acc = acc + xl[e] * yl[e];")],
    "leaf_start_fma_from_zero": [("float acc = xl[0] * yl[0];", "float acc = fmaf(xl[0], yl[0], 0.0f);")],
    "serial_leaf_sum": [("leaf[l] = leaf[l] + leaf[l + width];",
                         "leaf[0] = leaf[0] + leaf[l + width];")],
    "strided_leaves": [("const float *xl = x + l * m, *yl = y + l * m;",
                        "const float *xl = x + l, *yl = y + l;"),
                       ("float acc = xl[0] * yl[0];", "float acc = xl[0] * yl[0]; (void)xl;"),
                       ("acc = fmaf(xl[e], yl[e], acc);",
                        "acc = fmaf(xl[e * ORACLE_LEAVES], yl[e * ORACLE_LEAVES], acc);")],
    "value_row_reversed": [("(t * J->Hv + h) * (int64_t)J->dv + i, J->dtype)",
                            "(t * J->Hv + h) * (int64_t)J->dv + (J->dv - 1 - i), J->dtype)")],
    "initial_state_ignored": [("s[e] = J->S0 ? J->S0[", "s[e] = J->S0 ? 0.0f * J->S0[")],
    "chunk_states_all_in_slot_0": [("((j + 1) / J->C - 1) * J->cs_stride", "0 * J->cs_stride")],
    "resync_off_by_one": [("((int64_t)pos[n] + 1) % C == 0", "((int64_t)pos[n]) % C == 0")],
    "bf16_widening_wrong_half": [("(uint32_t)((const uint16_t *)base)[index] << 16",
                                  "(uint32_t)((const uint16_t *)base)[index] << 15")],
    # backward
    "bwd_sh_update_unfused": [("shr[e] = fmaf(gg, qq[e], shr[e]);", "shr[e] = gg * qq[e] + shr[e];")],
    "bwd_dq_from_previous_state": [("pq[(int64_t)i * dk + e] = gg * s_cur[e];",
                                    "pq[(int64_t)i * dk + e] = gg * s_prev[e];")],
    "bwd_du_sign": [("const float uh = -dvi;", "const float uh = dvi;")],
    "bwd_dk_drops_delta_term": [("pk[(int64_t)i * dk + e] = fmaf(uh, x[e], ds);",
                                 "pk[(int64_t)i * dk + e] = uh * x[e] + 0.0f * ds;")],
    "bwd_da_from_current_state": [("pa[i] = contract_dot(xh, s_prev, dk);",
                                   "pa[i] = contract_dot(xh, s_cur, dk);")],
    "bwd_no_decay": [("for (int e = 0; e < dk; ++e) shr[e] = A * xh[e];",
                      "for (int e = 0; e < dk; ++e) shr[e] = xh[e];")],
    "bwd_db_uses_delta": [("pb[i] = dh * diff;", "pb[i] = dh * delta;")],
    "bwd_row_sum_serial": [("""  for (int w = 1; w < P; w *= 2)
    for (int j = 0; j + w < count; j += 2 * w) vals[(int64_t)j * stride] =
        vals[(int64_t)j * stride] + vals[(int64_t)(j + w) * stride];""",
                            """  for (int j = 1; j < count && P; ++j)
    vals[0] = vals[0] + vals[(int64_t)j * stride];""")],
    "bwd_group_sum_right_to_left": [("""      for (int g = 1; g < G; ++g) {
        accq = accq + DQh[((int64_t)g * Tn + j) * dk + e];
        acck = acck + DKh[((int64_t)g * Tn + j) * dk + e];
      }""", """      if (G > 1) {
        float rq = DQh[((int64_t)(G - 1) * Tn + j) * dk + e];
        float rk = DKh[((int64_t)(G - 1) * Tn + j) * dk + e];
        for (int g = G - 2; g >= 1; --g) {
          rq = DQh[((int64_t)g * Tn + j) * dk + e] + rq;
          rk = DKh[((int64_t)g * Tn + j) * dk + e] + rk;
        }
        accq = accq + rq;
        acck = acck + rk;
      }""")],
    "bwd_final_state_gradient_ignored": [("sh[(int64_t)i * dk + e] = J->dSf ? J->dSf[",
                                          "sh[(int64_t)i * dk + e] = J->dSf ? 0.0f * J->dSf[")],
    # two-level CPR
    "cpr2_B_added_last": [("      float acc = B[(int64_t)i * dk + j];\n      for (int kk = 0; kk < dk; ++kk) acc = fmaf(S[(int64_t)i * dk + kk], A[(int64_t)kk * dk + j], acc);",
                           "      float acc = 0.0f;\n      for (int kk = 0; kk < dk; ++kk) acc = fmaf(S[(int64_t)i * dk + kk], A[(int64_t)kk * dk + j], acc);\n      acc = acc + B[(int64_t)i * dk + j];")],
    "cpr2_transition_absorbs_v": [("row_absorb(A + (int64_t)j * dk, dk, a[t], b[t], 0.0f, kt);",
                                   "row_absorb(A + (int64_t)j * dk, dk, a[t], b[t], v[(int64_t)t * dv + (j % dv)], kt);")],
    "cpr2_outputs_from_next_boundary": [("    /* outputs: the rows restart from the boundary state S */\n    memcpy(R, S, sizeof(float) * st);",
                                         "    /* outputs: the rows restart from the boundary state S */\n    memcpy(R, S, sizeof(float) * st);\n    if (n_tok == C && c > 0) { chunk_transition(kb, vb, ab, bb, C, dk, dv, A, B); boundary_step(S, A, B, R, dv, dk); }")],
    "cpr2_final_always_recurrent": [("const float *fin = (Tn % C == 0) ? S : R;", "const float *fin = R;")],
    "cpr2_decode_cache_slot_shifted": [("const int slot = pos[n] % C;", "const int slot = (pos[n] + 1) % C;")],
    # linear region
    "linear_w_transposed": [("col[k] = load_widened(J->w, (int64_t)k * J->N + n, J->wdtype);",
                             "col[k] = load_widened(J->w, ((int64_t)n * J->K + k) % "
                             "((int64_t)J->K * J->N), J->wdtype);")],
    "linear_x_rows_shifted": [("contract_dot(J->xf + (int64_t)m * J->K, col, J->K);",
                               "contract_dot(J->xf + (int64_t)(m > 0 ? m - 1 : 0) * J->K, col, "
                               "J->K);")],
}


def _apply(src, edits):
    for old, new in edits:
        assert old in src, f"mutation anchor not found: {old!r}"
        src = src.replace(old, new)
    return src


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    mutant_src = tmp_path / f"{name}.c"
    mutant_src.write_text(_apply(src, MUTANTS[name]))
    lib = O.build(force=True, src=str(mutant_src), out=str(tmp_path / f"lib{name}.so"))
    orc = O.Oracle(lib)
    # backward mutants are most quickly caught by the backward pins: try those first
    def family(n):
        for f in ("bwd", "linear", "cpr2"):
            if f in n:
                return f
        return "fwd"

    pins = sorted(oracle_pins.ALL_PINS,
                  key=lambda p: (family(name) != family(p.__name__), p.__name__))
    caught = None
    for pin in pins:
        try:
            pin(orc)
        except (AssertionError, FloatingPointError):
            caught = pin.__name__
            break
    assert caught, f"mutant {name} passed every pin"
