"""The oracle's pins must fail on plausible mistakes.

Each case copies oracle/oracle.c to a temporary directory, plants one
mistake (a wrong tie rule, a dropped term, a transposed operand, ...),
builds it, and runs the oracle pin tests against the planted copy in a
child process.  Every planted copy must fail at least one pin.  Nothing
here touches the product path or a GPU.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PIN_FILES = [
    "tests/test_oracle_mask.py",
    "tests/test_oracle_gamma_ternary.py",
    "tests/test_oracle_actq_fwd.py",
    "tests/test_oracle_bwd_pack.py",
    "tests/test_oracle_bf16_y.py",
]

MUTANTS = {
    "tie_to_higher_index": ("ai == aj && i < j", "ai == aj && i > j"),
    "keep_one_too_many": ("if (rank < n)", "if (rank <= n)"),
    "subnormal_scale": ("*shift = 0; }", "*shift = 1; }"),
    "normal_scale": ("*shift = (int)e - 1;", "*shift = (int)e;"),
    "round_half_up": ("if (half && (sticky || (sig & 1u))) sig += 1;", "if (half) sig += 1;"),
    "ternary_half_to_one": ("2.0 * fabs(w) > gamma", "2.0 * fabs(w) >= gamma"),
    "ternary_ignores_mask": ("if (mask_bit(mask, k, r, c) && gamma", "if (gamma"),
    "act_round_half_away": ("q = nearbyint(", "q = round("),
    "act_scale_128": ("scale[t] = a / 127.0;", "scale[t] = a / 128.0;"),
    "fwd_transposed_weights": ("(int64_t)j->T[r * j->k + c]", "(int64_t)j->T[c * j->n_out + r]"),
    "fwd_drops_token_scale": ("(double)s * j->gamma * j->scale[t]", "(double)s * j->gamma"),
    "dx_drops_gamma": ("j->dX[t * j->k + c] = j->gamma * s;", "j->dX[t * j->k + c] = s;"),
    "dw_drops_token_scale": ("j->scale[t] *", "1.0 *"),
    "pack_high_sign_order": ("sign |= 1u << (s - 1 - nhi);", "sign |= 1u << (nlo + nhi);"),
    "unpack_high_sign_order": ("((sign >> (s - 1 - nhi)) & 1u)", "((sign >> (nlo + nhi)) & 1u)"),
    "layout_group_roles_swapped": ("int h = g / 8, q = (g % 8) / 2, e = g % 2;",
                                   "int h = g % 2, q = (g % 8) / 2, e = g / 8;"),
    "layout_chunks_transposed": ("* 64 + r16 + 16 * q;", "* 64 + q + 4 * r16;"),
    "sp24_index_bits_reversed": ("idx |= (uint32_t)pos[sl] << (2 * e);", "idx |= (uint32_t)pos[sl] << (30 - 2 * e);"),
    "sp24_value_codes_linear": ("val |= code << (8 * (e % 4) + 2 * (e / 4));", "val |= code << (2 * e);"),
    "sp24_one_nonzero_slot": ("else { pos[1] = pos[0]; pos[0] = 0; }", "else { pos[1] = pos[0] == 3 ? 2 : 3; }"),
    "sp24_lane_groups_swapped": ("(strip * nkb + kb) * 64 + rr % 16 + 16 * q", "(strip * nkb + kb) * 64 + q + 4 * (rr % 16)"),
    "bf16y_scale_product_in_binary32": ("float g32 = (float)(gamma * (double)s32);", "float g32 = (float)gamma * s32;"),
    "bf16y_rounded_from_binary64": ("float y32 = a32 * g32;", "float y32 = (float)((double)(int32_t)s * gamma * scale[t]);"),
    "bf16y_truncated": ("            Y[t * n_out + r] = nearest_bf16(y32);",
                        "            { uint32_t u; memcpy(&u, &y32, 4); Y[t * n_out + r] = (uint16_t)(u >> 16); }"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("no C compiler")
    old, new = MUTANTS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert src.count(old) >= 1, "mutation site vanished: update the planted mistake"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new, 1))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared",
                    "-o", str(lib), str(mut), "-lpthread", "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu"] + PIN_FILES, cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake '{name}' passed every pin:\n{r.stdout[-2000:]}"
