"""Mutation evidence: copies of the oracle with one planted mistake each must
fail at least one pin.  Mistakes are planted in a copy of oracle.c, compiled
with gcc into a temporary library; nothing touches a GPU."""
import ctypes
import os
import subprocess

import pytest

import pins

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "oracle.c")

MUTANTS = {
    "nibble_order": ("(row[j / 2] >> (4 * (j % 2)))", "(row[j / 2] >> (4 * (1 - j % 2)))"),
    "pair_order": ("(row[j / 4] >> (2 * (j % 4)))", "(row[j / 4] >> (2 * (3 - j % 4)))"),
    "zero_point": ("return bits == 4 ? 7.5 : 1.5;", "return bits == 4 ? 8.0 : 2.0;"),
    "weight_sign": ("((double)code_at(row, bits, j) - Z) / Z * s",
                    "(Z - (double)code_at(row, bits, j)) / Z * s"),
    "scale_index": ("j / group]", "(j / 64) % (cols / group)]"),
    "row_stride": ("codes + r * (cols * bits / 8)", "codes + r * (cols / 2)"),
    "silu_sign": ("t / (1.0 + exp(-t))", "t / (1.0 + exp(t))"),
    "bf16_shift": ("(uint32_t)b << 16", "(uint32_t)b << 15"),
    "f16_bias": ("(double)(1024 + m), e - 25)", "(double)(1024 + m), e - 24)"),
    "f16_subnormal": ("ldexp((double)m, -24)", "ldexp((double)(1024 + m), -25)"),
    "combine_overwrite": ("o[j] += r * y[j]", "o[j] = r * y[j]"),
    "hidden_product": ("hidden[i] = oracle_silu(g[i]) * u[i]", "hidden[i] = oracle_silu(u[i]) * g[i]"),
    "routed_slot_weight": ("(double)w[t * top_k + s]", "(double)w[t * top_k]"),
    "routed_slot_index": ("ids[t * top_k + s]", "ids[s * T + t]"),
    "norm_eps_outside": ("1.0 / sqrt(ss / (double)hd + eps)", "1.0 / (sqrt(ss / (double)hd) + eps)"),
    "norm_gain_index": ("xh[d] * inv * (double)w[d]", "xh[d] * inv * (double)w[0]"),
    "rope_pairing": ("i + half]", "i ^ 1]"),
    "rope_sign": ("xh[i] = a * cs - b * sn", "xh[i] = a * cs + b * sn"),
    "rope_frequency": ("-2.0 * (double)i / (double)hd", "-1.0 * (double)i / (double)hd"),
    "gqa_index": ("const long g = h / (n_head / n_kv);", "const long g = h % n_kv;"),
    "attn_scale": ("s[j] = dot / sqrt((double)hd);", "s[j] = dot;"),
    "softmax_denominator": ("att[h * hd + d] = acc / den;", "att[h * hd + d] = acc;"),
    "attn_window": ("ctx_stride, pos + 1, att)", "ctx_stride, pos > 0 ? pos : 1, att)"),
    "append_row": ("v_cache[(g * ctx_stride + pos) * hd + d]", "v_cache[(g * ctx_stride + (pos > 0 ? pos - 1 : 0)) * hd + d]"),
    "append_swap": ("= (float)kn[g * hd + d];", "= (float)v[g * hd + d];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(ORACLE_C).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    (tmp_path / "oracle.h").write_text(open(ORACLE_C.replace(".c", ".h")).read())
    (tmp_path / "oracle.c").write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-o", str(so),
                    str(tmp_path / "oracle.c"), "-lm"], check=True)
    L = pins.bind(ctypes.CDLL(str(so)))
    assert pins.run_core_pins(L), f"mutant {name} passed every pin"
