"""The oracle's pins must catch plausible mistakes.  Each case plants one
mistake in a copy of the oracle's C source (never in the product), builds it
with gcc into a temporary library, swaps it in, and checks that at least one
pin from test_oracle.py fails.  CPU only."""
import ctypes as C
import os
import subprocess

import pytest

import oracle
import test_oracle as P

SRC = open(oracle.SRC).read()

MUTATIONS = {
    "silu replaced by the logistic function": (
        "double v = g[m] / (1.0 + exp(-g[m])) * u[m];", "double v = 1.0 / (1.0 + exp(-g[m])) * u[m];",
        [P.test_gate_up_hand_example]),
    "gate and up swapped in the producer": (
        "double v = g[m] / (1.0 + exp(-g[m])) * u[m];", "double v = u[m] / (1.0 + exp(-u[m])) * g[m];",
        [P.test_gate_up_equals_library_products]),
    "bfloat16 rounding truncates": (
        "nearbyint(a / q) * q;", "floor(a / q) * q;",
        [P.test_gate_up_rounding_ties_and_subnormals]),
    "producer tile maxima over the whole batch": (
        "float *pm = pmax + (t / tile) * Mi + m;", "float *pm = pmax + 0 * (t / tile) * Mi + m;",
        [P.test_gate_up_hand_example]),
    "scorer sums instead of max": (
        "                if (v > a)\n                    a = v;\n",
        "                a += v;\n",
        [lambda: P.test_scorer_max_then_scale_equals_scale_then_max("f32")]),
    "ties go to the higher index": (
        "    return (u->pos > v->pos) - (u->pos < v->pos);\n}\n\nstatic int by_pos_asc",
        "    return (u->pos < v->pos) - (u->pos > v->pos);\n}\n\nstatic int by_pos_asc",
        [P.test_select_brute_force_ties]),
    "kept list not re-sorted ascending": (
        "    qsort(it, (size_t)k, sizeof *it, by_pos_asc);\n", "",
        [lambda: P.test_select_count_and_order("tiny")]),
    "keep count rounds down": (
        "? near : ceil(prod);", "? near : floor(prod);",
        [lambda: P.test_keep_count_closed_form(17)]),
    "reduced product drops the first kept slice": (
        "        for (int64_t i = 0; i < k; ++i) {\n            int64_t j = J[i];\n            double xv",
        "        for (int64_t i = 1; i < k; ++i) {\n            int64_t j = J[i];\n            double xv",
        [lambda: P.test_linear_r1_equals_dense("f32"), lambda: P.test_linear_dropped_slice_identity("f32", 4)]),
    "tokens read the wrong tile's slices": (
        "const int32_t *J = idx + (t / tile) * k;", "const int32_t *J = idx + (t % tile) * k;",
        [lambda: P.test_linear_dropped_slice_identity("f32", 2)]),
    "product sign flipped": (
        "acc[m] += xv * (double)elem(wt, wtt, j * ldw + m);", "acc[m] -= xv * (double)elem(wt, wtt, j * ldw + m);",
        [lambda: P.test_linear_r1_equals_dense("bf16")]),
    "logits miss the scale": (
        "l[s] = (double)scale * a;\n                }\n                double mx = l[0];",
        "l[s] = a;\n                }\n                double mx = l[0];",
        [lambda: P.test_attn_full_ratios_equal_textbook(0)]),
    "softmax over kept positions only": (
        "                    for (int64_t i = 0; i < ks; ++i) {\n                        int64_t s = Js[i];\n"
        "                        a += pg[hh * S + s] * (double)bf16_value(V[s * D + d]);\n                    }\n",
        "                    double zk = 0.0;\n                    for (int64_t i = 0; i < ks; ++i)\n"
        "                        zk += pg[hh * S + Js[i]];\n                    for (int64_t i = 0; i < ks; ++i) {\n"
        "                        int64_t s = Js[i];\n"
        "                        a += pg[hh * S + s] / zk * (double)bf16_value(V[s * D + d]);\n                    }\n",
        [lambda: P.test_attn_dropped_position_identity(0)]),
    "position score sums the group's heads": (
        "                    if (pg[hh * S + s] > a)\n                        a = pg[hh * S + s];\n",
        "                    a += pg[hh * S + s];\n",
        [lambda: P.test_attn_selections_brute_force(0)]),
    "block keep count rounds up": (
        "    double p = floor((double)nb * keep);", "    double p = ceil((double)nb * keep);",
        [lambda: P.test_block_keep_count_truncates(100, 0.29, 28)]),
    "blocks interleaved instead of contiguous": (
        "                int64_t j = b * block + e;\n                float a = 0.0f;",
        "                int64_t j = e * nb + b;\n                float a = 0.0f;",
        [lambda: P.test_block_select_brute_force(3)]),
    "value norms ignored": (
        "pis[s] = vn ? a * (double)vn[(b * Hkv + g) * ldv + s] : a;", "pis[s] = a;",
        [lambda: P.test_attn_vn_brute_force(0)]),
    "value norms read with the wrong pitch": (
        "pis[s] = vn ? a * (double)vn[(b * Hkv + g) * ldv + s] : a;",
        "pis[s] = vn ? a * (double)vn[(b * Hkv + g) * S + s] : a;",
        [P.test_attn_vn_strided_equals_packed]),
    "head_dim score reads one head only": (
        "for (int64_t h = h0; h < h0 + gsize; ++h) {\n                    float qa",
        "for (int64_t h = h0; h < h0 + 1; ++h) {\n                    float qa",
        [lambda: P.test_attn_selections_brute_force(0)]),
    "keys read with the wrong stride": (
        "(double)bf16_value(K[j * ldk + s]);\n                    }\n                    l[s]",
        "(double)bf16_value(K[j * S + s]);\n                    }\n                    l[s]",
        [P.test_attn_strided_cache_equals_packed]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path, monkeypatch):
    old, new, pins = MUTATIONS[name]
    assert SRC.count(old) == 1, f"mutation anchor for '{name}' not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(SRC.replace(old, new))
    hdr = os.path.join(os.path.dirname(oracle.SRC), "rmm_oracle.h")
    (tmp_path / "rmm_oracle.h").write_text(open(hdr).read())
    so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", *oracle.CFLAGS, str(src), "-o", str(so), "-lm"])
    monkeypatch.setattr(oracle, "LIB", str(so))
    monkeypatch.setattr(oracle, "_lib", None)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    monkeypatch.setattr(oracle, "_lib", None)
    assert caught > 0, f"no pin caught the planted mistake '{name}'"
