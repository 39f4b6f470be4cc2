"""Planted mistakes in the CPU oracle must be caught by its pins.

Each case edits one line of a temporary copy of ``oracle/bq_oracle.c`` (a wrong
constant, a wrong rounding direction, a wrong index, a wrong order, a wrong
sign), builds it with the oracle's own flags, points the oracle wrapper at the
mutant library and runs the named pin tests, which must fail.  Everything runs
on the CPU; the real oracle library is restored afterwards.
"""
from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

MUTANTS = [
    ("divisor 128 instead of 127", "#define I8_QMAX 127.0f", "#define I8_QMAX 128.0f",
     ["test_i8_worked_examples"]),
    ("ties away from zero in INT8 rounding", "float r = rintf(t);", "float r = roundf(t);",
     ["test_i8_worked_examples"]),
    ("bf16 ties away from zero", "(lo == 0x8000u && (hi & 1u))", "(lo == 0x8000u)",
     ["test_bf16_rounding_matches_torch_structured_sweep"]),
    ("ring chunk index off by one", "int c = mod(r - 1 - k, W);", "int c = mod(r - k, W);",
     ["test_ring_allreduce_exact_sums_and_canonical_payload"]),
    ("A2A sources summed in reverse order", "for (int s = 0; s < nsrc; s++) {",
     "for (int s = nsrc - 1; s >= 0; s--) {",
     ["test_accum_respects_array_order_and_rounds_each_product"]),
    ("E8M0 rounds an exact power of two up", "int e = (f == 0.5f) ? k - 1 : k;", "int e = k;",
     ["test_mx_worked_examples"]),
    ("E8M0 by the OCP floor rule, floor(log2 amax) - 8", "    int e = (f == 0.5f) ? k - 1 : k;",
     "    int e = k; { int ka; (void)frexpf(amax, &ka); e = ka - 9; (void)f; }",
     ["test_mx_worked_examples", "test_e8m0_exhaustive_over_bf16_amax"]),
    ("E4M3 ties always upward", "code = (lo % 2 == 0) ? lo : hi;", "code = hi;",
     ["test_e4m3_encode_midpoints_and_random_fp32"]),
    ("hop subtracts the local partial", "sum[i] = deq + loc;", "sum[i] = deq - loc;",
     ["test_ring_hop_bruteforce_and_identities"]),
    ("zero block stores scale 1", "*scale = 0.0f;", "*scale = 1.0f;",
     ["test_i8_worked_examples"]),
    ("MX dequant exponent sign flipped", "return ldexpf(orc_e4m3_decode(code), (int)byte - 127);",
     "return ldexpf(orc_e4m3_decode(code), 127 - (int)byte);",
     ["test_mx_dequant_matches_torch_decode"]),
    ("E4M3-b128 divides by 127", "float s = amax / E4M3_MAX;", "float s = amax / I8_QMAX;",
     ["test_e4m3_b128_worked_examples"]),
    ("MX hop subtracts the local partial", "sums[i] = dq + lp;", "sums[i] = dq - lp;",
     ["test_mx_ring_hop_bruteforce_and_identities"]),
    ("MX accumulate in reverse source order", "for (int src = 0; src < nsrc; ++src) {",
     "for (int src = nsrc - 1; src >= 0; --src) {", ["test_mx_accum_order_and_bruteforce"]),
    ("MX ring chunk index off by one", "int chunk = mod(r - 1 - k, W);",
     "int chunk = mod(r - k, W);", ["test_mx_ring_allreduce_exact_sums_and_canonical_payload"]),
    ("E8M0 of an underflowed quotient left at byte 127", "if (d == 0.0f)", "if (d < 0.0f)",
     ["test_e8m0_quotient_underflow_saturates_to_the_smallest_byte"]),
    ("MX hop rounds the sums to bf16 first", "            sums[i] = dq + lp;",
     "            sums[i] = orc_bf16_to_f32(orc_f32_to_bf16(dq + lp));",
     ["test_mx_ring_hop_bruteforce_and_identities"]),
    ("INT8 hop rounds the sums to bf16 first", "            sum[i] = deq + loc;",
     "            sum[i] = orc_bf16_to_f32(orc_f32_to_bf16(deq + loc));",
     ["test_ring_hop_bruteforce_and_identities"]),
    ("INT8 hop fuses the dequantize into the add",
     "            float deq = (float)q_in[b * BLK + i] * s_in[b];\n"
     "            float loc = orc_bf16_to_f32(local[b * BLK + i]);\n            sum[i] = deq + loc;",
     "            float loc = orc_bf16_to_f32(local[b * BLK + i]);\n"
     "            sum[i] = fmaf((float)q_in[b * BLK + i], s_in[b], loc);",
     ["test_ring_hop_bruteforce_and_identities"]),
    ("A2A accumulate fuses multiply and add",
     "            float term = (float)q[s][i] * scale[s][i / BLK];\n            acc = acc + term;",
     "            acc = fmaf((float)q[s][i], scale[s][i / BLK], acc);",
     ["test_accum_respects_array_order_and_rounds_each_product"]),
    ("materialization truncates to bf16",
     "        float v = (float)q[i] * scale[i / BLK];\n        y[i] = orc_f32_to_bf16(v);",
     "        float v = (float)q[i] * scale[i / BLK];\n"
     "        { uint32_t u_; memcpy(&u_, &v, 4); y[i] = (uint16_t)(u_ >> 16); }",
     ["test_i8_dequant_matches_torch_products"]),
    ("E4M3-b128 zero block stores scale 1", "            scale[b] = 0.0f;", "            scale[b] = 1.0f;",
     ["test_e4m3_b128_worked_examples"]),
    ("A2A requantizes the binary32 sum, not the bf16 sum",
     "        orc_quant_i8(red + j * m, m, q_final + j * m, s_final + j * mb);",
     "        for (int64_t b = 0; b < mb; b++) {\n"
     "            float f32s[BLK];\n"
     "            for (int i = 0; i < BLK; i++) {\n"
     "                float acc = 0.0f;\n"
     "                for (int k = 0; k < W; k++)\n"
     "                    acc = acc + (float)qp[k][b * BLK + i] * sp[k][b];\n"
     "                f32s[i] = acc;\n"
     "            }\n"
     "            quant_block_f32(f32s, q_final + j * m + b * BLK, s_final + j * mb + b);\n"
     "        }",
     ["test_a2a_requantizes_the_bf16_sum"]),
    ("MX A2A requantizes the binary32 sum, not the bf16 sum",
     "        quant_mx_flat(red + j * m, m, v_final + j * m, e_final + j * mg);",
     "        for (int64_t g = 0; g < mg; g++) {\n"
     "            float f32s[MXG];\n"
     "            for (int i = 0; i < MXG; i++) {\n"
     "                float acc = 0.0f;\n"
     "                for (int r = 0; r < W; r++)\n"
     "                    acc = acc + mx_value(vp[r][g * MXG + i], ep[r][g]);\n"
     "                f32s[i] = acc;\n"
     "            }\n"
     "            quant_group_mx(f32s, v_final + j * m + g * MXG, e_final + j * mg + g);\n"
     "        }",
     ["test_mx_a2a_reduce_is_accumulate_then_quantize_then_materialize"]),
    ("A2A owner materializes from its bf16 sum, not the payload",
     "            orc_dequant_i8(q_out + j * seg_n, s_out + j * sb, seg_n, y_out[j]);",
     "            memcpy(y_out[j], sum, (size_t)seg_n * sizeof(uint16_t));",
     ["test_a2a_reduce_is_accumulate_then_quantize_then_materialize"]),
    ("binary16 exponent bias off by one","ldexpf((float)(1024 + man), ex - 25)",
     "ldexpf((float)(1024 + man), ex - 24)", ["test_f16_decode_exhaustive_matches_numpy"]),
    ("binary16 subnormal step 2^-23", "ldexpf((float)man, -24)", "ldexpf((float)man, -23)",
     ["test_f16_decode_exhaustive_matches_numpy"]),
    ("A2A requantizes only the first shard", "for (int j = 0; j < W; j++) {\n        for (int s = 0; s < W; s++) {",
     "for (int j = 0; j < 1; j++) {\n        for (int s = 0; s < W; s++) {",
     ["test_a2a_requantizes_the_bf16_sum"]),
    ("staged slice scales at column off/128",
     "orc_quant_mx(x, rows, cols, ldx, v + col_off, ldv, e8m0 + col_off / MXG, lds);",
     "orc_quant_mx(x, rows, cols, ldx, v + col_off, ldv, e8m0 + col_off / 128, lds);",
     ["test_mx_slices_equal_concatenation_and_leave_the_rest_untouched"]),
    ("binary16 staged slice values at column off/2",
     "orc_quant_mx_f16(x, rows, cols, ldx, v + col_off, ldv, e8m0 + col_off / MXG, lds);",
     "orc_quant_mx_f16(x, rows, cols, ldx, v + col_off / 2, ldv, e8m0 + col_off / MXG, lds);",
     ["test_mx_f16_slices_equal_concatenation_and_leave_the_rest_untouched"]),
    ("MX dequant reads the scale of column c/128", "e8m0[r * lds + c / MXG]",
     "e8m0[r * lds + c / 128]", ["test_mx_dequant_matches_torch_decode"]),
    ("binary16 rows decoded as bf16", "quant_mx_rows(orc_f16_to_f32, x",
     "quant_mx_rows(orc_bf16_to_f32, x", ["test_mx_f16_quant_bruteforce_rows"]),
    ("E4M3 subnormal step 2^-10", "mag = ldexpf((float)man, -9);", "mag = ldexpf((float)man, -10);",
     ["test_e4m3_decode_all_codes"]),
    ("E4M3-b128 dequant uses the first block's scale",
     "float val = orc_e4m3_decode(v[i]) * scale[i / BLK];",
     "float val = orc_e4m3_decode(v[i]) * scale[0];", ["test_e4m3_b128_bruteforce_and_dequant"]),
    ("INT8 quotients not clamped to [-127, 127]",
     "        if (r > I8_QMAX)\n            r = I8_QMAX;\n        if (r < -I8_QMAX)\n            r = -I8_QMAX;\n",
     "",
     ["test_ring_hop_clamps_the_quotients_of_few_bit_subnormal_scales",
      "test_ring_allreduce_of_cancelling_partials_clamps_like_the_brute_force"]),
    ("MFMA layout swaps the K step and the 32-column block",
     "    int64_t lane = 16 * block + row % 16; /* the lane that supplies this byte */",
     "    int64_t lane = 16 * step + row % 16; step = block;",
     ["test_mx_mfma_layout_worked_offsets", "test_mx_mfma_layout_is_lane_words_of_k_steps"]),
    ("MFMA layout orders tiles by row block first",
     "    int64_t tile = kgroup * row_blocks + rblock;",
     "    int64_t tile = rblock * row_blocks + kgroup;",
     ["test_mx_mfma_layout_worked_offsets", "test_mx_mfma_layout_is_lane_words_of_k_steps"]),
    ("MFMA layout puts a row's four blocks in adjacent lanes",
     "    int64_t lane = 16 * block + row % 16; /* the lane that supplies this byte */",
     "    int64_t lane = 4 * (row % 16) + block;",
     ["test_mx_mfma_layout_worked_offsets", "test_mx_mfma_layout_is_lane_words_of_k_steps"]),
    ("E4M3 saturates to the NaN code", "return (uint8_t)(sign | 0x7E);",
     "return (uint8_t)(sign | 0x7F);", ["test_e4m3_encode_signed_zero_and_saturation"]),
]


@pytest.fixture
def mutant_lib(tmp_path, monkeypatch):
    src = open(oracle._SRC).read()

    def build(old: str, new: str) -> None:
        assert src.count(old) == 1, f"mutation site not unique: {old!r}"
        d = tmp_path / "m"
        d.mkdir(exist_ok=True)
        (d / "bq_oracle.h").write_text(open(oracle._HDR).read())
        (d / "bq_oracle.c").write_text(src.replace(old, new))
        so = d / "liboracle_mutant.so"
        subprocess.run(["gcc", *oracle.CFLAGS, str(d / "bq_oracle.c"), "-o", str(so), "-lm"],
                       check=True)
        monkeypatch.setattr(oracle, "_LIB", str(so))
        monkeypatch.setattr(oracle, "_SRC", str(d / "bq_oracle.c"))
        monkeypatch.setattr(oracle, "_HDR", str(d / "bq_oracle.h"))
        monkeypatch.setattr(oracle, "_lib", None)

    yield build
    oracle._lib = None


@pytest.mark.parametrize("desc,old,new,tests", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(mutant_lib, desc, old, new, tests, tmp_path):
    mutant_lib(old, new)
    for name in tests:
        fn = getattr(pins, name)
        kwargs = {}
        if "W" in fn.__code__.co_varnames[: fn.__code__.co_argcount]:
            kwargs["W"] = 4
        with pytest.raises(AssertionError):
            fn(**kwargs)


def _mm_with_values(values_fn):
    def mm(xv, xe, wv, we):
        X, Wt = values_fn(xv, xe), values_fn(wv, we)
        return X @ Wt.T, np.abs(X) @ np.abs(Wt).T
    return mm


def _values_exponent_off_by_one(v, e):
    table = np.array([oracle.lib().orc_e4m3_decode(c) for c in range(256)], np.float64)
    return table[v] * np.ldexp(1.0, np.repeat(e.astype(np.int64) - 126, 32, axis=1))[:, :v.shape[1]]


def _values_group_of_64(v, e):
    table = np.array([oracle.lib().orc_e4m3_decode(c) for c in range(256)], np.float64)
    return table[v] * np.ldexp(1.0, np.repeat(e[:, ::2].astype(np.int64) - 127, 64, axis=1))


def _mm_sums_magnitudes(xv, xe, wv, we):
    X, Wt = oracle.mx_values_f64(xv, xe), oracle.mx_values_f64(wv, we)
    return np.abs(X) @ np.abs(Wt).T, np.abs(X) @ np.abs(Wt).T


PY_MUTANTS = [
    ("GEMM scale exponent off by one", _mm_with_values(_values_exponent_off_by_one),
     ["test_mm_mx_worked_cases", "test_mm_mx_bruteforce_tiny"]),
    ("GEMM scale groups of 64 columns", _mm_with_values(_values_group_of_64),
     ["test_mm_mx_worked_cases", "test_mm_mx_bruteforce_tiny"]),
    ("GEMM drops the signs", _mm_sums_magnitudes,
     ["test_mm_mx_worked_cases", "test_mm_mx_bruteforce_tiny"]),
]


@pytest.mark.parametrize("desc,fn,tests", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_pins_catch_planted_python_mistake(monkeypatch, desc, fn, tests):
    monkeypatch.setattr(oracle, "mm_mx", fn)
    for name in tests:
        with pytest.raises(AssertionError):
            getattr(pins, name)()
