"""Planted mistakes: each copy of the oracle below carries one plausible bug
(dropped dedup, wrong order, wrong index, unfused or reordered sum, wrong
rounding, flushed subnormals ...).  The pin battery must reject every copy.
A copy runs in a child process, so one that crashes also counts as caught."""

import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

MUTANTS = {
    "no_rank_dedup": ("for (int r = 0; r < R; ++r)\n            if (token_hits_rank(row, k, Epr, r)) o->rank_count[r] += 1;",
                      "for (int j = 0; j < k; ++j) o->rank_count[row[j] / Epr] += 1;"),
    "ranks_descending": ("for (int r = 0; r < R; ++r) {\n            row_of_rank[r] = -1;",
                         "for (int r = R - 1; r >= 0; --r) {\n            row_of_rank[r] = -1;"),
    "tokens_descending": ("for (int t = 0; t < T; ++t) {\n        const int32_t* row = idx + (int64_t)t * k;\n        int slot = 0;",
                          "for (int t = T - 1; t >= 0; --t) {\n        const int32_t* row = idx + (int64_t)t * k;\n        int slot = 0;"),
    "wrong_rank_of_expert": ("o->fan_src[q] = row_of_rank[e / Epr];", "o->fan_src[q] = row_of_rank[e % R];"),
    "fan_dst_descending": ("for (int64_t q = 0; q < (int64_t)T * k; ++q) {\n        int p = o->fan_src[q];",
                           "for (int64_t q = (int64_t)T * k - 1; q >= 0; --q) {\n        int p = o->fan_src[q];"),
    "send_wrong_source": ("memcpy(xr + p * H, x + (int64_t)send_token[p] * H, row_bytes);",
                          "memcpy(xr + p * H, x + (int64_t)(send_token[p] + 1 < d->num_tokens ? send_token[p] + 1 : 0) * H, row_bytes);"),
    "fanout_reads_x": ("memcpy(xe + q * H, xr + (int64_t)fan_src[q] * H, row_bytes);",
                       "memcpy(xe + q * H, x + (int64_t)fan_src[q] % d->num_tokens * H, row_bytes);"),
    "combine_descending_k": ("for (int j = 0; j < k; ++j) {\n                int64_t q = comb_row",
                             "for (int j = k - 1; j >= 0; --j) {\n                int64_t q = comb_row"),
    "combine_drops_last_term": ("for (int j = 0; j < k; ++j) {\n                int64_t q = comb_row",
                                "for (int j = 0; j < k - 1; ++j) {\n                int64_t q = comb_row"),
    "combine_unfused": ("acc = fmaf(w[(int64_t)t * k + j], bf16_to_f32(ye[q * H + h]), acc);",
                        "acc = acc + w[(int64_t)t * k + j] * bf16_to_f32(ye[q * H + h]);"),
    "combine_wrong_gate_index": ("acc = fmaf(w[(int64_t)t * k + j], bf16_to_f32(ye[q * H + h]), acc);",
                                 "acc = fmaf(w[(int64_t)t * k + (k - 1 - j)], bf16_to_f32(ye[q * H + h]), acc);"),
    "combine_start_minus_zero": ("float acc = 0.0f;\n            for (int j = 0; j < k; ++j) {",
                                 "float acc = -0.0f;\n            for (int j = 0; j < k; ++j) {"),
    "round_truncate": ("if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;", ""),
    "round_ties_away": ("if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;",
                        "if (rest >= 0x8000u) keep += 1u;"),
    "dbwd_receiver_descending": ("for (int i = 0; i < D; ++i) {\n                int64_t q = fan_dst[p * D + i];\n                if (q < 0) break;\n                acc = acc + bf16_to_f32(grad_xe[q * H + h]);",
                                 "for (int i = D - 1; i >= 0; --i) {\n                int64_t q = fan_dst[p * D + i];\n                if (q < 0) continue;\n                acc = acc + bf16_to_f32(grad_xe[q * H + h]);"),
    "dbwd_sender_skips_first_rank": ("acc = acc + bf16_to_f32(grad_xr[p * H + h]);",
                                     "acc = i ? acc + bf16_to_f32(grad_xr[p * H + h]) : acc;"),
    "cbwd_wrong_gate": ("const float wj = w[t * k + j];", "const float wj = w[t * k + (k - 1 - j)];"),
    "cbwd_dot_drops_last": ("dot += (double)g * (double)bf16_to_f32(ye[q * H + h]);",
                            "dot += (h + 1 < H) ? (double)g * (double)bf16_to_f32(ye[q * H + h]) : 0.0;"),
    "partial_gate_by_slot": ("for (int64_t i = 0; i < Tk; ++i) gate[comb_row[i]] = w[i];",
                             "for (int64_t i = 0; i < Tk; ++i) gate[i] = w[i];"),
    "partial_truncates": ("partial[p * H + h] = f32_to_bf16_rne(acc);",
                          "{ uint32_t u_; memcpy(&u_, &acc, 4); partial[p * H + h] = (uint16_t)(u_ >> 16); }"),
    "partial_f32_rounded_to_bf16": ("            partial[p * H + h] = sum;",
                                    "            partial[p * H + h] = bf16_to_f32(f32_to_bf16_rne(sum));"),
    "partial_f32_unfused": ("sum = fmaf(g[q], bf16_to_f32(ye[q * H + h]), sum);",
                            "sum = sum + g[q] * bf16_to_f32(ye[q * H + h]);"),
    "partial_f32_ranks_descending": ("for (int r = 0; r < KR; ++r) {\n                const int64_t p = tok_rank_row[t * KR + r];\n                if (p < 0) break;",
                                     "for (int r = KR - 1; r >= 0; --r) {\n                const int64_t p = tok_rank_row[t * KR + r];\n                if (p < 0) continue;"),
    "round_nan_to_inf": ("if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);", ""),
    "round_nan_drops_sign": ("if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);",
                             "if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x7fffu) | 0x0040u);"),
    "round_nan_not_quieted": ("if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);",
                              "if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(u >> 16);"),
    "round_saturates": ("    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;\n    return (uint16_t)keep;",
                        "    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;\n"
                        "    if ((keep & 0x7fffu) == 0x7f80u && (u & 0x7fffffffu) < 0x7f800000u) keep -= 1u;\n"
                        "    return (uint16_t)keep;"),
    "flush_subnormals": ("uint32_t u = (uint32_t)b << 16;\n    float f;",
                         "uint32_t u = (uint32_t)b << 16;\n    if ((u & 0x7f800000u) == 0) u &= 0x80000000u;\n    float f;"),
}

RUNNER = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, pins
orc = oracle.Oracle({lib!r})
try:
    pins.run_battery(orc)
except AssertionError as e:
    print("caught:", str(e)[:200]); sys.exit(3)
sys.exit(0)
"""


def _build_variant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    oracle.build(str(path), str(lib))
    return str(lib)


def _run(lib):
    code = RUNNER.format(root=os.path.dirname(HERE), tests=HERE, lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)


def test_unmodified_oracle_passes_battery(tmp_path):
    lib = tmp_path / "libclean.so"
    oracle.build(SRC, str(lib))
    r = _run(str(lib))
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    r = _run(_build_variant(tmp_path, name, old, new))
    assert r.returncode != 0, f"planted mistake {name} survived the pins"
