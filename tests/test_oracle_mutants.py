"""The pins have teeth: plant a plausible mistake in a copy of the oracle's C
source (on the CPU), build it, run the pins against it, and require that at
least one pin fails.  The real oracle is restored after each case."""

from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import pinlib
from gen import config_inputs, random_case

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")

# The two LL combines share their first lines; these tails tell them apart.
_LL_BF16_TAIL = ("            float w = topk_weights[t * K + k];\n"
                 "            int64_t cell = ((e % epr) * R + e / epr) * num_slots + s;\n"
                 "            for (int64_t h = 0; h < H; ++h)\n"
                 "                acc[h] = fmaf(w, bf16_to_f32")
_LL_FP8_TAIL = ("            float w = topk_weights[t * K + k];\n"
                "            int64_t cell = ((e % epr) * R + e / epr) * num_slots + s;\n"
                "            for (int64_t h = 0; h < H; ++h) {\n"
                "                float v = oracle_e4m3_to_f32")

# The head of the bf16 LL combine's slot loop (shared with the FP8 one).
_LL_BF16_HEAD = ("        for (int64_t k = 0; k < K; ++k) {\n"
                 "            int64_t e = topk_idx[t * K + k];\n"
                 "            int64_t s = slot[t * K + k];\n"
                 "            if (e < 0 || s < 0 || s >= num_slots)\n"
                 "                continue;\n"
                 "            if (combine_mask != NULL && combine_mask[e / epr] != 0)\n"
                 "                continue;\n")

# The LL slot assignment's loops, token-major as the reading fixes.
_LL_SLOT_LOOPS = ("    for (int64_t t = 0; t < T; ++t) {\n        for (int64_t k = 0; k < K; ++k) {\n"
                  "            int64_t e = topk_idx[t * K + k];\n"
                  "            if (!ll_live(e, E, epr, rank_mask)) {")


def _biases_first():
    """The combine's rank sum followed by its bias additions, and the same
    code with the bias additions moved before the rank sum."""
    src = open(SRC).read()
    zero = "        for (int64_t h = 0; h < H; ++h)\n            acc[h] = 0.0f;\n"
    i0 = src.index(zero + "        for (int64_t r = 0; r < R; ++r) {")
    tail = "                acc[h] += bf16_to_f32(bias1[t * H + h]);\n"
    i1 = src.index(tail, i0) + len(tail)
    block = src[i0:i1]
    cut = block.index("        if (bias0 != NULL)")
    return block, zero + block[cut:] + block[len(zero):cut]


# (name, original text, planted text): each original must occur exactly once.
MUTANTS = [
    ("bf16 ties away from zero", "u += 0x7fffu + lsb;", "u += 0x8000u;"),
    ("bf16 truncation", "u += 0x7fffu + lsb;", "u += 0u * lsb;"),
    ("rank of an expert by modulo", "is_token_in_rank[t * R + e / epr] = 1;",
     "is_token_in_rank[t * R + e % R] = 1;"),
    ("channel end one channel early", "int64_t e = (c + 1) * per;", "int64_t e = c * per;"),
    ("inclusive recv channel prefix",
     "recv_channel_prefix_matrix[r * C + c] = c > 0 ? channel_prefix_matrix[r * C + c - 1] : 0;",
     "recv_channel_prefix_matrix[r * C + c] = channel_prefix_matrix[r * C + c];"),
    ("send_head counted from one", "send_head[t * R + r] = pos++;", "send_head[t * R + r] = ++pos;"),
    ("expert counts skip the last slot", "for (int64_t k = 0; k < K; ++k) {\n            int64_t e = topk_idx[t * K + k];\n            if (e < 0)\n                continue; /* masked slot",
     "for (int64_t k = 0; k < K - 1; ++k) {\n            int64_t e = topk_idx[t * K + k];\n            if (e < 0)\n                continue; /* masked slot"),
    ("local expert id off by rank", "recv_topk_idx[row * K + k] = mine ? e - r * epr : -1;",
     "recv_topk_idx[row * K + k] = mine ? e - r : -1;"),
    ("non-local weight kept", "recv_topk_weights[row * K + k] = mine ? topk_weights[t * K + k] : 0.0f;",
     "recv_topk_weights[row * K + k] = topk_weights[t * K + k];"),
    ("combine drops the last rank", "            if (p < 0)\n                continue;\n            int64_t row = (r > 0 ? rank_prefix_matrix[r - 1] : 0) + p;\n            for (int64_t h = 0; h < H; ++h)",
     "            if (p < 0 || r == R - 1)\n                continue;\n            int64_t row = (r > 0 ? rank_prefix_matrix[r - 1] : 0) + p;\n            for (int64_t h = 0; h < H; ++h)"),
    ("combine weights from slot 0", "w += recv_topk_weights[row * K + k];",
     "w += recv_topk_weights[row * K];"),
    ("combine bias added twice", "acc[h] += bf16_to_f32(bias0[t * H + h]);",
     "acc[h] += 2.0f * bf16_to_f32(bias0[t * H + h]);"),
    ("LL slot counter shared by a rank's experts", "            slot[t * K + k] = count[e]++;",
     "            slot[t * K + k] = count[e / epr * epr]++;"),
    ("LL rank mask ignored", "if (rank_mask != NULL && rank_mask[e / epr] != 0)",
     "if (rank_mask != NULL && rank_mask[e / epr] != 0 && 0)"),
    ("LL counts transposed", "counts[(e % epr) * R + e / epr] = cnt[e];", "counts[e] = cnt[e];"),
    ("LL combine terms scaled by 1 + 1e-7", "acc[h] = fmaf(w, bf16_to_f32(buf[cell * H + h]), acc[h]);",
     "acc[h] = fmaf(w * 1.0000001f, bf16_to_f32(buf[cell * H + h]), acc[h]);"),
    ("combine rows scaled by 1 + 1e-7", "acc[h] += bf16_to_f32(y[row * H + h]);",
     "acc[h] += bf16_to_f32(y[row * H + h]) * 1.0000001f;"),
    ("e4m3 ties away", "double mi = rint((2.0 * fr - 1.0) * 8.0);",
     "double mi = round((2.0 * fr - 1.0) * 8.0);"),
    ("e4m3 no saturation", "        return sign | 0x7E;\n    if (a < ldexp",
     "        return sign | 0x7F;\n    if (a < ldexp"),
    ("fp8 scale inverted", "float sinv = 448.0f / amax;", "float sinv = amax / 448.0f;"),
    ("fp8 amax floor dropped", "if (amax < 1e-4f)\n                amax = 1e-4f;",
     "if (amax < 0.0f)\n                amax = 1e-4f;"),
    ("reduce grads from zero", "acc[p] = bf16_to_f32(expert_grads[e * P + p]);", "acc[p] = 0.0f;"),
    ("layout rank mask ignored", "if (rank_masked(rank_mask, e / epr))",
     "if (0 && rank_masked(rank_mask, e / epr))"),
    ("combine rank mask ignored", "            if (rank_masked(rank_mask, r))\n                continue;",
     "            if (0)\n                continue;"),
    ("combine weights ignore the rank mask", "if (p < 0 || rank_masked(rank_mask, r))",
     "if (p < 0)"),
    ("LL combine-time mask ignored",
     "if (combine_mask != NULL && combine_mask[e / epr] != 0)\n                continue;\n" + _LL_BF16_TAIL,
     "if (combine_mask != NULL && combine_mask[e / epr] != 0 && 0)\n                continue;\n"
     + _LL_BF16_TAIL),
    ("LL combine cell with rank and local expert swapped", _LL_BF16_TAIL,
     _LL_BF16_TAIL.replace("((e % epr) * R + e / epr)", "((e / epr) * epr + e % epr)")),
    ("fp8 combine-time mask ignored",
     "if (combine_mask != NULL && combine_mask[e / epr] != 0)\n                continue;\n" + _LL_FP8_TAIL,
     "if (combine_mask != NULL && combine_mask[e / epr] != 0 && 0)\n                continue;\n"
     + _LL_FP8_TAIL),
    ("fp8 amax always from the first block",
     "for (int64_t h = b * 128; h < (b + 1) * 128; ++h) {\n                float v = fabsf",
     "for (int64_t h = 0; h < 128; ++h) {\n                float v = fabsf"),
    ("e4m3 subnormals in units of 2^-8", "double q = rint(a * 512.0);", "double q = rint(a * 256.0);"),
    ("e4m3 exponent bias 8", "int code = ((e + 7) << 3) | (int)mi;", "int code = ((e + 8) << 3) | (int)mi;"),
    ("combine bias1 ignored", "if (bias1 != NULL)", "if (bias1 != NULL && 0)"),
    ("reduce grads keeps only the last replica",
     "acc[p] += bf16_to_f32(redundant_grads[j * P + p]);",
     "acc[p] = bf16_to_f32(expert_grads[e * P + p]) + bf16_to_f32(redundant_grads[j * P + p]);"),
    ("fp8 combine ignores the scales",
     "float v = oracle_e4m3_to_f32(q[cell * H + h]) * scale[cell * nb + h / 128];",
     "float v = oracle_e4m3_to_f32(q[cell * H + h]);"),
    ("fp8 combine uses the first block's scale",
     "float v = oracle_e4m3_to_f32(q[cell * H + h]) * scale[cell * nb + h / 128];",
     "float v = oracle_e4m3_to_f32(q[cell * H + h]) * scale[cell * nb];"),
    ("prefetch ignores mapping", "memcpy(redundant_weights + j * P, expert_weights + e * P,",
     "memcpy(redundant_weights + j * P, expert_weights + j % E * P,"),
    ("recv_src_idx without the segment base",
     "recv_src_idx[base + send_head[t * R + r]] = (int32_t)t;",
     "recv_src_idx[send_head[t * R + r]] = (int32_t)t;"),
    ("exclusive rank prefix", "        acc += num_tokens_per_rank[r];\n        rank_prefix_matrix[r] = acc;",
     "        rank_prefix_matrix[r] = acc;\n        acc += num_tokens_per_rank[r];"),
    ("membership counted per slot", "is_token_in_rank[t * R + e / epr] = 1;",
     "is_token_in_rank[t * R + e / epr] += 1;"),
    ("combine sums ranks in descending order",
     "        for (int64_t r = 0; r < R; ++r) {\n            int32_t p = send_head[t * R + r];\n"
     "            if (rank_masked(rank_mask, r))",
     "        for (int64_t r = R - 1; r >= 0; --r) {\n            int32_t p = send_head[t * R + r];\n"
     "            if (rank_masked(rank_mask, r))"),
    ("LL combine sums slots in descending order", _LL_BF16_HEAD + _LL_BF16_TAIL,
     _LL_BF16_HEAD.replace("for (int64_t k = 0; k < K; ++k)", "for (int64_t k = K - 1; k >= 0; --k)")
     + _LL_BF16_TAIL),
    ("reduce grads sums replicas in descending order",
     "        for (int64_t j = 0; j < n_rep; ++j)\n            if (mapping[j] == e)\n",
     "        for (int64_t j = n_rep - 1; j >= 0; --j)\n            if (mapping[j] == e)\n"),
    ("LL src_info holds the slot", "            src_info[cell] = (int32_t)t;",
     "            src_info[cell] = (int32_t)s;"),
    ("LL counts capped at capacity", "        counts[(e % epr) * R + e / epr] = cnt[e];",
     "        counts[(e % epr) * R + e / epr] = cnt[e] < num_slots ? cnt[e] : (int32_t)num_slots;"),
    ("e4m3 sign dropped", "    uint8_t sign = signbit(f) ? 0x80 : 0;", "    uint8_t sign = 0;"),
    ("LL combine without fma", "acc[h] = fmaf(w, bf16_to_f32(buf[cell * H + h]), acc[h]);",
     "acc[h] = acc[h] + w * bf16_to_f32(buf[cell * H + h]);"),
    ("fp8 LL combine without fma", "acc[h] = fmaf(w, v, acc[h]);", "acc[h] = acc[h] + w * v;"),
    ("biases before the rank sum",) + _biases_first(),
    ("LL slots in slot-major order", _LL_SLOT_LOOPS,
     _LL_SLOT_LOOPS.replace("    for (int64_t t = 0; t < T; ++t) {\n        for (int64_t k = 0; k < K; ++k) {",
                            "    for (int64_t k = 0; k < K; ++k) {\n        for (int64_t t = 0; t < T; ++t) {")),
    ("channel size rounded down", "    int64_t per = (T + C - 1) / C;",
     "    int64_t per = T / C > 0 ? T / C : 1;"),
    ("e4m3 NaN saturates", "    if (isnan(f))\n        return 0x7F;", "    if (isnan(f))\n        return 0x7E;"),
    ("bf16 NaN not special-cased",
     "    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)\n",
     "    if (0)\n"),
    ("expert counts ignore the rank mask",
     "            if (rank_masked(rank_mask, e / epr))\n"
     "                continue; /* expert on a masked rank: as a masked slot */\n"
     "            num_tokens_per_expert[e] += 1;",
     "            num_tokens_per_expert[e] += 1;\n"
     "            if (rank_masked(rank_mask, e / epr))\n"
     "                continue; /* expert on a masked rank: as a masked slot */"),
]


def quick_pins():
    """A fast subset of the pins (each a few seconds at most)."""
    pinlib.check_hand_example()
    pinlib.check_bruteforce_exhaustive(T=2, K=2, E=4, Rs=(1, 2, 4))
    pinlib.check_bruteforce_dispatch_combine(seed=1, cases=60)
    pinlib.check_layout_invariants(random_case(2, 257, 8, 24, 5, 6, 7, mask=0.2, dup=0.3))
    pinlib.check_special_cases()
    pinlib.check_identity_combine(random_case(5, 120, 16, 16, 6, 4, 3, mask=0.25, dup=0.4))
    pinlib.check_combine_fp64(0)
    pinlib.check_ll(random_case(3, 40, 16, 8, 4, 2, 1, mask=0.2, dup=0.5, slots=12))
    pinlib.check_ll(config_inputs(3))
    pinlib.check_ll_fp64(0)
    pinlib.check_bf16_edges()
    pinlib.check_bf16_patterns(step=(1 << 14) + 1, chunk=1 << 14)
    m = np.array([0, 1, 0, 0, 1, 1, 0, 0], np.int32)
    pinlib.check_ll_rank_mask(random_case(8, 50, 24, 16, 4, 8, 1, mask=0.1, dup=0.3, slots=60), m)
    pinlib.check_ll_mask_extremes(random_case(9, 30, 16, 8, 3, 4, 1, slots=30))
    pinlib.check_combine_bias(0)
    pinlib.check_layout_rank_mask(random_case(21, 60, 8, 24, 5, 6, 4, mask=0.1, dup=0.2),
                                  np.array([0, 1, 0, 1, 0, 0], np.int32))
    pinlib.check_combine_rank_mask(0)
    pinlib.check_lb_ops(0)
    pinlib.check_e4m3()
    pinlib.check_ll_fp8(random_case(4, 40, 256, 16, 4, 4, 1, mask=0.2, slots=40))
    pinlib.check_ll_fp8(pinlib.fp8_edge_case())
    pinlib.check_tie_rounding()
    pinlib.check_sum_order()
    pinlib.check_fma_and_bias_order()
    pinlib.check_ll_combine_fp8(random_case(12, 40, 384, 16, 4, 4, 1, mask=0.2, dup=0.2, slots=40),
                                rank_mask=np.array([0, 0, 1, 0], np.int32), seed=1)


def build_mutant(orig: str, planted: str, workdir: str) -> str:
    src = open(SRC).read()
    assert src.count(orig) == 1, f"mutation site not unique or missing: {orig!r}"
    path_c = os.path.join(workdir, "mutant.c")
    path_so = os.path.join(workdir, "libmutant.so")
    open(path_c, "w").write(src.replace(orig, planted))
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-o", path_so, path_c, "-lm"])
    return path_so


def test_real_oracle_passes_quick_pins():
    quick_pins()


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, orig, planted):
    real = oracle._load()
    with tempfile.TemporaryDirectory() as d:
        so = build_mutant(orig, planted, d)
        oracle._lib = oracle._configure(ctypes.CDLL(so))
        try:
            with pytest.raises((AssertionError, ValueError)):
                quick_pins()
        finally:
            oracle._lib = real
