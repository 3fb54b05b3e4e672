"""Plant plausible mistakes in copies of the oracle source and check the pins catch each one.

Every mutant is built with gcc into a temporary directory and loaded as a
separate library; the committed oracle is never modified.  The mutations are
memory-safe (no mutant reads outside its buffers).  A mutation whose text no
longer occurs exactly once in oracle.c fails the test, so the list stays in
step with the source.
"""
import os

import pytest

import oracle
import oracle_pins

MUTATIONS = [
    ("rope dropped from the scores",
     "for (int d = 0; d < DQK; ++d) acc += qrow[d] * k[d];",
     "for (int d = 0; d < DV; ++d) acc += qrow[d] * k[d];"),
    ("V taken from the end of the row instead of its c_kv part",
     "const double *v = kbuf + (int64_t)j * DQK;  /* V = first d_v of K */",
     "const double *v = kbuf + (int64_t)j * DQK + (DQK - DV);"),
    ("sign of the max subtraction flipped",
     "score[j] = exp(score[j] - m);",
     "score[j] = exp(m - score[j]);"),
    ("softmax scale dropped",
     "score[j] = J->scale * acc;",
     "score[j] = acc;"),
    ("block table ignored",
     "return (int64_t)blk * J->block_size + p % J->block_size;",
     "return (int64_t)p;"),
    ("slot inside the block off by one",
     "return (int64_t)blk * J->block_size + p % J->block_size;",
     "return (int64_t)blk * J->block_size + (p + 1) % J->block_size;"),
    ("max dropped from the lse",
     "J->lse[r * H + h] = m + log(z);",
     "J->lse[r * H + h] = log(z);"),
    ("output not normalised",
     "for (int d = 0; d < DV; ++d) o[d] /= z;",
     ""),
    ("e4m3 exponent bias off by one",
     "v = ldexp(1.0 + m / 8.0, e - 7);",
     "v = ldexp(1.0 + m / 8.0, e - 8);"),
    ("bf16 mantissa width wrong",
     "v = ldexp(1.0 + m / 128.0, e - 127);",
     "v = ldexp(1.0 + m / 256.0, e - 127);"),
    ("fp8 scale group index wrong",
     "* oracle_f32_le_to_f64(scales + 4 * (d / 128));",
     "* oracle_f32_le_to_f64(scales + 4 * ((d % 128) / 32));"),
    ("fp32 scale: subnormal exponent off by one",
     "v = ldexp((double)m, -149);",
     "v = ldexp((double)m, -150);"),
    ("fp32 scale: infinity decoded as NaN",
     "        v = (m == 0) ? INFINITY : NAN;\n    else if (e == 0)\n        v = ldexp((double)m, -149);",
     "        v = NAN;\n    else if (e == 0)\n        v = ldexp((double)m, -149);"),
    ("fp32 scale: exponent bias off by one",
     "v = ldexp(1.0 + m / 8388608.0, e - 127);",
     "v = ldexp(1.0 + m / 8388608.0, e - 126);"),
    ("indexer abs_sum doubled",
     "        a += fabs(t);",
     "        a += 2.0 * fabs(t);"),
    ("indexer abs_sum one too large per term",
     "        a += fabs(t);",
     "        a += fabs(t) + 1.0;"),
    ("indexer abs_sum of signed terms",
     "        a += fabs(t);",
     "        a += t;"),
    ("rope elements shifted by one",
     "k[d] = oracle_bf16_to_f64(load_u16_le(rope + 2 * (d - d_v)));",
     "k[d] = oracle_bf16_to_f64(load_u16_le(rope + 2 * (d - d_v + 1)));"),
    ("bf16 row elements swapped pairwise",
     "for (int d = 0; d < d_qk; ++d) k[d] = oracle_bf16_to_f64(load_u16_le(row + 2 * d));",
     "for (int d = 0; d < d_qk; ++d) k[d] = oracle_bf16_to_f64(load_u16_le(row + 2 * (d ^ 1)));"),
    ("UE8M0 exponent bias off by one",
     "return e == 0xff ? NAN : ldexp(1.0, (int)e - 127);",
     "return e == 0xff ? NAN : ldexp(1.0, (int)e - 126);"),
    ("UE8M0 scale group of 128 instead of 64",
     "k[d] = oracle_e4m3fn_to_f64(row[d]) * oracle_ue8m0_to_f64(scales[d / V4_GROUP]);",
     "k[d] = oracle_e4m3fn_to_f64(row[d]) * oracle_ue8m0_to_f64(scales[d / 128]);"),
    ("scale record taken from the token row instead of the block's record area",
     "const uint8_t *scales = block + (int64_t)block_size * V4_DATA_BYTES + (int64_t)slot * V4_SCALE_BYTES;",
     "const uint8_t *scales = row + 2 * V4_NOPE / 2 + 2;"),
    ("scale records packed at 7 bytes",
     "const uint8_t *scales = block + (int64_t)block_size * V4_DATA_BYTES + (int64_t)slot * V4_SCALE_BYTES;",
     "const uint8_t *scales = block + (int64_t)block_size * V4_DATA_BYTES + (int64_t)slot * 7;"),
    ("rope read from the start of the row",
     "k[d] = oracle_bf16_to_f64(load_u16_le(row + V4_NOPE + 2 * (d - V4_NOPE)));",
     "k[d] = oracle_bf16_to_f64(load_u16_le(row + 2 * (d - V4_NOPE)));"),
    ("token rows strided by the 584-byte slot",
     "const uint8_t *row = block + (int64_t)slot * V4_DATA_BYTES;",
     "const uint8_t *row = block + (int64_t)slot * (V4_DATA_BYTES + V4_SCALE_BYTES);"),
    ("indexer ties go to the higher position",
     "return sa > sb || (sa == sb && pa < pb);",
     "return sa > sb || (sa == sb && pa > pb);"),
    ("indexer keeps the lowest scores",
     "return sa > sb || (sa == sb && pa < pb);",
     "return sa < sb || (sa == sb && pa < pb);"),
    ("indexer list not in position order",
     "        for (int64_t p = 0; p < cap; ++p) {\n            if (!taken[p]) continue;",
     "        for (int64_t p = cap - 1; p >= 0; --p) {\n            if (!taken[p]) continue;"),
    ("indexer ignores seq_lens",
     "    if ((int64_t)seq_lens[b] < cap) cap = seq_lens[b];\n",
     ""),
    ("indexer key rows strided by half a row",
     "const int64_t row_bytes = 2 * (int64_t)d_idx;",
     "const int64_t row_bytes = (int64_t)d_idx;"),
    ("indexer drops the last key dimension",
     "    for (int d = 0; d < d_idx; ++d) {\n        double t = oracle_bf16_to_f64(q[d])",
     "    for (int d = 0; d < d_idx - 1; ++d) {\n        double t = oracle_bf16_to_f64(q[d])"),
    ("seq_lens ignored",
     "if (J->seq_lens && (int64_t)J->seq_lens[b] < cap) cap = J->seq_lens[b];",
     ""),
    ("empty row gives lse 0",
     "J->lse[r * H + h] = -INFINITY;\n            continue;",
     "J->lse[r * H + h] = 0.0;\n            continue;"),
    ("combine weights not normalised by the total",
     "double w = exp(part_lse[(int64_t)s * n + i] - total);",
     "double w = exp(part_lse[(int64_t)s * n + i] - M);"),
    ("combine lse without the max",
     "double total = M + log(z);",
     "double total = log(z);"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutant(name, old, new, tmp_path):
    src = open(oracle.SOURCE).read()
    assert src.count(old) == 1, f"mutation text for '{name}' must occur exactly once in oracle.c"
    mutated = src.replace(old, new)
    path = os.path.join(str(tmp_path), "mutant.c")
    with open(path, "w") as f:
        f.write(mutated)
    lib_path = oracle.build(force=True, src=path, out_path=os.path.join(str(tmp_path), "libmutant.so"))
    orc = oracle.Oracle(lib_path)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake: {name}"
