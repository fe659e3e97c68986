"""Plant plausible mistakes in copies of the oracle source (on the CPU) and
require every one to be caught by at least one pin.  This is the evidence
that the pins constrain each part of the oracle: addressing, layout,
grouping, softmax, scaling, merge and the element decoders."""
import pytest

import oracle
from tests import oracle_pins

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("no_max_subtraction", "s[t] = exp(s[t] - m);", "s[t] = exp(s[t]);"),
    ("no_normalisation", "const double w = s[t] / z;", "const double w = s[t];"),
    ("scale_dropped", "s[t] = scale * dot;", "s[t] = dot;"),
    ("strided_gqa_mapping", "const int64_t h = g * G + k;", "const int64_t h = k * num_kv_heads + g;"),
    ("v_read_token_major", "V[t * D + d] = elem(v_pool, dtype, tile + (slot / S) * D * S + d * S + slot % S);",
     "V[t * D + d] = elem(v_pool, dtype, tile + slot * D + d);"),
    ("v_groups_ignored", "V[t * D + d] = elem(v_pool, dtype, tile + (slot / S) * D * S + d * S + slot % S);",
     "V[t * D + d] = elem(v_pool, dtype, tile + d * B + slot);"),
    ("v_group_size_wrong", "const int64_t S = (B % 16 == 0) ? 16 : B;", "const int64_t S = (B % 32 == 0) ? 32 : B;"),
    ("k_read_dim_major", "K[t * D + d] = elem(k_pool, dtype, tile + slot * D + d);",
     "K[t * D + d] = elem(k_pool, dtype, tile + d * B + slot);"),
    ("slot_off_by_one", "const int64_t slot = t % B;", "const int64_t slot = (t + 1) % B;"),
    ("block_index_rounding", "const int64_t j = t / B;", "const int64_t j = (t + 1) / B;"),
    ("table_row_offset_missing", "block_tables[(int64_t)b * max_blocks_per_seq + j]", "block_tables[j]"),
    ("kv_head_stride_missing", "const int64_t tile = (phys * H + g) * B * D; /* same tile base",
     "const int64_t tile = (phys + g) * B * D; /* same tile base"),
    ("slack_slots_attended", "const int64_t L = seq_lens[b] > 0 ? seq_lens[b] : 0;",
     "const int64_t L = seq_lens[b] > 0 ? ((seq_lens[b] + block_size - 1) / block_size) * block_size : 0;"),
    ("q_element_size_swapped", "(dtype == ORC_F32 ? 4 : 2)", "(dtype == ORC_F32 ? 2 : 4)"),
    ("merge_o_not_rescaled", "o[d] = o1[d] * a1 + o2[d] * a2;", "o[d] = o1[d] + o2[d];"),
    ("merge_exponent_sign", "const double a1 = (m1 == -INFINITY) ? 0.0 : exp(m1 - m);",
     "const double a1 = (m1 == -INFINITY) ? 0.0 : exp(m - m1);"),
    ("merge_empty_guard_missing", "const double a2 = (m2 == -INFINITY) ? 0.0 : exp(m2 - m);",
     "const double a2 = exp(m2 - m);"),
    ("partial_max_not_used", "const double p = exp(scale * dot - m);", "const double p = exp(scale * dot);"),
    ("f16_exponent_bias", "v = ldexp((double)(0x400 | f), e - 25);", "v = ldexp((double)(0x400 | f), e - 24);"),
    ("f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    ("f16_hidden_bit_missing", "v = ldexp((double)(0x400 | f), e - 25);", "v = ldexp((double)f, e - 25);"),
    ("bf16_wrong_half", "const uint32_t u = (uint32_t)b << 16;", "const uint32_t u = (uint32_t)b;"),
    # writing the cache
    ("append_slot_off_by_one", "const int64_t j = t / B, slot = t % B;",
     "const int64_t j = t / B, slot = (t + 1) % B;"),
    ("append_v_not_transposed", "const int64_t vdst = tile + (slot / G) * D * G + d * G + slot % G;",
     "const int64_t vdst = tile + slot * D + d;"),
    ("append_kv_head_stride_missing",
     "const int64_t tile = (phys * H + g) * B * D;\n      const int64_t src",
     "const int64_t tile = (phys + g) * B * D;\n      const int64_t src"),
    ("append_source_rows_head_major", "const int64_t src = (b * H + g) * D;",
     "const int64_t src = (g * num_seqs + b) * D;"),
    ("append_table_row_offset_missing", "const int64_t phys = block_tables[b * max_blocks_per_seq + j];",
     "const int64_t phys = block_tables[j];"),
    ("copy_block_bytes_one_head", "const int64_t block_bytes = (int64_t)num_kv_heads * block_size * head_dim * esize;",
     "const int64_t block_bytes = (int64_t)block_size * head_dim * esize;"),
    ("copy_direction_swapped",
     "memmove((char*)k_pool + dst[i] * block_bytes, (const char*)k_pool + src[i] * block_bytes,",
     "memmove((char*)k_pool + src[i] * block_bytes, (const char*)k_pool + dst[i] * block_bytes,"),
    ("copy_v_pool_skipped",
     "memmove((char*)v_pool + dst[i] * block_bytes, (const char*)v_pool + src[i] * block_bytes,\n            block_bytes);",
     "(void)v_pool;"),
    # block-wise eviction scoring
    ("score_first_head_only", "for (int64_t g = 0; g < H; ++g) {\n          const int64_t base",
     "for (int64_t g = 0; g < 1; ++g) {\n          const int64_t base"),
    ("score_squared_norms", "ratio_sum += sqrt(vv) / sqrt(kk);", "ratio_sum += vv / kk;"),
    ("score_ratio_inverted", "ratio_sum += sqrt(vv) / sqrt(kk);", "ratio_sum += sqrt(kk) / sqrt(vv);"),
    ("score_sum_not_mean", "scores[b * M + j] = ratio_sum / (double)B;", "scores[b * M + j] = ratio_sum;"),
    ("score_partial_block_scored", "const int64_t full = L / B;", "const int64_t full = (L + B - 1) / B;"),
    ("score_v_read_token_major",
     "const double v = elem(v_pool, dtype, base + (slot / G) * D * G + d * G + slot % G);",
     "const double v = elem(v_pool, dtype, base + slot * D + d);"),
    ("evict_without_full_last_block", "if (L > 0 && L % B == 0) {", "if (L > 0) {"),
    ("evict_ties_pick_last", "if (scores[b * M + j] < best) {", "if (scores[b * M + j] <= best) {"),
    ("evict_picks_highest", "if (scores[b * M + j] < best) {",
     "if (best == INFINITY || scores[b * M + j] > best) {"),
    # paged prefill
    ("prefill_not_causal", "oracle_attention(qrow, K, V, p + 1, D, scale, out + off, s);",
     "oracle_attention(qrow, K, V, Lb, D, scale, out + off, s);"),
    ("prefill_position_off_by_one", "const int64_t p = Lb - n + i; ", "const int64_t p = Lb - n + i - 1; "),
    ("prefill_causal_top_left", "const int64_t p = Lb - n + i; ", "const int64_t p = i; "),
    ("prefill_rows_from_zero", "const int64_t row = q_start[b] + i;", "const int64_t row = i;"),
    ("prefill_head_mapping_strided", "const int64_t off = (row * num_q_heads + g * G + k) * D;",
     "const int64_t off = (row * num_q_heads + k * num_kv_heads + g) * D;"),
    ("prefill_rows_beyond_cache_accepted", "if (n < 0 || seq_lens[b] < 0 || n > seq_lens[b]) return -2;",
     "if (n < 0 || seq_lens[b] < 0) return -2;"),
]


@pytest.fixture(scope="module")
def src():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, src, name, old, new):
    assert src.count(old) == 1, f"mutation site for {name} not unique in oracle.c"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.compile_source(str(path), str(tmp_path / f"lib{name}.so"))
    O = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.PINS:
        try:
            pin(O)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin catches mutant {name}"
