"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin catches each one.

Each mutation patches one oracle function for the duration of the test. A
pin that still passes under the mutation would be a pin that cannot see that
mistake.
"""

import numpy as np
import pytest

from oracle import attention as A
from oracle import paging as P
import test_oracle_attention as TA
import test_oracle_paging as TP
import test_oracle_cache_write as TW


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_scale_is_caught(monkeypatch):
    orig = A.softmax_attend
    monkeypatch.setattr(A, "softmax_attend", lambda q, K, V, scale: orig(q, K, V, 1.0))
    _fails(TA.test_decode_matches_bruteforce_contiguous, "f16", 8, 8)


def test_wrong_head_grouping_is_caught(monkeypatch):
    # Interleaved grouping (h % Hkv) instead of consecutive (h // g).
    def bad(q_bits, dtype, ki, kv, vi, vv, layer, bt, ctx, bs, Hkv, D, scale, select=None):
        q = q_bits.copy()
        Hq = q.shape[1]
        perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]
        out = orig(q[:, perm], dtype, ki, kv, vi, vv, layer, bt, ctx, bs, Hkv, D, scale, select)
        res = np.empty_like(out)
        res[:, perm] = out
        return res
    orig = A.paged_decode
    monkeypatch.setattr(A, "paged_decode", bad)
    _fails(TA.test_head_grouping_matches_page)


def test_causal_off_by_one_is_caught(monkeypatch):
    orig = A.softmax_attend
    monkeypatch.setattr(A, "softmax_attend",
                        lambda q, K, V, s: orig(q, K[:-1], V[:-1], s) if len(K) > 1 else orig(q, K, V, s))
    _fails(TA.test_chunk_rows_match_decode_causal_and_unchunked)


def test_transposed_slot_split_is_caught(monkeypatch):
    monkeypatch.setattr(P, "split_slot", lambda slot, bs: (int(slot) % int(bs), int(slot) // int(bs)))
    _fails(TP.test_slot_322_from_page)


def test_wrong_mla_scale_group_is_caught(monkeypatch):
    def bad(rows):
        lat, rope = orig(rows)
        return lat[:, ::-1].copy(), rope          # latent values paired with the wrong positions
    orig = A.mla_parse_rows
    monkeypatch.setattr(A, "mla_parse_rows", bad)
    _fails(TA.test_mla_matches_bruteforce_with_library_fp8_decode)


def test_wrong_layer_stride_is_caught(monkeypatch):
    monkeypatch.setattr(P, "address", lambda v, layer, b, pos: v.offset + b * v.block_stride + pos * v.row_bytes)
    _fails(TP.test_blhnc_pages_views_and_addresses_from_page)


def test_missing_max_subtraction_in_merge_is_caught(monkeypatch):
    monkeypatch.setattr(A, "merge_partitions", lambda ms, ls, accs: (accs.sum(0)) / ls.sum())
    _fails(TA.test_partition_merge_identity, 16)


def test_write_at_wrong_row_is_caught(monkeypatch):
    orig = P.address
    monkeypatch.setattr(P, "address", lambda v, layer, b, pos: orig(v, layer, b, (pos + 1) % 16))
    _fails(TW.test_round_trip_and_untouched_bytes)


def test_truncating_fp8_encoder_is_caught(monkeypatch):
    from oracle import quant as Q
    import test_oracle_quant as TQ
    table = Q._POS_VALUES

    def truncating(q):
        q = np.asarray(q, dtype=np.float64)
        a = np.abs(q)
        idx = np.searchsorted(table, a, side="right") - 1       # round toward zero
        code = Q._POS_CODES[idx.clip(0, len(table) - 1)]
        return (code | np.where(np.signbit(q), 0x80, 0)).astype(np.uint8)
    monkeypatch.setattr(Q, "e4m3_encode", truncating)
    _fails(TQ.test_random_values_match_torch)


def test_wrong_fp8_scale_divisor_is_caught(monkeypatch):
    from oracle import quant as Q
    import test_oracle_quant as TQ
    monkeypatch.setattr(Q, "E4M3_MAX", 480.0)
    _fails(TQ.test_group_recipe_matches_torch, "normal")


def test_shifted_scale_group_is_caught(monkeypatch):
    from oracle import quant as Q
    import test_oracle_quant as TQ
    orig = Q.quantize_group

    def shifted(bits):                      # groups of 128 starting one value late
        bits = np.asarray(bits, dtype=np.uint16)
        return orig(np.roll(bits, 1))
    monkeypatch.setattr(Q, "quantize_group", shifted)
    _fails(TQ.test_row_layout_matches_page_byte_counts)


def test_short_block_copy_is_caught(monkeypatch):
    from oracle import cache_write as Wc

    def short_copy(image, view, pairs, num_layers, block_size):   # the last row of each page is left behind
        return orig(image, view, pairs, num_layers, block_size - 1)
    orig = Wc.copy_blocks
    monkeypatch.setattr(Wc, "copy_blocks", short_copy)
    _fails(TW.test_copy_blocks_is_copy_on_write_for_a_shared_prefix)


def test_swapped_fp8_scales_are_caught(monkeypatch):
    orig = A.paged_decode

    def swapped(*args, k_scale=1.0, v_scale=1.0, **kw):
        return orig(*args, k_scale=v_scale, v_scale=k_scale, **kw)
    monkeypatch.setattr(A, "paged_decode", swapped)
    _fails(TA.test_fp8_cache_decode_equals_bf16_decode_of_the_dequantized_values)


def test_dropped_indexer_relu_is_caught(monkeypatch):
    from oracle import dsa as D
    import test_oracle_dsa as TD

    def no_relu(q_bits, weights, rows):
        q = D.bf16_bits_to_f64(np.asarray(q_bits, dtype=np.uint16))
        return (D.index_keys(rows) @ q.T) @ np.asarray(weights, dtype=np.float64)
    monkeypatch.setattr(D, "index_scores_of_rows", no_relu)
    _fails(TD.test_one_hot_keys_closed_form)


def test_indexer_weights_on_the_wrong_heads_are_caught(monkeypatch):
    from oracle import dsa as D
    import test_oracle_dsa as TD
    orig = D.index_scores_of_rows
    monkeypatch.setattr(D, "index_scores_of_rows", lambda q, w, rows: orig(q, np.asarray(w)[::-1], rows))
    _fails(TD.test_one_hot_keys_closed_form)


def test_dropped_index_key_scale_is_caught(monkeypatch):
    from oracle import dsa as D
    import test_oracle_dsa as TD
    monkeypatch.setattr(D, "index_keys", lambda rows: D.e4m3_bytes_to_f64(np.asarray(rows)[:, :128]))
    _fails(TD.test_index_keys_match_torch_fp8_decoding)


def test_later_position_winning_ties_is_caught(monkeypatch):
    from oracle import dsa as D
    import test_oracle_dsa as TD

    def later_first(scores, top_k):
        n = len(scores)
        if top_k >= n:
            return np.arange(n, dtype=np.int64)
        ranked = sorted(range(n), key=lambda t: (-float(scores[t]), -t))
        return np.sort(np.array(ranked[:top_k], dtype=np.int64))
    monkeypatch.setattr(D, "topk_positions", later_first)
    _fails(TD.test_topk_ties_prefer_earlier_positions)


def test_neighbouring_row_in_sparse_decode_is_caught(monkeypatch):
    from oracle import dsa as D
    import test_oracle_dsa as TD
    monkeypatch.setattr(D, "split_slot", lambda slot, bs: (int(slot) // int(bs), (int(slot) + 1) % int(bs)))
    _fails(TD.test_sparse_decode_over_every_position_is_the_dense_decode)
