"""The pins have teeth: each plausible oracle mistake, planted here on the
CPU by swapping one oracle function for a mutated copy, makes at least one
pin fail. The real oracle is restored after every case."""
import numpy as np
import pytest

from oracle import dsa_oracle as O
import test_oracle_attention as TA
import test_oracle_indexer as TI
import test_oracle_topk as TT
import test_oracle_cp as TC
import test_oracle_pipeline as TPL


def _no_relu(q, w, keys):
    return ((keys @ q.T) @ w).astype(np.float32)


def _w_reversed(q, w, keys):
    z = keys @ q.T
    return (np.where(z > 0, z, 0) @ w[::-1]).astype(np.float32)


def _unstable(scores, k):
    s = np.asarray(scores, np.float32).astype(np.float64)
    order = np.argsort(-s, kind="stable")[::-1]
    order = order[np.argsort(-s[order], kind="stable")]   # ties end up high index first
    out = np.full(k, -1, np.int32)
    out[:min(k, s.size)] = order[:min(k, s.size)]
    return out


def _ascending(scores, k):
    s = np.asarray(scores, np.float32).astype(np.float64)
    order = np.argsort(s, kind="stable")
    out = np.full(k, -1, np.int32)
    out[:min(k, s.size)] = order[:min(k, s.size)]
    return out


def _value_from_rope_end(q, rows, scale):
    p, logits = O.attention_weights(q, rows, scale)
    mx = logits.max(axis=1)
    return p @ rows[:, 64:], mx + np.log(np.exp(logits - mx[:, None]).sum(axis=1))


def _no_scale(q, rows, scale):
    return _orig_attn(q, rows, 1.0)


def _latent_only_logits(q, rows, scale):
    return _orig_attn(q[:, :512], rows[:, :512], scale) if rows.shape[0] else _orig_attn(q, rows, scale)


_orig_attn = O.sparse_mla_row


def _causal_off_by_one(prob, rows=None):
    rows = range(prob.R) if rows is None else rows
    q_all = O.decode(prob.q_idx, prob.act_dtype)
    w_all = np.asarray(prob.head_w, np.float64)
    return [O.index_scores_row(q_all[r], w_all[r], O.indexer_keys(prob, int(prob.q_seq[r]), int(prob.q_pos[r])))
            for r in rows]


def _fp8_no_scale(prob, b, n):
    lo = int(prob.row_off[b])
    return O.decode(prob.k_idx[lo:lo + n], prob.key_dtype)


def _fp8_latent_no_scale(prob, cache_rows):
    return O.decode(prob.latent[np.asarray(cache_rows, np.int64)], O.latent_dtype(prob))


def _fp8_latent_scale_of_next_row(prob, cache_rows):
    cache_rows = np.asarray(cache_rows, np.int64)
    sc = np.asarray(prob.latent_scale, np.float64)
    nxt = np.minimum(cache_rows + 1, sc.shape[0] - 1)
    nxt = np.where(nxt == cache_rows, np.maximum(cache_rows - 1, 0), nxt)
    return O.decode(prob.latent[cache_rows], O.latent_dtype(prob)) * sc[nxt][:, None]


def _fp8_latent_scaled_keys_only(prob, cache_rows):
    rows = _orig_latent_rows(prob, cache_rows)
    raw = O.decode(prob.latent[np.asarray(cache_rows, np.int64)], O.latent_dtype(prob))
    rows[:, :512] = raw[:, :512]
    return rows


_orig_latent_rows = O.latent_rows


def _merge_ties_high_first(pair_scores, pair_idx, k):
    s = np.asarray(pair_scores, np.float32).reshape(-1)
    i = np.asarray(pair_idx, np.int64).reshape(-1)
    keep = i >= 0
    s, i = s[keep].astype(np.float64), i[keep]
    order = np.lexsort((-i, -s))
    out = np.full(k, -1, np.int32)
    out[:min(k, order.size)] = i[order[:k]]
    return out


def _page_row_without_page_base(prob, b, pos):
    pos = np.asarray(pos, np.int64)
    if getattr(prob, "block_table", None) is None:
        return int(prob.row_off[b]) + pos
    ps = int(prob.page_size)
    return np.asarray(prob.block_table, np.int64)[b][pos // ps] + pos % ps


def _merge_unweighted(o_parts, lse_parts):
    o = np.asarray(o_parts, np.float64)
    l = np.asarray(lse_parts, np.float64)
    fin = np.isfinite(l)
    out = np.where(fin[:, :, None], o, 0).sum(axis=0) / np.maximum(fin.sum(axis=0), 1)[:, None]
    m = np.where(fin, l, -np.inf).max(axis=0)
    return out, m + np.log(np.where(fin, np.exp(l - m), 0).sum(axis=0))


CASES = [
    ("index_scores_row", _no_relu, [TI.test_relu_zeroes_negative_dots, TI.test_golden_hand_case]),
    ("index_scores_row", _w_reversed, [TI.test_head_weights_follow_their_head]),
    ("index_scores", _causal_off_by_one, [TI.test_causal_bound_includes_own_key]),
    ("indexer_keys", _fp8_no_scale, [TI.test_fp8_keys_use_row_scale]),
    ("topk_row", _unstable, [TT.test_all_equal_is_index_order, TT.test_golden_hand_case]),
    ("topk_row", _ascending, [TT.test_strictly_increasing_gives_latest_first]),
    ("sparse_mla_row", _value_from_rope_end, [TA.test_single_key_gives_its_value_rows, TA.test_golden_hand_case]),
    ("sparse_mla_row", _no_scale, [TA.test_dense_equals_sdpa_when_k_covers_context]),
    ("sparse_mla_row", _latent_only_logits, [TA.test_golden_hand_case]),
    ("cache_rows_of", _page_row_without_page_base, [TPL.test_paged_cache_rows_hand_case,
                                                     lambda: TPL.test_paged_view_moves_rows_only(64)]),
    ("topk_merge", _merge_ties_high_first, [TC.test_merge_closed_forms]),
    ("attn_merge", _merge_unweighted, [TC.test_attention_merge_equals_whole_attention,
                                       TC.test_attention_merge_closed_forms]),
    ("latent_rows", _fp8_latent_no_scale, [TA.test_fp8_latent_golden_hand_case,
                                           TA.test_fp8_latent_single_key_is_its_scaled_row]),
    ("latent_rows", _fp8_latent_scale_of_next_row, [TA.test_fp8_latent_golden_hand_case,
                                                    TA.test_fp8_latent_single_key_is_its_scaled_row]),
    ("latent_rows", _fp8_latent_scaled_keys_only, [TA.test_fp8_latent_golden_hand_case,
                                                   TA.test_fp8_latent_single_key_is_its_scaled_row]),
]


@pytest.mark.parametrize("name,mutant,pins", CASES, ids=[f"{c[0]}:{c[1].__name__}" for c in CASES])
def test_planted_mistake_is_caught(monkeypatch, name, mutant, pins):
    monkeypatch.setattr(O, name, mutant)
    for pin in pins:
        with pytest.raises(AssertionError):
            pin()
