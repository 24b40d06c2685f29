"""Plain CPU oracle for the DSA (DeepSeek Sparse Attention) decode path.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The
product path (the HIP library and its Python binding) never does, and this
module imports nothing from the product package.

What it computes, stage by stage, in float64 (inputs are decoded exactly
from their storage formats; the one rounding to float32 is the indexer
score, because the top-k ranks the float32 scores the API emits):

1. Lightning indexer ("GLM-5: from Vibe Coding to Agentic Engineering",
   section 2.1.2 names the lightning indexer and its token-level sparsity;
   section 3.2, "DSA RL insights", describes it as an extra indexer that
   retrieves the top-k most relevant key-value pairs; "Zhipu AI / GLM",
   section 9.1, gives its shape, 32 heads x 128). The pages do not print the
   scoring formula; the reading used here is the DeepSeek-V3.2 form

       S[r, s] = sum_h  w[r, h] * ReLU( sum_d q[r, h, d] * k[s, d] )

   over candidate keys s = 0 .. q_pos[r] of the query's sequence (causal,
   the query's own key included), one key vector per token shared by all
   indexer heads, no extra scale (a caller folds any scale into w).
   fp8 keys are dequantised as e4m3(code) * bf16(row scale).

2. Top-k, k = 2048 ("Zhipu AI / GLM", sections 9.3 and 11.1). The
   selection must be deterministic: the pages report that a
   non-deterministic top-k desynchronised rollout and training and
   collapsed RL, and that the fix was the deterministic torch.topk
   ("GLM-5: from Vibe Coding...", section 3.2; "GLM-5 Notes", Replay; the
   "non-deterministic CUDA top-k bug" section of the agentic-RL analysis
   page). The oracle's definition: stably sort keys 0..n-1 by score,
   descending, and take the first k_eff = min(k, n); equal scores keep
   ascending key order (lower index wins), -0.0 equals +0.0. Slots past
   k_eff hold -1.

3. Sparse MLA in absorbed (MQA) form over the selected keys: one 576-d
   latent row per token ("GLM-5: from Vibe Coding...", section 2.1: a
   576-dim latent KV cache and 576-dim dot products in decoding) serves as
   the key (all 576 dims) and, in its first 512 dims, as the value:

       l_j = scale * q_abs[r, h, :] . C[idx_j, :]
       O[r, h, :] = sum_j softmax(l)_j * C[idx_j, :512]
       LSE[r, h] = log sum_j exp(l_j)

   The latent cache may also be stored in FP8 ("Zhipu AI / GLM", section
   11.4, lists an FP8 KV cache among GLM-5's rollout measures; the pages fix
   no scale granularity): the reading here is one float32 scale per cached
   token, C[s, :] = e4m3(code[s, :]) * scale[s], dequantised before any
   arithmetic, so the attention above is unchanged.

The caches may be paged: a block table maps each sequence's positions to
pages of a shared pool (cache_rows_of); the values are unchanged.

4. Context-parallel merges (key-range shards): the global top-k from the
   shards' local (score, key) lists, and the log-sum-exp merge of the
   shards' partial attentions (see the end of this module).

The pages print no worked numbers for any of these stages; the tests pin
this module to closed forms, brute force on tiny inputs, library routines
(torch scaled_dot_product_attention for the dense case, torch's fp8 and
bf16 decoders) and invariants.
"""
from __future__ import annotations

import numpy as np

LATENT_DIM = 576   # 512 latent + 64 RoPE per token
VALUE_DIM = 512    # the value is the latent part of the row


# --------------------------------------------------------------------------
# exact decoders of the storage formats
# --------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> float64 (exact: bf16 is the top half of fp32)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """OCP FP8 E4M3FN codes -> float64, from the format's definition.

    Bit layout s.eeee.mmm, exponent bias 7. e == 0 encodes subnormals
    m/8 * 2^-6; otherwise (1 + m/8) * 2^(e-7). The all-ones pattern
    (e == 15, m == 7) is NaN; there is no infinity, so e == 15 with m < 7
    is finite (up to 448).
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    normal = (1.0 + m / 8.0) * np.exp2(e - 7.0)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def decode(arr: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    if dtype == "bf16":
        return bf16_to_f64(arr)
    if dtype == "fp8_e4m3":
        return e4m3fn_to_f64(arr)
    raise ValueError(dtype)


def cache_rows_of(prob, b: int, pos: np.ndarray) -> np.ndarray:
    """Cache rows holding positions ``pos`` of sequence b: row_off[b] + pos, or
    through the block table when the cache is paged (position s sits in page
    table[b, s // page_size] at row s % page_size of that page)."""
    pos = np.asarray(pos, dtype=np.int64)
    table = getattr(prob, "block_table", None)
    if table is None:
        return int(prob.row_off[b]) + pos
    ps = int(prob.page_size)
    return np.asarray(table, dtype=np.int64)[b][pos // ps] * ps + pos % ps


def indexer_keys(prob, b: int, n: int) -> np.ndarray:
    """Keys 0..n-1 of sequence b as float64 (dequantised if fp8)."""
    rows = cache_rows_of(prob, b, np.arange(n))
    k = decode(prob.k_idx[rows], prob.key_dtype)
    if prob.key_dtype == "fp8_e4m3":
        k = k * bf16_to_f64(prob.k_scale[rows])[:, None]
    return k


# --------------------------------------------------------------------------
# stage 1: lightning indexer scores
# --------------------------------------------------------------------------

def index_scores_row(q: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """Scores of one query over ``keys`` ([n, D_I], float64).

    q: [H_I, D_I], w: [H_I]. Returns float32 [n]: the float64 score rounded
    once to float32 (nearest even).
    """
    z = keys @ q.T                      # z[s, h] = q_h . k_s
    a = np.where(z > 0.0, z, 0.0)       # ReLU
    s64 = a @ w                         # sum_h w_h * ReLU(z_h)
    return s64.astype(np.float32)


def index_scores(prob, rows=None) -> list:
    """Scores for the queries in ``rows`` (all when None): a list of float32
    arrays, entry i holding keys 0..q_pos[r] of query r = rows[i]."""
    rows = range(prob.R) if rows is None else rows
    q_all = decode(prob.q_idx, prob.act_dtype)
    w_all = np.asarray(prob.head_w, dtype=np.float64)
    out = []
    for r in rows:
        b = int(prob.q_seq[r])
        n = int(prob.q_pos[r]) + 1
        out.append(index_scores_row(q_all[r], w_all[r], indexer_keys(prob, b, n)))
    return out


# --------------------------------------------------------------------------
# stage 2: deterministic top-k
# --------------------------------------------------------------------------

def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """First k_eff = min(k, n) keys of the stable descending sort of the
    float32 ``scores``; ties keep ascending key index. Pads with -1 to k."""
    s = np.asarray(scores, dtype=np.float32).astype(np.float64)
    n = s.shape[0]
    k_eff = min(k, n)
    order = np.argsort(-s, kind="stable")   # -(+0) == -(-0) compare equal
    out = np.full(k, -1, dtype=np.int32)
    out[:k_eff] = order[:k_eff]
    return out


def topk(score_rows: list, k: int) -> np.ndarray:
    return np.stack([topk_row(s, k) for s in score_rows]) if score_rows else \
        np.zeros((0, k), np.int32)


# --------------------------------------------------------------------------
# stage 3: sparse MLA (absorbed form) over the selected latent rows
# --------------------------------------------------------------------------

def attention_weights(q_abs_r: np.ndarray, rows: np.ndarray, scale: float):
    """Softmax weights [H, m] and logits of every head over ``rows``."""
    logits = scale * (q_abs_r @ rows.T)            # [H, m], 576-dim dots
    mx = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - mx)
    return e / e.sum(axis=1, keepdims=True), logits


def sparse_mla_row(q_abs_r: np.ndarray, rows: np.ndarray, scale: float):
    """O [H, 512] and LSE [H] (natural log) of one query over ``rows`` [m, 576]."""
    if rows.shape[0] == 0:
        H = q_abs_r.shape[0]
        return np.zeros((H, VALUE_DIM)), np.full(H, -np.inf)
    p, logits = attention_weights(q_abs_r, rows, scale)
    out = p @ rows[:, :VALUE_DIM]
    mx = logits.max(axis=1)
    lse = mx + np.log(np.exp(logits - mx[:, None]).sum(axis=1))
    return out, lse


def latent_dtype(prob) -> str:
    """Storage dtype of the latent cache (the activation dtype unless set)."""
    return getattr(prob, "latent_dtype", None) or prob.act_dtype


def latent_rows(prob, cache_rows: np.ndarray) -> np.ndarray:
    """Latent rows (float64) at the absolute cache positions ``cache_rows``;
    fp8 rows are e4m3(code) * float32(row scale)."""
    cache_rows = np.asarray(cache_rows, dtype=np.int64)
    dt = latent_dtype(prob)
    c = decode(prob.latent[cache_rows], dt)
    if dt == "fp8_e4m3":
        sc = np.asarray(prob.latent_scale, dtype=np.float32)[cache_rows].astype(np.float64)
        c = c * sc[:, None]
    return c


def selected_rows(prob, r: int, idx_row: np.ndarray) -> np.ndarray:
    """Latent rows (float64) of the keys named by idx_row (entries < 0 skipped)."""
    b = int(prob.q_seq[r])
    sel = np.asarray(idx_row)
    sel = sel[sel >= 0].astype(np.int64)
    return latent_rows(prob, cache_rows_of(prob, b, sel))


def sparse_mla(prob, idx: np.ndarray, rows=None):
    """O [len(rows), H, 512] and LSE [len(rows), H] for the given index lists."""
    rows = list(range(prob.R)) if rows is None else list(rows)
    q_all = decode(prob.q_abs, prob.act_dtype)
    outs, lses = [], []
    for i, r in enumerate(rows):
        o, l = sparse_mla_row(q_all[r], selected_rows(prob, r, idx[i]), prob.scale)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


# --------------------------------------------------------------------------
# the whole path
# --------------------------------------------------------------------------

def dsa_forward(prob, rows=None):
    """Indexer -> top-k -> sparse MLA for the queries in ``rows``.

    Returns (scores list, idx [m, k], O [m, H, 512], LSE [m, H])."""
    rows = list(range(prob.R)) if rows is None else list(rows)
    scores = index_scores(prob, rows)
    idx = topk(scores, prob.k)
    out, lse = sparse_mla(prob, idx, rows)
    return scores, idx, out, lse


# --------------------------------------------------------------------------
# context parallelism: key-range shards, merged exactly
# --------------------------------------------------------------------------
# "GLM-5: from Vibe Coding to Agentic Engineering", section 2.4.2, splits
# long sequences over context-parallel groups. The reading here: shard p
# holds keys [lo_p, hi_p) of every sequence, selects its local top-k, and a
# merge of the shards' (score, key) lists gives the global selection; each
# shard then attends over the global winners it holds, and a log-sum-exp
# merge of the shards' (O, LSE) gives the output.

def topk_merge(pair_scores: np.ndarray, pair_idx: np.ndarray, k: int) -> np.ndarray:
    """Global top-k of P shards' candidate lists [P, m] (float32 scores,
    global key indices, -1 = empty): the first k of the union stably sorted
    by score descending, ties to the lower key. Pads with -1."""
    s = np.asarray(pair_scores, dtype=np.float32).reshape(-1)
    i = np.asarray(pair_idx, dtype=np.int64).reshape(-1)
    keep = i >= 0
    s, i = s[keep].astype(np.float64), i[keep]
    order = np.lexsort((i, -s))                 # primary: score desc; then key asc
    out = np.full(k, -1, dtype=np.int32)
    n = min(k, order.size)
    out[:n] = i[order[:n]]
    return out


def attn_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Merge P partial attentions over disjoint key sets: o_parts [P, H, 512]
    (each normalised over its own keys), lse_parts [P, H] (natural log,
    -inf = no key). O = sum_p exp(LSE_p - LSE) O_p, LSE = log sum_p exp(LSE_p)."""
    o = np.asarray(o_parts, dtype=np.float64)
    l = np.asarray(lse_parts, dtype=np.float64)
    H = l.shape[1]
    out = np.zeros(o.shape[1:])
    lse = np.full(H, -np.inf)
    for h in range(H):
        fin = np.isfinite(l[:, h])
        if not fin.any():
            continue
        m = l[fin, h].max()
        w = np.exp(l[fin, h] - m)
        lse[h] = m + np.log(w.sum())
        out[h] = (w[:, None] * o[fin, h]).sum(axis=0) / w.sum()
    return out, lse
