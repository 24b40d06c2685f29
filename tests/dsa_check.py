"""Shared checks for the GPU parity tests (bounds and tolerances).

Indexer score bound. The HIP path forms z_h = q_h . k_s with fp32
accumulation over D_I products, takes ReLU (1-Lipschitz), and sums
w_h * ReLU(z_h) over H_I heads in fp32 (plus one multiply by the fp8 row
scale). The standard recursive-summation bound, valid for any summation
order, gives

    |S_gpu - S| <= gamma * sum_h |w_h| sum_d |q_hd k_sd|,  gamma = (D_I + H_I + 4) * u

and the oracle's float32 score is within u*|S| (u*|S| more for the fp8
scale). Here u is taken as 2^-23 (twice the fp32 unit roundoff) so the bound
also holds if the matrix cores truncate instead of rounding.

Attention tolerance: for bf16 inputs with fp32 accumulation, max |O - O_ref|
<= 2e-2 and ||O - O_ref||_2 / ||O_ref||_2 <= 1e-2 per case and also for every
(query, head) row of O separately; fp32 inputs use 1e-5 for all three.
"""
import numpy as np

from oracle import dsa_oracle as O

U = 2.0 ** -23


def abs_products(prob, r, keys_idx):
    """sum_h |w_h| sum_d |q_hd k_sd| for query r over the given key positions."""
    q = np.abs(O.decode(prob.q_idx[r], prob.act_dtype))                 # [H_I, D_I]
    w = np.abs(np.asarray(prob.head_w[r], np.float64))
    b = int(prob.q_seq[r])
    keys = np.abs(O.indexer_keys(prob, b, int(prob.q_pos[r]) + 1)[keys_idx])
    return (keys @ q.T) @ w


def score_bound(prob, r, keys_idx, ref):
    gamma = (prob.D_I + prob.H_I + 4) * U
    extra = 2 * U if prob.key_dtype == "fp8_e4m3" else U
    return gamma * abs_products(prob, r, keys_idx) + extra * np.abs(ref)


def assert_scores_close(prob, r, gpu_row, keys_idx=None):
    """GPU scores of query r (at keys_idx, all when None) within the bound."""
    n = int(prob.q_pos[r]) + 1
    keys_idx = np.arange(n) if keys_idx is None else np.asarray(keys_idx)
    ref = O.index_scores(prob, rows=[r])[0][keys_idx].astype(np.float64)
    got = np.asarray(gpu_row, np.float64)[keys_idx]
    bound = score_bound(prob, r, keys_idx, ref)
    bad = np.abs(got - ref) > bound
    assert not bad.any(), (f"row {r}: {bad.sum()} scores outside the bound; worst at key "
                           f"{keys_idx[np.argmax(np.abs(got - ref) - bound)]}")
    return ref, bound


def assert_attn_close(out, ref, lse=None, lse_ref=None, fp32=False):
    out = np.asarray(out, np.float64)
    ref = np.asarray(ref, np.float64)
    atol, rtol = (1e-5, 1e-5) if fp32 else (2e-2, 1e-2)
    err = np.abs(out - ref)
    assert err.max() <= atol, f"max abs err {err.max():.3e}"
    rel = np.linalg.norm(out - ref) / max(np.linalg.norm(ref), 1e-30)
    assert rel <= rtol, f"relative err {rel:.3e}"
    # the same relative bound for every (query, head) row of O, so a wrong head
    # or query cannot hide behind the others in the global norm; rows whose
    # reference is zero (no key selected) must be zero
    if out.ndim >= 2:
        o2 = out.reshape(-1, out.shape[-1])
        r2 = ref.reshape(-1, ref.shape[-1])
        nr = np.linalg.norm(r2, axis=1)
        ne = np.linalg.norm(o2 - r2, axis=1)
        zero = nr == 0
        assert (ne[zero] == 0).all(), "a row with no selected key is not zero"
        per = ne[~zero] / nr[~zero]
        if per.size:
            worst = int(np.argmax(per))
            assert per.max() <= rtol, f"row {np.flatnonzero(~zero)[worst]}: relative err {per.max():.3e}"
    if lse is not None:
        lse = np.asarray(lse, np.float64)
        lse_ref = np.asarray(lse_ref, np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lse), fin)
        tol = 1e-5 if fp32 else 2e-3
        assert np.abs(lse[fin] - lse_ref[fin]).max(initial=0) <= tol * max(1.0, np.abs(lse_ref[fin]).max(initial=1))
    return err.max(), rel


def assert_index_invariants(idx, q_pos, k):
    idx = np.asarray(idx)
    for r in range(idx.shape[0]):
        n = int(q_pos[r]) + 1
        k_eff = min(k, n)
        row = idx[r]
        assert (row[:k_eff] >= 0).all() and (row[:k_eff] < n).all()
        assert np.unique(row[:k_eff]).size == k_eff
        assert (row[k_eff:] == -1).all()


def near_tie_swaps(gpu_idx, ref_idx, ref_scores, bound):
    """Keys selected by one side only must sit within the score bound of the
    k-th oracle score. Returns the number of such swaps."""
    g = set(int(x) for x in gpu_idx if x >= 0)
    o = set(int(x) for x in ref_idx if x >= 0)
    diff = g ^ o
    if not diff:
        return 0
    kth = ref_idx[ref_idx >= 0][-1]
    for key in diff:
        gap = abs(ref_scores[key] - ref_scores[kth])
        assert gap <= 2 * (bound[key] + bound[kth]), f"key {key}: gap {gap} beyond the bound"
    return len(diff) // 2
