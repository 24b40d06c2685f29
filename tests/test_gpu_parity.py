"""GPU parity: every entry point of libdsa.so against the oracle, at sizes
the oracle finishes in seconds (several tiles, ragged tails, edge cases).

Top-k is compared array-exactly with the oracle applied to the *same* fp32
scores; scores are compared bit-for-bit on exact-arithmetic inputs and
within the summation error bound otherwise; attention within the
tolerances of dsa_check. Outputs are poisoned before each call so unwritten
elements show.
"""
import zlib

import numpy as np
import pytest

from oracle import dsa_oracle as O
from sparse_attention_05_amd import inputs
import dsa_check as C

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_attention_05_amd import dsa as mod
    return mod


def _say(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------------------
# top-k on identical scores
# ------------------------------------------------------------------------------

def _score_rows(kind, n, rng):
    if kind == "normal":
        return rng.standard_normal(n).astype(np.float32)
    if kind == "ties8":
        return (rng.integers(0, 8, n) / 8.0).astype(np.float32)
    if kind == "equal":
        return np.full(n, 3.25, np.float32)
    if kind == "zeros":
        return np.where(rng.random(n) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    if kind == "relu":  # half the scores ReLU-killed to +0 or -0, a positive tail
        v = np.maximum(rng.standard_normal(n), 0).astype(np.float32)
        return np.where((v == 0) & (rng.random(n) < 0.5), np.float32(-0.0), v).astype(np.float32)
    if kind == "increasing":
        return np.arange(n, dtype=np.float32)
    if kind == "wide":  # magnitudes over the whole fp32 range, both signs, denormals
        e = rng.uniform(-140, 120, n)
        return (np.sign(rng.standard_normal(n)) * np.exp2(e)).astype(np.float32)
    if kind == "twoclass":  # two tie classes far apart straddle k
        v = np.ones(n, np.float32)
        v[rng.choice(n, 1000, replace=False)] = 100.0
        return v
    if kind == "outlier":  # one huge score above a tight cluster
        v = (1.0 + rng.standard_normal(n) * 1e-3).astype(np.float32)
        v[rng.integers(n)] = 1e30
        return v
    if kind == "steps":  # tie classes of 64 consecutive keys
        return (np.arange(n) // 64).astype(np.float32)
    if kind == "fineties":  # N(0,1) rounded to 1/1024: moderate ties everywhere
        return (np.round(rng.standard_normal(n) * 1024) / 1024).astype(np.float32)
    raise KeyError(kind)


def _run_topk(dsa, rows, k, split=True):
    import torch
    R = len(rows)
    max_n = max(len(x) for x in rows)
    ld = (max_n + 3) // 4 * 4
    S = np.full((R, ld), np.nan, np.float32)   # entries past n are garbage by contract
    for r, x in enumerate(rows):
        S[r, :len(x)] = x
    q_pos = np.array([len(x) - 1 for x in rows], np.int32)
    s_d = torch.from_numpy(S).cuda()
    q_d = torch.from_numpy(q_pos).cuda()
    idx = torch.randint(-7, 1 << 30, (R, k), dtype=torch.int32, device="cuda")
    dsa.dsa_topk(s_d, q_d, max_n, k, idx_out=idx, workspace=None if split else False)
    return idx.cpu().numpy()


TOPK_CASES = [
    ("normal", [1, 2, 63, 64, 65, 2047, 2048, 2049, 4095, 4096, 4097], 2048),
    ("normal", [10000, 16384, 16385, 32767, 32768], 2048),
    ("normal", [32769, 65536, 100003], 2048),
    ("normal", [200000], 2048),
    ("normal", [5000, 70000], 1),
    ("normal", [5000, 4097], 777),
    ("ties8", [4096, 4097, 65536], 2048),
    ("ties8", [200000], 2048),
    ("equal", [3000, 40000], 2048),
    ("zeros", [9000, 50000], 2048),
    ("relu", [32768], 2048),
    ("increasing", [32768, 2100], 2048),
    ("wide", [32768, 3000, 80000], 2048),
    ("twoclass", [32768, 5000, 70000], 2048),
    ("outlier", [32768, 9000, 66000], 2048),
    ("steps", [32768, 4000, 100000], 2048),
    ("fineties", [32768, 65536, 2100], 2048),
    ("normal", [2049, 2050, 2100, 2500], 2048),
]


@pytest.mark.parametrize("split", [True, False], ids=["ws", "nows"])
@pytest.mark.parametrize("kind,lens,k", TOPK_CASES, ids=[f"{c[0]}-{len(c[1])}rows-k{c[2]}" for c in TOPK_CASES])
def test_topk_matches_oracle_on_identical_scores(dsa, kind, lens, k, split):
    """With a workspace, rows longer than 8192 go through the split selection
    (slices, shared pivot, last slice sorts); without, one workgroup per row."""
    rng = np.random.default_rng(zlib.crc32(repr((kind, lens, k)).encode()))
    rows = [_score_rows(kind, n, rng) for n in lens]
    _say("topk", kind, lens, k, "split" if split else "single")
    got = _run_topk(dsa, rows, k, split)
    for r, x in enumerate(rows):
        want = O.topk_row(x, k)
        assert np.array_equal(got[r], want), f"row {r} (n={len(x)}): first diff at {np.argmax(got[r] != want)}"


def test_topk_is_repeatable(dsa):
    rng = np.random.default_rng(11)
    rows = [_score_rows("ties8", n, rng) for n in (65536, 33000, 4097)]
    first = _run_topk(dsa, rows, 2048)
    for _ in range(10):
        assert np.array_equal(_run_topk(dsa, rows, 2048), first)


# ------------------------------------------------------------------------------
# indexer scores
# ------------------------------------------------------------------------------

def _gpu_scores(dsa, prob, d=None):
    import torch
    d = d or inputs.to_torch(prob)
    ld = (prob.max_n + 3) // 4 * 4
    scores = torch.full((prob.R, ld), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, d.row_off, d.q_pos, prob.max_n, k_scale=d.k_scale,
                         q_seq=d.q_seq, scores=scores)
    return scores.cpu().numpy(), d


def test_scores_exact_on_integer_inputs_fp32(dsa):
    p = inputs.tiny_config(seed=0, quantized=True)
    got, _ = _gpu_scores(dsa, p)
    ref = O.index_scores(p)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(got[r, :n], ref[r]), f"row {r}"
        assert np.isnan(got[r, n:]).all()   # past q_pos: untouched


def test_scores_exact_on_tie_class_inputs_bf16(dsa):
    p = inputs.decode_config([5000, 4097, 3, 700], seed=1, tie_levels=8, k=2048)
    got, _ = _gpu_scores(dsa, p)
    ref = O.index_scores(p)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(got[r, :n], ref[r]), f"row {r}"


@pytest.mark.parametrize("case", ["tiny", "bf16", "bf16-h32", "fp8", "fp8-boost"])
def test_scores_within_error_bound(dsa, case):
    if case == "tiny":
        p = inputs.tiny_config(seed=3)
    elif case == "bf16":
        p = inputs.decode_config([3000, 4096, 5000, 65], seed=2, k=2048)
    elif case == "bf16-h32":
        p = inputs.decode_config([3001, 1000], seed=2, H_I=32, k=2048)
    elif case == "fp8":
        p = inputs.decode_config([3000, 4100, 129], seed=4, key_dtype="fp8_e4m3", k=2048)
    else:
        p = inputs.decode_config([6000, 2500], seed=5, key_dtype="fp8_e4m3", boost_frac=0.02, k=2048)
    _say("scores", case)
    got, _ = _gpu_scores(dsa, p)
    for r in range(p.R):
        C.assert_scores_close(p, r, got[r])


@pytest.mark.parametrize("key_dtype,lens", [
    ("bf16", [70000, 66000, 300]),       # up to 64 rows: the length-balanced split
    ("fp8_e4m3", [70000, 66000, 300]),
    ("bf16", [3000] * 80),               # more rows: the (query, key chunk) grid
    ("fp8_e4m3", [3000] * 79 + [40]),
])
def test_scores_several_groups_per_wave_and_negative_fp8_scales(dsa, key_dtype, lens):
    """Rows long enough that each wave of the decode-form indexer streams
    several 64-key groups (a tile's products multiplied while the previous
    tile's epilogue runs), in both grid forms; fp8 keys with a tenth of the
    row scales negated (relu(scale * dot) per head there). Scores within the
    bound of the oracle's, through both the q_pos and the seq_len entry."""
    import torch
    fp8 = key_dtype == "fp8_e4m3"
    p = inputs.decode_config(lens, seed=90 + len(lens), k=2048, key_dtype=key_dtype,
                             boost_frac=0.02 if fp8 else 0.0)
    if fp8:
        rng = np.random.default_rng(len(lens))
        neg = rng.random(p.k_scale.shape[0]) < 0.1
        p.k_scale = np.where(neg, p.k_scale | np.uint16(0x8000), p.k_scale).astype(np.uint16)
    _say("scores, several groups per wave", key_dtype, len(lens), "rows")
    got, d = _gpu_scores(dsa, p)
    dec = dsa.dsa_index_scores_decode(d.q_idx, d.head_w, d.k_idx, d.row_off, d.seq_len, int(p.seq_len.max()),
                                      k_scale=d.k_scale)
    torch.cuda.synchronize()
    dec = dec.cpu().numpy()
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        C.assert_scores_close(p, r, got[r])
        assert np.array_equal(dec[r, :n], got[r, :n]), f"row {r}: the two entries differ"


def test_read_probe_reads_every_piece_once(dsa):
    """The streaming-read reference (a measurement aid beside the indexer's
    roofline) reads each 16-byte piece once: the workgroups' sums add up to
    the buffer's, for a size that is no multiple of the grid's sweep."""
    import torch
    n = (1 << 20) + 12
    x = torch.arange(n, dtype=torch.float32, device="cuda") % 7   # small integers: fp32 sums are exact
    out = dsa.dsa_read_probe(x)
    torch.cuda.synchronize()
    assert out.numel() == dsa.lib.dsa_read_probe_blocks()
    assert float(out.double().sum()) == float(x.double().sum())


def test_fp8_codes_decode_exactly(dsa):
    # Row s holds code (s*128 + d) mod 256 in dim d: every code appears. Two
    # heads read dim d with signs +1/-1 and weights 1 and 0.5, so the score is
    # v (v >= 0) or -0.5 v (v < 0) for the decoded value v = e4m3(code) * scale.
    D = 128
    codes = ((np.arange(2)[:, None] * 128 + np.arange(D)[None, :]) % 256).astype(np.uint8)
    codes = np.repeat(codes, 64, axis=0)                     # 128 keys
    bad = (codes & 0x7F) == 0x7F                              # NaN codes
    codes[bad] = 0
    n = codes.shape[0]
    R = D
    q = np.zeros((R, 2, D), np.float32)
    for r in range(R):
        q[r, 0, r] = 1.0
        q[r, 1, r] = -1.0
    q_bits = inputs.f32_to_bf16_bits(q)
    scale = inputs.f32_to_bf16_bits(np.full(n, 0.5, np.float32))
    p = inputs.DSAProblem(
        name="fp8-codes", q_idx=q_bits, head_w=np.tile(np.array([[1.0, 0.5]], np.float32), (R, 1)),
        k_idx=codes, k_scale=scale, q_abs=np.zeros((R, 1, 576), np.uint16),
        latent=np.zeros((n, 576), np.uint16), row_off=np.zeros(1, np.int64),
        seq_len=np.array([n], np.int32), q_seq=np.zeros(R, np.int32),
        q_pos=np.full(R, n - 1, np.int32), k=8, scale=1.0, act_dtype="bf16", key_dtype="fp8_e4m3")
    got, _ = _gpu_scores(dsa, p)
    ref = O.index_scores(p)
    for r in range(R):
        assert np.array_equal(got[r, :n], ref[r]), f"dim {r}"


# ------------------------------------------------------------------------------
# sparse attention
# ------------------------------------------------------------------------------

def _gpu_attn(dsa, prob, idx, d=None):
    import torch
    d = d or inputs.to_torch(prob)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).cuda()
    out = torch.full((prob.R, prob.H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((prob.R, prob.H), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, idx_d, prob.scale, latent_scale=d.latent_scale,
                            q_seq=d.q_seq, out=out, lse=lse)
    return out.cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("H,k,std", [(64, 2048, 1.0), (64, 2048, 30.0), (8, 64, 1.0), (72, 256, 1.0),
                                     (128, 512, 3.0), (16, 1, 1.0), (64, 100, 1.0)])
def test_attention_matches_oracle(dsa, H, k, std):
    p = inputs.decode_config([3000, 2500, 4096], seed=6, H=H, k=k, q_abs_std=std)
    rng = np.random.default_rng(H * 7 + k)
    idx = np.full((p.R, k), -1, np.int32)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        m = min(k, n) if r != 1 else min(k, n) // 2 + (k == 1)   # row 1: a ragged -1 tail
        idx[r, :m] = rng.choice(n, size=m, replace=False)
    _say("attention", H, k, std)
    out, lse = _gpu_attn(dsa, p, idx)
    ref, lse_ref = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref, lse, lse_ref)


def test_attention_holes_and_empty_rows(dsa):
    p = inputs.decode_config([3000, 2500, 4096, 100], seed=7, H=64, k=2048)
    rng = np.random.default_rng(0)
    idx = rng.integers(0, 100, (p.R, 2048)).astype(np.int32)
    idx[rng.random(idx.shape) < 0.3] = -1      # holes anywhere, duplicates allowed
    idx[3] = -1                                # a row with no valid key
    out, lse = _gpu_attn(dsa, p, idx)
    ref, lse_ref = O.sparse_mla(p, idx)
    assert (out[3] == 0).all() and np.isneginf(lse[3]).all()
    C.assert_attn_close(out[:3], ref[:3], lse[:3], lse_ref[:3])


def test_attention_missing_keys_never_touch_other_rows(dsa):
    """A missing key (-1: a hole, a row shorter than k, the chunk tail past a
    split's end) contributes exactly nothing: the gather writes zeros for it
    instead of loading a cache row. Every sequence's position 0 (cache row 0
    among them) and a row past every sequence hold NaN and are never selected,
    so a missing key that read any of them would turn the outputs into NaN."""
    p = inputs.decode_config([3000, 2500, 4096, 100], seed=11, H=64, k=2048)
    nan_bf16 = np.uint16(0x7FC0)
    for b in range(p.B):
        p.latent[int(p.row_off[b])] = nan_bf16
    p.latent = np.concatenate([p.latent, np.full((1, 576), nan_bf16, np.uint16)])
    rng = np.random.default_rng(5)
    idx = np.full((p.R, 2048), -1, np.int32)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        m = min(2048, n - 1) if r != 1 else 700           # row 1: a ragged -1 tail inside a chunk
        idx[r, :m] = 1 + rng.choice(n - 1, size=m, replace=False)
    idx[rng.random(idx.shape) < 0.2] = -1                   # holes anywhere
    idx[3] = -1                                             # a row with no valid key
    _say("attention missing keys, NaN rows unselected")
    out, lse = _gpu_attn(dsa, p, idx)
    ref, lse_ref = O.sparse_mla(p, idx)
    assert np.isfinite(out).all() and np.isfinite(lse[:3]).all()
    assert (out[3] == 0).all() and np.isneginf(lse[3]).all()
    C.assert_attn_close(out[:3], ref[:3], lse[:3], lse_ref[:3])


@pytest.mark.parametrize("std,k", [(1.0, 512), (30.0, 512), (3.0, 200)])
def test_attention_many_queries_matches_oracle(dsa, std, k):
    """Enough queries for the one-workgroup-per-query (all heads) kernel:
    several 64-key chunks, holes anywhere, one empty row, a peaked softmax
    (q_abs std 30) and a key count that leaves a partial last chunk."""
    p = inputs.decode_config([600] * 160, seed=12, H=64, k=k, q_abs_std=std)
    rng = np.random.default_rng(int(std * 10) + k)
    idx = np.full((p.R, k), -1, np.int32)
    for r in range(p.R):
        idx[r] = rng.choice(600, size=k, replace=False)
    idx[rng.random(idx.shape) < 0.2] = -1      # holes anywhere
    idx[5] = -1                                # a row with no valid key
    idx[7, k // 2:] = -1                       # a row whose selection stops half way
    out, lse = _gpu_attn(dsa, p, idx)
    rows = [0, 5, 7, 80, p.R - 1]
    ref, lse_ref = O.sparse_mla(p, idx[rows], rows=rows)
    assert (out[5] == 0).all() and np.isneginf(lse[5]).all()
    keep = [0, 2, 3, 4]
    C.assert_attn_close(out[rows][keep], ref[keep], lse[rows][keep], lse_ref[keep])


@pytest.mark.parametrize("k", [2048, 512, 100])
def test_attention_many_query_batches_agree_bitwise(dsa, k):
    """More queries than CUs (the all-heads kernel, 750 queries): every row
    must equal, bit for bit, the same row computed in a batch of 150-200
    rows (a row's result may not depend on which workgroup or batch
    position computes it), and sampled rows the oracle. Planted: empty rows,
    rows of one, two and three chunks, holes, and a row whose only key sits
    at the last position."""
    import torch
    p = inputs.decode_config([1200] * 150, seed=21, H=64, k=k, tokens_per_seq=5)
    R = p.R
    rng = np.random.default_rng(k)
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):
        n = int(p.q_pos[r]) + 1
        m = min(k, n)
        idx[r, :m] = rng.choice(n, size=m, replace=False)
    idx[rng.random(idx.shape) < 0.1] = -1
    idx[R - 1 - 256] = -1                       # empty, second of workgroup 0
    idx[R - 2 - 256, 1:] = -1                   # one chunk
    idx[R - 3 - 256, 100:] = -1                 # two chunks (k permitting)
    idx[R - 4 - 256, 150:] = -1                 # three chunks
    idx[R - 5] = -1                             # empty, first of workgroup 4
    idx[R - 6, :] = -1
    idx[R - 6, k - 1] = 7                       # a single key, at the last position
    idx[R - 7, 5:] = -1                         # short first query
    d = inputs.to_torch(p)
    out, lse = _gpu_attn(dsa, p, idx, d)
    assert (out[R - 1 - 256] == 0).all() and np.isneginf(lse[R - 1 - 256]).all()
    assert (out[R - 5] == 0).all() and np.isneginf(lse[R - 5]).all()
    # one query per workgroup: slices of 150-200 rows (still the all-heads kernel)
    idx_d = torch.from_numpy(idx).cuda()
    for lo in range(0, R, 200):
        hi = min(R, lo + 200)
        o_s = torch.full((hi - lo, p.H, 512), float("nan"), dtype=torch.float32, device="cuda")
        l_s = torch.full((hi - lo, p.H), float("nan"), dtype=torch.float32, device="cuda")
        dsa.dsa_sparse_mla_attn(d.q_abs[lo:hi], d.latent, d.row_off, idx_d[lo:hi], p.scale,
                                q_seq=d.q_seq[lo:hi], out=o_s, lse=l_s)
        assert np.array_equal(o_s.cpu().numpy(), out[lo:hi], equal_nan=True), f"rows {lo}..{hi}"
        assert np.array_equal(l_s.cpu().numpy(), lse[lo:hi], equal_nan=True), f"rows {lo}..{hi}"
    rows = [0, 1, R // 2, R - 1, R - 2, R - 2 - 256, R - 3 - 256, R - 4 - 256, R - 6, R - 7, R - 1 - 512]
    ref, lse_ref = O.sparse_mla(p, idx[rows], rows=rows)
    C.assert_attn_close(out[rows], ref, lse[rows], lse_ref)


# ------------------------------------------------------------------------------
# whole path
# ------------------------------------------------------------------------------

def _pipeline(dsa, p):
    """index_scores -> topk -> sparse_mla through the three entry points."""
    import torch
    scores, d = _gpu_scores(dsa, p)
    s_d = torch.from_numpy(scores).cuda()
    idx = torch.full((p.R, p.k), 12345, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(s_d, d.q_pos, p.max_n, p.k, idx_out=idx)
    out, lse = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, idx, p.scale, latent_scale=d.latent_scale,
                                       q_seq=d.q_seq)
    return scores, idx.cpu().numpy(), out.cpu().numpy(), lse.cpu().numpy()


def test_tiny_pipeline_fp32(dsa):
    p = inputs.tiny_config(seed=0)
    scores, idx, out, lse = _pipeline(dsa, p)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        ref, bound = C.assert_scores_close(p, r, scores[r])
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k))
        C.near_tie_swaps(idx[r], O.topk_row(ref.astype(np.float32), p.k), ref, bound)
    ref_o, ref_l = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref_o, lse, ref_l, fp32=True)


def test_tiny_quantized_pipeline_is_exact_end_to_end(dsa):
    p = inputs.tiny_config(seed=0, quantized=True)
    scores, idx, out, lse = _pipeline(dsa, p)
    _, ref_idx, ref_o, ref_l = O.dsa_forward(p)
    assert np.array_equal(idx, ref_idx)
    C.assert_attn_close(out, ref_o, lse, ref_l, fp32=True)


def _fused(dsa, p, d, ws=None):
    import torch
    out = torch.full((p.B, p.H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((p.B, p.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((p.B, p.k), 777, dtype=torch.int32, device="cuda")
    dsa.dsa_decode_fused(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len,
                         int(p.seq_len.max()), p.k, p.scale, k_scale=d.k_scale, latent_scale=d.latent_scale,
                         out=out, lse=lse, idx_out=idx, workspace=ws)
    return out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy()


@pytest.mark.parametrize("key_dtype", ["bf16", "fp8_e4m3"])
def test_fused_decode_matches_entry_points_and_oracle(dsa, key_dtype):
    p = inputs.decode_config([4096, 3000, 2049, 1500, 7001], seed=8, k=2048, key_dtype=key_dtype,
                             boost_frac=0.02 if key_dtype == "fp8_e4m3" else 0.0)
    d = inputs.to_torch(p)
    out, lse, idx = _fused(dsa, p, d)
    scores, idx2, out2, lse2 = _pipeline(dsa, p)
    # the fused step enqueues the same kernels: identical bits
    assert np.array_equal(idx, idx2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    swaps = 0
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k))
        ref, bound = C.assert_scores_close(p, r, scores[r])
        swaps += C.near_tie_swaps(idx[r], O.topk_row(ref.astype(np.float32), p.k), ref, bound)
    _say("near-tie swaps vs oracle scores:", swaps)
    ref_o, ref_l = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)


def test_fused_decode_repeatable_and_replayable(dsa):
    import torch
    p = inputs.decode_config([8192, 8192, 6000, 8192], seed=9, tie_levels=8, k=2048)
    d = inputs.to_torch(p)
    runs = [_fused(dsa, p, d) for _ in range(3)]
    for o, l, i in runs[1:]:
        assert np.array_equal(o, runs[0][0]) and np.array_equal(l, runs[0][1]) and np.array_equal(i, runs[0][2])
    out, lse, idx = runs[0]
    _, ref_idx, ref_o, ref_l = O.dsa_forward(p)
    assert np.array_equal(idx, ref_idx)            # exact scores: end-to-end equality
    rep_o, rep_l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, torch.from_numpy(idx).cuda(), p.scale)
    assert np.array_equal(rep_o.cpu().numpy(), out) and np.array_equal(rep_l.cpu().numpy(), lse)
    C.assert_attn_close(out, ref_o, lse, ref_l)


def test_fused_split_decode_replay_at_the_all_heads_boundary(dsa):
    """As many rows as half the CUs with one row past 8K: the fused step
    takes the split selection, and replaying its indices must run the same
    attention kernel (the all-heads one starts at more rows), bit for bit."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    R = cus // 2
    p = inputs.decode_config([8300] + [300] * (R - 1), seed=23, H=64, k=2048)
    d = inputs.to_torch(p)
    out, lse, idx = _fused(dsa, p, d)
    rep_o, rep_l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, torch.from_numpy(idx).cuda(), p.scale)
    assert np.array_equal(rep_o.cpu().numpy(), out) and np.array_equal(rep_l.cpu().numpy(), lse)
    rows = [0, 1, R - 1]
    ref_o, ref_l = O.sparse_mla(p, idx[rows], rows=rows)
    C.assert_attn_close(out[rows], ref_o, lse[rows], ref_l)


@pytest.mark.parametrize("lens,k", [([12000, 9000, 20000], 2048), ([30000], 1000),
                                    ([9000, 16385, 12000, 10000, 9001], 512)])
def test_fused_split_decode_matches_pipeline_and_replay(dsa, lens, k):
    """Contexts past 8K take the split selection fused with the attention
    (selection of each split's ranks, then attention over them, in one
    workgroup): the same bits as the three entry points and as replaying the
    recorded indices; k = 1000 leaves a partial last chunk."""
    import torch
    p = inputs.decode_config(lens, seed=11, k=k)
    d = inputs.to_torch(p)
    out, lse, idx = _fused(dsa, p, d)
    scores, idx2, out2, lse2 = _pipeline(dsa, p)
    assert np.array_equal(idx, idx2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k)), f"row {r}"
    rep_o, rep_l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, torch.from_numpy(idx).cuda(), p.scale)
    assert np.array_equal(rep_o.cpu().numpy(), out) and np.array_equal(rep_l.cpu().numpy(), lse)
    rows = [0, p.R - 1]
    ref_o, ref_l = O.sparse_mla(p, idx[rows], rows=rows)
    C.assert_attn_close(out[rows], ref_o, lse[rows], ref_l)


def test_fused_split_decode_whole_window_with_tie_classes(dsa):
    """64 queries over 8,200 keys: one attention split per query, so each
    fused workgroup selects all 2,048 ranks itself. Keys drawn from 100
    prototypes make about 100 score classes of ~80 keys each, so a window
    meets more dense buckets than one bucket pass lists and the selection
    takes its general form (candidates gathered, then sorted). Indices equal
    the stable order of the scores; the fused step equals the entry points."""
    p = inputs.decode_config([8200] * 64, seed=12, tie_levels=100, k=2048)
    d = inputs.to_torch(p)
    out, lse, idx = _fused(dsa, p, d)
    scores, idx2, out2, lse2 = _pipeline(dsa, p)
    assert np.array_equal(idx, idx2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k)), f"row {r}"


def _bad_entries(idx, q_pos):
    """numpy count of what dsa_check_indices counts (test-side restatement of
    the structure a top-k index array must have)."""
    bad = 0
    R, k = idx.shape
    for r in range(R):
        n = int(q_pos[r]) + 1
        ke = max(0, min(k, n))
        head = idx[r, :ke]
        ok = (head >= 0) & (head < n)
        bad += int((~ok).sum())
        vals = np.sort(head[ok])
        bad += int((vals[1:] == vals[:-1]).sum())
        bad += int((idx[r, ke:] != -1).sum())
    return bad


def test_check_indices_counts_planted_faults(dsa):
    """The validator finds nothing in a real fused-decode index array, and
    counts exactly the entries planted wrong: out of range, repeated, wrong
    padding, a negative position, a row with no candidates."""
    import torch
    p = inputs.decode_config([3000, 2049, 700, 5000], seed=13, k=2048)
    d = inputs.to_torch(p)
    _, _, idx = _fused(dsa, p, d)
    q_pos = torch.from_numpy(p.q_pos.astype(np.int32)).cuda()
    assert int(dsa.dsa_check_indices(torch.from_numpy(idx).cuda(), q_pos).item()) == 0
    bad = idx.copy()
    bad[0, 5] = bad[0, 9]            # repeat
    bad[0, 10] = 3000                # out of range (n = 3000)
    bad[1, 0] = -3                   # negative
    bad[2, 700] = 7                  # padding that is not -1
    bad[2, 701] = 8
    bad[3, 100] = bad[3, 101] = bad[3, 102]  # two repeats of one value
    want = _bad_entries(bad, p.q_pos)
    assert want == 7
    got = dsa.dsa_check_indices(torch.from_numpy(bad).cuda(), q_pos)
    assert int(got.item()) == want
    # accumulation across calls, and q_pos < 0 (every entry must be -1)
    neg = torch.full((1, 64), -1, dtype=torch.int32, device="cuda")
    neg[0, 3] = 0
    acc = dsa.dsa_check_indices(neg, torch.tensor([-1], dtype=torch.int32, device="cuda"), n_bad=got)
    assert int(acc.item()) == want + 1


# ------------------------------------------------------------------------------
# causal prefill form (one sequence, a query per position)
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("T,H_I,D_I", [(777, 64, 128), (300, 32, 64), (100, 16, 128), (40, 64, 64)])
def test_prefill_form_scores_topk_attention(dsa, T, H_I, D_I):
    """Every row's scores within the bound of the oracle (this form runs the
    multi-query indexer: 8 rows per workgroup sharing the key tiles), top-k
    equal to the stable order of those scores, attention on a few rows."""
    import torch
    p = inputs.prefill_config(T, seed=3, H_I=H_I, D_I=D_I, k=64)
    d = inputs.to_torch(p)
    sentinel = -12345.5
    s_d = torch.full((T, (T + 3) // 4 * 4), sentinel, dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, d.row_off, d.q_pos, T, q_seq=d.q_seq, scores=s_d)
    idx_d = dsa.dsa_topk(s_d, d.q_pos, T, p.k)
    scores, idx = s_d.cpu().numpy(), idx_d.cpu().numpy()
    ref_rows = O.index_scores(p)
    for r in range(p.R):
        n = r + 1
        ref = ref_rows[r].astype(np.float64)
        bound = C.score_bound(p, r, np.arange(n), ref)
        assert not (np.abs(scores[r, :n] - ref) > bound).any(), f"row {r}"
        assert (scores[r, n:] == sentinel).all(), f"row {r}: entries past q_pos written"
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k)), f"row {r}"
    rows = [0, 1, T // 2, T - 1]
    out, lse = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, idx_d, p.scale, q_seq=d.q_seq)
    ref_o, ref_l = O.sparse_mla(p, idx[rows], rows=rows)
    C.assert_attn_close(out.cpu().numpy()[rows], ref_o, lse.cpu().numpy()[rows], ref_l)


# ------------------------------------------------------------------------------
# FP8 latent cache (e4m3 codes, one float32 scale per row)
# ------------------------------------------------------------------------------

def _fp8_attn_problem(lens, seed, H, k, std=1.0, scale_spread=0.0):
    p = inputs.decode_config(lens, seed=seed, H=H, k=k, q_abs_std=std, latent_dtype="fp8_e4m3")
    if scale_spread:
        rng = np.random.default_rng(seed)
        p.latent_scale = (p.latent_scale * 10.0 ** rng.uniform(-scale_spread, scale_spread,
                                                               p.latent_scale.shape)).astype(np.float32)
    return p


@pytest.mark.parametrize("H,k,std,spread", [(64, 2048, 1.0, 0.0), (64, 2048, 30.0, 0.0), (8, 64, 1.0, 0.0),
                                            (72, 256, 1.0, 0.0), (16, 1, 1.0, 0.0), (64, 100, 1.0, 0.0),
                                            (64, 2048, 1.0, 1.0)])
def test_attention_fp8_latent_matches_oracle(dsa, H, k, std, spread):
    """fp8 rows: ragged tails, partial chunks, H not a multiple of 16, a
    peaked softmax, and row scales spread over two decades either way."""
    p = _fp8_attn_problem([3000, 2500, 4096], 16, H, k, std, spread)
    rng = np.random.default_rng(H * 5 + k)
    idx = np.full((p.R, k), -1, np.int32)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        m = min(k, n) if r != 1 else min(k, n) // 2 + (k == 1)
        idx[r, :m] = rng.choice(n, size=m, replace=False)
    _say("fp8 attention", H, k, std, spread)
    out, lse = _gpu_attn(dsa, p, idx)
    ref, lse_ref = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref, lse, lse_ref)


def test_attention_fp8_latent_holes_empty_rows_and_many_queries(dsa):
    p = _fp8_attn_problem([600] * 160, 17, 64, 512)
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(600, size=512, replace=False) for _ in range(p.R)]).astype(np.int32)
    idx[rng.random(idx.shape) < 0.2] = -1
    idx[5] = -1
    idx[7, 256:] = -1
    idx[9, :] = 123                            # one key repeated: every entry counts
    out, lse = _gpu_attn(dsa, p, idx)
    rows = [0, 5, 7, 9, 80, p.R - 1]
    ref, lse_ref = O.sparse_mla(p, idx[rows], rows=rows)
    assert (out[5] == 0).all() and np.isneginf(lse[5]).all()
    keep = [0, 2, 3, 4, 5]
    C.assert_attn_close(out[rows][keep], ref[keep], lse[rows][keep], lse_ref[keep])


@pytest.mark.parametrize("lens,k", [([4096, 3000, 2049, 1500, 7001], 2048), ([12000, 9000, 20000], 2048),
                                    ([9000, 16385, 12000, 10000, 9001], 512)])
def test_fused_decode_fp8_latent_matches_pipeline_replay_and_oracle(dsa, lens, k):
    """Short contexts take selection then the attention kernel; past 8K the
    selection is fused with the attention: both give the bits of the three
    entry points and of replaying the recorded indices."""
    import torch
    p = inputs.decode_config(lens, seed=18, k=k, latent_dtype="fp8_e4m3")
    d = inputs.to_torch(p)
    out, lse, idx = _fused(dsa, p, d)
    out_b, lse_b, idx_b = _fused(dsa, p, d)
    assert np.array_equal(out, out_b) and np.array_equal(lse, lse_b) and np.array_equal(idx, idx_b)
    scores, idx2, out2, lse2 = _pipeline(dsa, p)
    assert np.array_equal(idx, idx2)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k)), f"row {r}"
    rep_o, rep_l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, torch.from_numpy(idx).cuda(), p.scale,
                                           latent_scale=d.latent_scale)
    assert np.array_equal(rep_o.cpu().numpy(), out) and np.array_equal(rep_l.cpu().numpy(), lse)
    ref_o, ref_l = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)


# ------------------------------------------------------------------------------
# multi-token decode: several new tokens per sequence in one fused step
# ------------------------------------------------------------------------------

def _fused_multi(dsa, p, d):
    """The fused step for p.tokens_per_seq tokens per sequence; also returns
    the scores it left in its workspace (region 0: [R, ld] fp32)."""
    import torch
    m = p.tokens_per_seq
    max_len = int(p.seq_len.max())
    nbytes = dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, p.R, max_len, p.k, p.H)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((p.R, p.H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((p.R, p.H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((p.R, p.k), 777, dtype=torch.int32, device="cuda")
    dsa.dsa_decode_fused(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len, max_len, p.k,
                         p.scale, k_scale=d.k_scale, latent_scale=d.latent_scale, q_per_seq=m, out=out, lse=lse,
                         idx_out=idx, workspace=ws)
    torch.cuda.synchronize()
    ld = (max_len + 3) // 4 * 4
    scores = ws[:p.R * ld * 4].view(torch.float32).reshape(p.R, ld).cpu().numpy().copy()
    return out.cpu().numpy(), lse.cpu().numpy(), idx.cpu().numpy(), scores


@pytest.mark.parametrize("m,lens,key_dtype,latent_dtype", [
    (4, [4096, 3000, 2049, 700], "bf16", "bf16"),          # selection, then the attention kernel
    (4, [12000, 9000, 20000], "bf16", "bf16"),              # selection fused with the attention
    (2, [9000, 16385, 12000], "bf16", "fp8_e4m3"),
    (3, [5000, 8200, 4], "bf16", "bf16"),                   # idle wave; a sequence of 4 tokens
    (8, [10000, 2500], "bf16", "bf16"),                     # eight waves, one per token
    (2, [700] * 66 + [3000], "bf16", "bf16"),               # over 64 sequences: the (slice, sequence) grid
    (2, [700] * 66 + [3000], "fp8_e4m3", "bf16"),
    (4, [9000, 3000], "fp8_e4m3", "bf16"),                  # fp8 keys in the shared key stream
])
def test_fused_multi_token_decode(dsa, m, lens, key_dtype, latent_dtype):
    """Each token selects its own top-k over its own causal range: indices equal
    the stable order of the step's own scores, scores within the bound of the
    oracle, attention within tolerance, two runs and an index replay bitwise
    equal."""
    import torch
    p = inputs.decode_config(lens, seed=21 + m, k=2048, key_dtype=key_dtype, latent_dtype=latent_dtype,
                             boost_frac=0.02 if key_dtype == "fp8_e4m3" else 0.0, tokens_per_seq=m)
    d = inputs.to_torch(p)
    out, lse, idx, scores = _fused_multi(dsa, p, d)
    out2, lse2, idx2, _ = _fused_multi(dsa, p, d)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2) and np.array_equal(idx, idx2)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    swaps = 0
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k)), f"row {r}"
        ref, bound = C.assert_scores_close(p, r, scores[r])
        swaps += C.near_tie_swaps(idx[r], O.topk_row(ref.astype(np.float32), p.k), ref, bound)
    _say(f"multi-token m={m}: near-tie swaps {swaps}")
    # the decode-form indexer entry runs the step's indexer: the same scores
    alone = dsa.dsa_index_scores_decode(d.q_idx, d.head_w, d.k_idx, d.row_off, d.seq_len, int(p.seq_len.max()),
                                        q_per_seq=m, k_scale=d.k_scale).cpu().numpy()
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(alone[r, :n], scores[r, :n]), f"row {r}"
    rep_o, rep_l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, torch.from_numpy(idx).cuda(), p.scale,
                                           latent_scale=d.latent_scale, q_seq=d.q_seq)
    assert np.array_equal(rep_o.cpu().numpy(), out) and np.array_equal(rep_l.cpu().numpy(), lse)
    ref_o, ref_l = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)


def test_fused_multi_token_exact_scores_end_to_end(dsa):
    """Tie-class inputs (every score exact in fp32): the shared-key-stream
    scores equal the oracle's bit for bit and the indices end to end."""
    p = inputs.decode_config([9000, 6000, 12000], seed=31, k=2048, tie_levels=8, tokens_per_seq=4)
    d = inputs.to_torch(p)
    out, lse, idx, scores = _fused_multi(dsa, p, d)
    ref_scores, ref_idx, ref_o, ref_l = O.dsa_forward(p)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(scores[r, :n], ref_scores[r]), f"row {r}"
    assert np.array_equal(idx, ref_idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)


# ------------------------------------------------------------------------------
# context parallelism over key ranges, rehearsed with P shards on one device
# ------------------------------------------------------------------------------

def _cp_step(dsa, p, d, P):
    """Each shard scores its own keys, selects locally and lists its candidates;
    the merged lists give the selection; each shard attends over the winners
    it holds; the partial outputs are merged."""
    import torch
    max_len = int(p.seq_len.max())
    edges = [int(x) // 64 * 64 for x in np.linspace(0, max_len, P + 1)]
    edges[-1] = max_len
    q_pos = d.q_pos.long()
    ps, pi, shards = [], [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        off = (d.row_off + lo).contiguous()
        qp = (torch.minimum(q_pos, torch.full_like(q_pos, hi - 1)) - lo).to(torch.int32).contiguous()
        sc = dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, off, qp, hi - lo, k_scale=d.k_scale)
        loc = dsa.dsa_topk(sc, qp, hi - lo, p.k)
        a, b = dsa.dsa_topk_pairs(sc, loc, lo)
        ps.append(a)
        pi.append(b)
        shards.append((lo, hi, off))
    ps = torch.stack(ps).contiguous()
    pi = torch.stack(pi).contiguous()
    idx = dsa.dsa_topk_merge(ps, pi)
    o_parts, l_parts = [], []
    for lo, hi, off in shards:
        loc = dsa.dsa_shard_indices(idx, lo, hi)
        o, l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, off, loc, p.scale, latent_scale=d.latent_scale,
                                       q_seq=d.q_seq)
        o_parts.append(o)
        l_parts.append(l)
    o_parts = torch.stack(o_parts).contiguous()
    l_parts = torch.stack(l_parts).contiguous()
    out, lse = dsa.dsa_attn_merge(o_parts, l_parts)
    torch.cuda.synchronize()
    return (ps.cpu().numpy(), pi.cpu().numpy(), idx.cpu().numpy(), o_parts.cpu().numpy(), l_parts.cpu().numpy(),
            out.cpu().numpy(), lse.cpu().numpy())


@pytest.mark.parametrize("P,lens,tie_levels", [(2, [9000, 5000], 0), (4, [32768, 20000, 6000], 0),
                                               (8, [16385, 12000, 900], 8), (3, [7000, 700], 0)])
def test_context_parallel_rehearsal(dsa, P, lens, tie_levels):
    """The merged selection equals the unsharded top-k bit for bit (and the
    oracle's merge of the same lists); the merged output equals the oracle's
    merge of the same partial outputs and the attention over the selection
    within the attention tolerances; two runs are bitwise equal."""
    import torch
    p = inputs.decode_config(lens, seed=41 + P, k=2048, tie_levels=tie_levels)
    d = inputs.to_torch(p)
    max_len = int(p.seq_len.max())
    ps, pi, idx, o_parts, l_parts, out, lse = _cp_step(dsa, p, d, P)
    full = dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, d.row_off, d.q_pos, max_len, k_scale=d.k_scale)
    idx_full = dsa.dsa_topk(full, d.q_pos, max_len, p.k).cpu().numpy()
    assert np.array_equal(idx, idx_full)
    for r in range(p.R):
        assert np.array_equal(idx[r], O.topk_merge(ps[:, r], pi[:, r], p.k)), f"row {r}"
    C.assert_index_invariants(idx, p.q_pos, p.k)
    for r in range(p.R):
        ref_o, ref_l = O.attn_merge(o_parts[:, r], l_parts[:, r])
        C.assert_attn_close(out[r:r + 1], ref_o[None], lse[r:r + 1], ref_l[None], fp32=True)
    ref_o, ref_l = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)
    again = _cp_step(dsa, p, d, P)
    assert np.array_equal(again[2], idx) and np.array_equal(again[5], out) and np.array_equal(again[6], lse)


def test_topk_merge_matches_oracle_on_random_lists(dsa):
    """Lists of every length up to k, ties across lists, signed zeros."""
    import torch
    rng = np.random.default_rng(3)
    P, R, k = 5, 6, 512
    ps = np.full((P, R, k), -np.inf, np.float32)
    pi = np.full((P, R, k), -1, np.int32)
    for r in range(R):
        keys = rng.permutation(P * 4000)[:P * k]
        for q in range(P):
            m = int(rng.integers(0, k + 1)) if r % 2 else k
            s = (rng.integers(-3, 4, m) / 2.0).astype(np.float32)
            s[s == 0] = np.where(rng.random((s == 0).sum()) < 0.5, np.float32(0.0), np.float32(-0.0))
            kk = keys[q * k:q * k + m]
            order = np.lexsort((kk, -s.astype(np.float64)))
            ps[q, r, :m] = s[order]
            pi[q, r, :m] = kk[order]
    got = dsa.dsa_topk_merge(torch.from_numpy(ps).cuda(), torch.from_numpy(pi).cuda()).cpu().numpy()
    for r in range(R):
        assert np.array_equal(got[r], O.topk_merge(ps[:, r], pi[:, r], k)), f"row {r}"


# ------------------------------------------------------------------------------
# paged caches: a block table over a shuffled page pool
# ------------------------------------------------------------------------------

def _decode_run(dsa, p, d):
    import torch
    max_len = int(p.seq_len.max())
    call = dsa.DecodeCall(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len, max_len, p.k,
                          p.scale, k_scale=d.k_scale, latent_scale=d.latent_scale, q_per_seq=p.tokens_per_seq,
                          block_table=d.block_table, page_size=p.page_size)
    o, l, i = call()
    torch.cuda.synchronize()
    return o.cpu().numpy().copy(), l.cpu().numpy().copy(), i.cpu().numpy().copy()


@pytest.mark.parametrize("page,lens,key_dtype,latent_dtype", [
    (64, [12000, 9000, 20000], "bf16", "bf16"),            # selection fused with the attention
    (256, [4096, 3000, 700], "bf16", "bf16"),              # selection, then the attention kernel
    (128, [9000, 16385], "fp8_e4m3", "fp8_e4m3"),
    (64, [600] * 70, "bf16", "bf16"),                       # many rows
])
def test_paged_decode_equals_contiguous(dsa, page, lens, key_dtype, latent_dtype):
    """Where a key is stored does not change its arithmetic: the paged step
    gives the contiguous step's indices and outputs bit for bit, and so does
    the paged attention entry replaying the indices."""
    import torch
    p = inputs.decode_config(lens, seed=51, k=2048, key_dtype=key_dtype, latent_dtype=latent_dtype,
                             boost_frac=0.02 if key_dtype == "fp8_e4m3" else 0.0)
    q = inputs.paged_view(p, page_size=page, seed=5)
    o1, l1, i1 = _decode_run(dsa, p, inputs.to_torch(p))
    dq = inputs.to_torch(q)
    o2, l2, i2 = _decode_run(dsa, q, dq)
    assert np.array_equal(i1, i2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    rep_o, rep_l = dsa.dsa_sparse_mla_attn(dq.q_abs, dq.latent, None, torch.from_numpy(i2).cuda(), q.scale,
                                           latent_scale=dq.latent_scale, block_table=dq.block_table,
                                           page_size=page)
    assert np.array_equal(rep_o.cpu().numpy(), o2) and np.array_equal(rep_l.cpu().numpy(), l2)
    rows = [0, q.R - 1]
    ref_o, ref_l = O.sparse_mla(q, i2[rows], rows=rows)
    C.assert_attn_close(o2[rows], ref_o, l2[rows], ref_l)


def test_paged_multi_token_decode_matches_oracle(dsa):
    """Several new tokens per sequence on a paged cache (one key stream per
    token): indices equal the oracle's on tie-class inputs (exact scores)."""
    p = inputs.decode_config([9000, 6000], seed=52, k=2048, tie_levels=8, tokens_per_seq=3)
    q = inputs.paged_view(p, page_size=64, seed=6)
    o, l, i = _decode_run(dsa, q, inputs.to_torch(q))
    _, ref_idx, ref_o, ref_l = O.dsa_forward(q)
    assert np.array_equal(i, ref_idx)
    C.assert_attn_close(o, ref_o, l, ref_l)


# ------------------------------------------------------------------------------
# edge cases of the next rows
# ------------------------------------------------------------------------------

def test_edges_fp8_latent_128_heads(dsa):
    p = _fp8_attn_problem([5000, 3000], 61, 128, 2048, std=3.0)
    rng = np.random.default_rng(61)
    idx = np.stack([rng.choice(int(p.q_pos[r]) + 1, 2048, replace=False) for r in range(p.R)]).astype(np.int32)
    out, lse = _gpu_attn(dsa, p, idx)
    ref, lse_ref = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref, lse, lse_ref)


@pytest.mark.parametrize("m,k", [(5, 32), (2, 2048)])
def test_edges_multi_token(dsa, m, k):
    """Five tokens (the eight-wave shared ring), k below one chunk; two tokens."""
    p = inputs.decode_config([9000, 600, 5], seed=62 + m, k=k, tie_levels=8, tokens_per_seq=m)
    d = inputs.to_torch(p)
    out, lse, idx, scores = _fused_multi(dsa, p, d)
    ref_scores, ref_idx, ref_o, ref_l = O.dsa_forward(p)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        if n > 0:
            assert np.array_equal(scores[r, :n], ref_scores[r]), f"row {r}"
    assert np.array_equal(idx, ref_idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)


def test_edges_paged_large_pages(dsa):
    p = inputs.decode_config([9000, 5000, 2100], seed=63, k=2048)
    q = inputs.paged_view(p, page_size=1024, seed=7, spare_pages=1)
    o1, l1, i1 = _decode_run(dsa, p, inputs.to_torch(p))
    o2, l2, i2 = _decode_run(dsa, q, inputs.to_torch(q))
    assert np.array_equal(i1, i2) and np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_edges_context_parallel_one_shard(dsa):
    p = inputs.decode_config([9000, 3000], seed=64, k=2048)
    d = inputs.to_torch(p)
    ps, pi, idx, o_parts, l_parts, out, lse = _cp_step(dsa, p, d, 1)
    full = dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, d.row_off, d.q_pos, int(p.seq_len.max()))
    assert np.array_equal(idx, dsa.dsa_topk(full, d.q_pos, int(p.seq_len.max()), p.k).cpu().numpy())
    assert np.array_equal(out, o_parts[0]) and np.array_equal(lse, l_parts[0])   # one part: itself


@pytest.mark.parametrize("m,H_I,D_I,lens", [
    (4, 64, 128, [9000, 5000, 300]),
    (6, 64, 128, [9000, 5000, 300]),
    (2, 16, 64, [9000, 2500, 10]),      # one head tile, 64-d keys; a sequence shorter than a scale block
    (4, 32, 128, [9000, 2500, 10]),
    (3, 64, 64, [9000, 2500, 10]),
])
def test_multi_token_fp8_keys_with_negative_scales(dsa, m, H_I, D_I, lens):
    """fp8 keys in the shared-key-stream indexer, a tenth of the row scales
    negated (relu(scale * dot) per head there): scores within the bound of the
    oracle's, indices the stable order of the step's own scores. Every
    (heads, dim) instantiation of the kernel, and a sequence of 10 tokens."""
    p = inputs.decode_config(lens, seed=70 + m + H_I + D_I, k=2048, key_dtype="fp8_e4m3", boost_frac=0.02,
                             tokens_per_seq=m, H_I=H_I, D_I=D_I)
    rng = np.random.default_rng(m)
    neg = rng.random(p.k_scale.shape[0]) < 0.1
    p.k_scale = np.where(neg, p.k_scale | np.uint16(0x8000), p.k_scale).astype(np.uint16)
    d = inputs.to_torch(p)
    out, lse, idx, scores = _fused_multi(dsa, p, d)
    C.assert_index_invariants(idx, p.q_pos, p.k)
    for r in range(p.R):
        n = int(p.q_pos[r]) + 1
        assert np.array_equal(idx[r], O.topk_row(scores[r, :n], p.k)), f"row {r}"
        C.assert_scores_close(p, r, scores[r])
    ref_o, ref_l = O.sparse_mla(p, idx)
    C.assert_attn_close(out, ref_o, lse, ref_l)


def test_index_share_block_layers_over_recorded_indices(dsa):
    """A block of four layers sharing one selection (cross-layer index reuse,
    "Zhipu AI / GLM", section 11.1: one indexer per 4-layer block): layer 0
    runs the fused step and records its indices; layers 1..3, each with its
    own absorbed queries and latent cache, run the sparse attention over those
    indices. Every layer's output is checked against the oracle's attention
    over the recorded indices with that layer's own arrays; layer 0's indices
    equal the stable order of its own scores."""
    import torch
    lens = [12000, 9001, 700, 20000]
    layers = [inputs.decode_config(lens, seed=300 + l, k=2048) for l in range(4)]
    ds = [inputs.to_torch(p, "cuda") for p in layers]
    p0, d0 = layers[0], ds[0]
    max_len = int(p0.seq_len.max())
    out0, lse0, idx = dsa.dsa_decode_fused(d0.q_idx, d0.head_w, d0.k_idx, d0.q_abs, d0.latent, d0.row_off,
                                           d0.seq_len, max_len, p0.k, p0.scale)
    scores = dsa.dsa_index_scores(d0.q_idx, d0.head_w, d0.k_idx, d0.row_off, d0.q_pos, max_len)
    torch.cuda.synchronize()
    idx_np, sc = idx.cpu().numpy(), scores.cpu().numpy()
    for r in range(p0.R):
        n = int(p0.q_pos[r]) + 1
        assert np.array_equal(idx_np[r], O.topk_row(sc[r, :n], p0.k)), f"layer 0 row {r}"
    outs = [(out0.cpu().numpy(), lse0.cpu().numpy())]
    for l in range(1, 4):
        d = ds[l]
        o, ls = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, idx, layers[l].scale)
        torch.cuda.synchronize()
        outs.append((o.cpu().numpy(), ls.cpu().numpy()))
    for l, (o, ls) in enumerate(outs):
        ref_o, ref_l = O.sparse_mla(layers[l], idx_np)
        C.assert_attn_close(o, ref_o, ls, ref_l)
    # layers differ (their own arrays), so no layer's output can stand in for another's
    assert not np.array_equal(outs[1][0], outs[2][0])
