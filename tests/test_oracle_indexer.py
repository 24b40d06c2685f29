"""Pins of the oracle's indexer scores and storage decoders.

Decoders are checked against torch's own bf16 / float8_e4m3fn casts (a
library routine independent of the oracle) and the OCP E4M3FN spec points.
Scores are checked against a hand-worked case, closed forms that expose a
dropped ReLU, a wrong head-weight index, an off-by-one causal bound or a
missing fp8 row scale, and exact rational arithmetic on integer inputs.
"""
import json
import os
from fractions import Fraction

import numpy as np
import torch

from oracle import dsa_oracle as O
from sparse_attention_05_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3_decoder_matches_torch_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3fn_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert nan.sum() == 2  # 0x7F and 0xFF only


def test_e4m3_spec_points():
    pts = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
           0x38: 1.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in pts.items():
        assert O.e4m3fn_to_f64(np.array([c], np.uint8))[0] == v
    z = O.e4m3fn_to_f64(np.array([0x80], np.uint8))[0]
    assert z == 0.0 and np.signbit(z)


def test_bf16_decoder_matches_torch():
    rng = np.random.default_rng(1)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite only
    ours = O.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_golden_hand_case():
    g = json.load(open(os.path.join(GOLDEN, "indexer_hand.json")))
    q = np.asarray(g["q"], np.float64)
    w = np.asarray(g["w"], np.float64)
    keys = np.asarray(g["keys"], np.float64)
    got = O.index_scores_row(q, w, keys)
    assert got.dtype == np.float32
    assert got.tolist() == g["scores"]


def _problem(q, w, keys, q_pos, k_scale=None, key_dtype="f32"):
    q = np.asarray(q, np.float32)
    R = q.shape[0]
    keys = np.asarray(keys)
    rows = keys.shape[0]
    return inputs.DSAProblem(
        name="t", q_idx=q, head_w=np.asarray(w, np.float32), k_idx=keys, k_scale=k_scale,
        q_abs=np.zeros((R, 1, 576), np.float32), latent=np.zeros((rows, 576), np.float32),
        row_off=np.zeros(1, np.int64), seq_len=np.array([rows], np.int32),
        q_seq=np.zeros(R, np.int32), q_pos=np.asarray(q_pos, np.int32), k=4, scale=1.0,
        act_dtype="f32", key_dtype=key_dtype)


def test_closed_form_linear_keys():
    # k_s = s * e0, every head's query = e0, w = 1 -> S[s] = H_I * s
    H_I, D, n = 3, 8, 50
    keys = np.zeros((n, D), np.float32)
    keys[:, 0] = np.arange(n)
    q = np.zeros((1, H_I, D), np.float32)
    q[0, :, 0] = 1.0
    p = _problem(q, np.ones((1, H_I)), keys, [n - 1])
    s = O.index_scores(p)[0]
    assert s.tolist() == (H_I * np.arange(n)).astype(np.float32).tolist()


def test_relu_zeroes_negative_dots():
    H_I, D, n = 2, 4, 10
    keys = np.zeros((n, D), np.float32)
    keys[:, 0] = np.arange(1, n + 1)
    q = np.zeros((1, H_I, D), np.float32)
    q[0, :, 0] = -1.0
    p = _problem(q, np.full((1, H_I), 3.0), keys, [n - 1])
    assert (O.index_scores(p)[0] == 0.0).all()
    # one head positive, one negative: only the positive head's weight counts
    q[0, 1, 0] = 2.0
    p = _problem(q, np.array([[3.0, 0.5]]), keys, [n - 1])
    assert O.index_scores(p)[0].tolist() == (0.5 * 2.0 * keys[:, 0]).tolist()


def test_head_weights_follow_their_head():
    # distinct heads pick distinct key dims; w[r, h] must scale head h of row r
    D, n = 4, 4
    keys = np.eye(n, D, dtype=np.float32)
    q = np.zeros((2, 4, D), np.float32)
    for h in range(4):
        q[:, h, h] = 1.0
    w = np.array([[1, 10, 100, 1000], [2, 20, 200, 2000]], np.float32)
    p = _problem(q, w, keys, [3, 2])
    s = O.index_scores(p)
    assert s[0].tolist() == [1, 10, 100, 1000]
    assert s[1].tolist() == [2, 20, 200]


def test_causal_bound_includes_own_key():
    rng = np.random.default_rng(5)
    n = 30
    keys = rng.standard_normal((n, 8)).astype(np.float32)
    q = rng.standard_normal((3, 2, 8)).astype(np.float32)
    pos = [0, 17, 29]
    p = _problem(q, np.ones((3, 2)), keys, pos)
    s = O.index_scores(p)
    assert [len(x) for x in s] == [1, 18, 30]
    # score of the query's own key equals the score computed from that key alone
    for i, t in enumerate(pos):
        alone = O.index_scores_row(q[i].astype(np.float64), np.ones(2), keys[t:t + 1].astype(np.float64))
        assert s[i][t] == alone[0]


def test_fp8_keys_use_row_scale():
    # code 0x38 is 1.0; row s has scale 2^(s-3) -> key = 2^(s-3) * ones
    n, D = 6, 4
    codes = np.full((n, D), 0x38, np.uint8)
    scales = inputs.f32_to_bf16_bits(np.exp2(np.arange(n) - 3.0).astype(np.float32))
    q = np.ones((1, 1, D), np.float32)
    p = _problem(q, [[1.0]], codes, [n - 1], k_scale=scales, key_dtype="fp8_e4m3")
    s = O.index_scores(p)[0]
    assert s.tolist() == (D * np.exp2(np.arange(n) - 3.0)).tolist()


def _exact_score(q, w, key):
    tot = Fraction(0)
    for h in range(q.shape[0]):
        z = sum(Fraction(float(q[h, d])) * Fraction(float(key[d])) for d in range(q.shape[1]))
        if z > 0:
            tot += Fraction(float(w[h])) * z
    return tot


def test_exact_rational_on_integer_grid():
    p = inputs.tiny_config(seed=2, quantized=True)
    s = O.index_scores(p, rows=[0, 15])
    for i, r in enumerate([0, 15]):
        n = int(p.q_pos[r]) + 1
        for sidx in list(range(0, 12)) + list(range(n - 12, n)):
            exact = _exact_score(p.q_idx[r], p.head_w[r], p.k_idx[sidx])
            assert Fraction(float(s[i][sidx])) == exact
