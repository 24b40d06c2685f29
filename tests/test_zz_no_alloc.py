"""The no-allocation decode entry (dsa_decode_fused_noalloc) against the
workspace entry (dsa_decode_fused): the same kernels, so the same bits, on
two calls in a row through the C ABI, the second one smaller (the shared
scratch keeps the first call's contents); a step too large for the scratch
is refused before anything is enqueued."""
import numpy as np
import pytest

from sparse_attention_05_amd import inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from sparse_attention_05_amd import dsa as mod
    return mod


def _step(dsa, p, d, noalloc):
    import torch
    max_len = int(p.seq_len.max())
    R, H = p.R, p.H
    out = torch.full((R, H, 512), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device="cuda")
    idx = torch.full((R, p.k), -7, dtype=torch.int32, device="cuda")
    fn = dsa.dsa_decode_fused_noalloc if noalloc else dsa.dsa_decode_fused
    fn(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len, max_len, p.k, p.scale,
       k_scale=d.k_scale, latent_scale=d.latent_scale, q_per_seq=p.tokens_per_seq, out=out, lse=lse, idx_out=idx)
    return out, lse, idx


@pytest.mark.parametrize("cases", [
    # (sequence lengths, tokens per sequence): the second call smaller than the first
    (([40000, 33000, 9000, 20000], 1), ([12000, 9001, 700], 1)),
    (([16384, 16384], 4), ([3000, 2500], 2)),
])
def test_noalloc_matches_workspace_entry(dsa, cases):
    import torch
    print(f"no-alloc decode, cases {cases}", flush=True)
    for i, (lens, m) in enumerate(cases):
        p = inputs.decode_config(lens, seed=11 + i, k=2048, tokens_per_seq=m)
        d = inputs.to_torch(p, "cuda:0")
        need = dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, p.R, int(p.seq_len.max()), p.k, p.H)
        assert need <= dsa.dsa_decode_noalloc_limit()
        ref = _step(dsa, p, d, noalloc=False)
        got = _step(dsa, p, d, noalloc=True)
        torch.cuda.synchronize()
        for name, a, b in zip(("out", "lse", "idx"), ref, got):
            assert torch.equal(a, b), f"call {i}: {name} differs from dsa_decode_fused"
        assert not torch.isnan(got[0]).any()
        assert (got[2] >= -1).all()


def test_noalloc_refuses_oversized_step(dsa):
    import torch
    p = inputs.decode_config([1000] * 16, seed=3, k=2048)
    d = inputs.to_torch(p, "cuda:0")
    max_len = 1 << 20
    assert dsa.dsa_workspace_size(dsa.DSA_ENTRY_DECODE, p.R, max_len, p.k, p.H) > dsa.dsa_decode_noalloc_limit()
    out = torch.full((p.R, p.H, 512), 5.0, dtype=torch.float32, device="cuda")
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_decode_fused_noalloc(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len, max_len,
                                     p.k, p.scale, out=out)
    assert e.value.status == dsa.DSA_ERR_WORKSPACE
    assert "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (out == 5.0).all()  # nothing was enqueued
