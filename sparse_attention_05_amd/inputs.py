"""Seeded synthetic inputs for the DSA decode path.

This module only *makes* inputs: it draws seeded random numbers and stores
them in the formats the caches use on the device (fp32, bf16 bit patterns,
OCP fp8-e4m3 codes with a per-row bf16 scale). It holds none of the
method's arithmetic (no indexer scoring, no selection, no attention); the
oracle and the HIP path each decode these arrays with their own code.

Shapes and distributions follow the workloads the DSA pages describe:
a 576-d latent KV row per token (512 latent + 64 RoPE, "GLM-5: from Vibe
Coding to Agentic Engineering", section 2.1, Multi-latent Attention), a
128-d indexer key per token with 32 or 64 indexer heads ("Zhipu AI / GLM",
section 9.1, "DSA index 32x128, top-k 2,048"), and k = 2048.

Every generator is deterministic in its seed: one ``SeedSequence(seed)`` is
spawned into child streams in a fixed tensor order, so every tensor is
reproducible on its own and on any machine.
"""
from __future__ import annotations

import math
import os
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

LATENT_DIM = 576
VALUE_DIM = 512
ROPE_DIM = 64

# Child-stream order for SeedSequence.spawn: never reorder, only append.
_STREAMS = ("q_idx", "head_w", "k_idx", "q_abs", "latent", "boost", "proto", "drift")


@dataclass
class DSAProblem:
    """One batch of DSA inputs in device storage formats.

    Indexer: ``q_idx`` [R, H_I, D_I], ``head_w`` [R, H_I] fp32, ``k_idx``
    [rows, D_I] (+ ``k_scale`` [rows] bf16 bits when the keys are fp8).
    Attention: ``q_abs`` [R, H, 576], ``latent`` [rows, 576] (+ ``latent_scale``
    [rows] float32 when the latent rows are fp8).
    Sequence b owns cache rows ``row_off[b] .. row_off[b]+seq_len[b]-1``;
    query r belongs to sequence ``q_seq[r]`` at position ``q_pos[r]`` and its
    candidates are keys 0..q_pos[r] of that sequence.

    Storage: dtype tags are "f32" (float32), "bf16" (uint16 bit patterns)
    and "fp8_e4m3" (uint8 OCP E4M3FN codes).
    """

    name: str
    q_idx: np.ndarray
    head_w: np.ndarray
    k_idx: np.ndarray
    k_scale: Optional[np.ndarray]
    q_abs: np.ndarray
    latent: np.ndarray
    row_off: np.ndarray
    seq_len: np.ndarray
    q_seq: np.ndarray
    q_pos: np.ndarray
    k: int
    scale: float
    act_dtype: str  # dtype of q_idx, q_abs (and latent unless latent_dtype is set)
    key_dtype: str  # dtype of k_idx
    meta: dict = field(default_factory=dict)
    latent_dtype: Optional[str] = None          # "fp8_e4m3": latent stored as codes ...
    latent_scale: Optional[np.ndarray] = None   # ... with one float32 scale per cache row
    block_table: Optional[np.ndarray] = None    # paged cache: [B, max_pages] page ids ...
    page_size: int = 0                          # ... of page_size rows; row_off unused

    @property
    def kv_dtype(self) -> str:
        """Storage dtype of the latent cache."""
        return self.latent_dtype or self.act_dtype

    @property
    def R(self) -> int:
        return int(self.q_pos.shape[0])

    @property
    def B(self) -> int:
        return int(self.row_off.shape[0])

    @property
    def H_I(self) -> int:
        return int(self.q_idx.shape[1])

    @property
    def D_I(self) -> int:
        return int(self.q_idx.shape[2])

    @property
    def H(self) -> int:
        return int(self.q_abs.shape[1])

    @property
    def cache_rows(self) -> int:
        return int(self.k_idx.shape[0])

    @property
    def max_n(self) -> int:
        return int(self.q_pos.max()) + 1

    @property
    def tokens_per_seq(self) -> int:
        return int(self.meta.get("tokens_per_seq", 1))

    def is_decode(self) -> bool:
        """tokens_per_seq queries per sequence (sequence-major), at its last positions."""
        m = self.tokens_per_seq
        i = np.arange(self.R) % m
        return (self.R == self.B * m and np.array_equal(self.q_seq, np.arange(self.R) // m)
                and np.array_equal(self.q_pos, np.repeat(self.seq_len, m) - m + i))


# --------------------------------------------------------------------------
# storage encoders (input preparation only)
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 (nearest, ties to even); return
    the bits. In 32-bit arithmetic: a finite value's bits plus 0x8000 stay
    below 2**32."""
    u = np.array(x, dtype=np.float32, copy=True).view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    u += r
    u >>= 16
    return u.astype(np.uint16)


def bf16_bits_round_up(x: np.ndarray) -> np.ndarray:
    """Smallest bf16 not below each positive float32 value (bits)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = f32_to_bf16_bits(x)
    back = (b.astype(np.uint32) << 16).view(np.float32)
    return np.where(back < x, b + 1, b).astype(np.uint16)


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Encode float32 values as OCP E4M3FN codes (nearest, ties to even).

    Inputs must lie within +-448. torch's float8_e4m3fn cast is the encoder.
    """
    import torch

    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.size and float(np.abs(x).max()) > 448.0:
        raise ValueError("e4m3 input out of range")
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy().copy()


def _normal_bf16(rng: np.random.Generator, shape, std: float = 1.0,
                 chunk: int = 1 << 22) -> np.ndarray:
    """N(0, std^2) samples stored as bf16 bits (nearest, ties to even).

    Chunk i of ``chunk`` values is drawn from the stream's bit generator
    jumped i times, so the chunks are independent and can be generated on
    several threads with a result that does not depend on the thread count.
    """
    from concurrent.futures import ThreadPoolExecutor

    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    base = rng.bit_generator

    def fill(i):
        lo, hi = i * chunk, min(total, (i + 1) * chunk)
        v = np.random.Generator(base.jumped(i + 1)).standard_normal(hi - lo, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        u = v.view(np.uint32)
        r = u >> 16
        r &= 1
        r += 0x7FFF
        u += r                                   # finite values: no 32-bit overflow
        out[lo:hi] = u.view(np.uint16)[1::2]     # high halves (little-endian)

    n_chunks = (total + chunk - 1) // chunk
    if n_chunks <= 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return out.reshape(shape)


def _normal_e4m3_rows(rng: np.random.Generator, rows: int, dim: int, std: float = 1.0,
                      chunk_rows: int = 1 << 13):
    """N(0, std^2) rows [rows, dim] stored as OCP E4M3FN codes with one
    float32 scale per row, scale = (row max |x|) / 448 (1 for an all-zero
    row), code = nearest e4m3 of x / scale (clipped to +-448).

    Block i of ``chunk_rows`` rows comes from the stream's bit generator
    jumped i + 1 times, as in _normal_bf16.
    """
    from concurrent.futures import ThreadPoolExecutor

    codes = np.empty((rows, dim), dtype=np.uint8)
    scales = np.empty(rows, dtype=np.float32)
    base = rng.bit_generator

    def fill(i):
        lo, hi = i * chunk_rows, min(rows, (i + 1) * chunk_rows)
        v = np.random.Generator(base.jumped(i + 1)).standard_normal((hi - lo, dim), dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        mx = np.abs(v).max(axis=1)
        sc = np.where(mx > 0, mx / np.float32(448.0), np.float32(1.0)).astype(np.float32)
        scales[lo:hi] = sc
        codes[lo:hi] = f32_to_e4m3_codes(np.clip(v / sc[:, None], -448.0, 448.0))

    n_chunks = (rows + chunk_rows - 1) // chunk_rows
    if n_chunks <= 1:
        for i in range(n_chunks):
            fill(i)
    else:
        with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, range(n_chunks)))
    return codes, scales


def _streams(seed: int):
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return {name: np.random.Generator(np.random.PCG64(c)) for name, c in zip(_STREAMS, children)}


def _offsets(seq_lens: Sequence[int]) -> np.ndarray:
    off = np.zeros(len(seq_lens), dtype=np.int64)
    if len(seq_lens) > 1:
        off[1:] = np.cumsum(np.asarray(seq_lens[:-1], dtype=np.int64))
    return off


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

def tiny_config(seed: int = 0, quantized: bool = False, n_keys: int = 512,
                n_queries: int = 16, k: int = 64) -> DSAProblem:
    """The tiny CPU-checkable case: one causal sequence of 512 keys with 16
    queries at the last positions; indexer 4 heads x 64, fp32; k = 64;
    attention 8 heads over fp32 576-d latent rows; scale 1/sqrt(192).

    ``quantized=True`` draws every indexer input from a small integer grid
    (q, k in {-4..3}, w in eighths) so every score is exact in fp32 under any
    summation order.
    """
    st = _streams(seed)
    H_I, D_I, H = 4, 64, 8
    if quantized:
        q_idx = st["q_idx"].integers(-4, 4, size=(n_queries, H_I, D_I)).astype(np.float32)
        k_idx = st["k_idx"].integers(-4, 4, size=(n_keys, D_I)).astype(np.float32)
        head_w = (st["head_w"].integers(1, 9, size=(n_queries, H_I)) / 8.0).astype(np.float32)
    else:
        q_idx = st["q_idx"].standard_normal((n_queries, H_I, D_I), dtype=np.float32)
        k_idx = st["k_idx"].standard_normal((n_keys, D_I), dtype=np.float32)
        head_w = st["head_w"].random((n_queries, H_I), dtype=np.float32)
    q_abs = st["q_abs"].standard_normal((n_queries, H, LATENT_DIM), dtype=np.float32)
    latent = (st["latent"].standard_normal((n_keys, LATENT_DIM), dtype=np.float32)
              * np.float32(0.1))
    return DSAProblem(
        name="tiny-quantized" if quantized else "tiny",
        q_idx=q_idx, head_w=head_w, k_idx=k_idx, k_scale=None,
        q_abs=q_abs, latent=latent,
        row_off=np.zeros(1, np.int64), seq_len=np.array([n_keys], np.int32),
        q_seq=np.zeros(n_queries, np.int32),
        q_pos=np.arange(n_keys - n_queries, n_keys, dtype=np.int32),
        k=k, scale=1.0 / math.sqrt(192.0), act_dtype="f32", key_dtype="f32",
        meta={"seed": seed},
    )


def decode_config(seq_lens: Sequence[int], seed: int = 0, H_I: int = 64, D_I: int = 128,
                  H: int = 64, k: int = 2048, key_dtype: str = "bf16",
                  boost_frac: float = 0.0, boost_sigma: float = 4.0,
                  tie_levels: int = 0, latent_std: float = 0.1, q_abs_std: float = 1.0,
                  latent_dtype: str = "bf16", tokens_per_seq: int = 1,
                  name: str = "decode") -> DSAProblem:
    """Decode batch: ``tokens_per_seq`` new queries per sequence at its last
    positions (query row b * tokens_per_seq + i at seq_len[b] - tokens_per_seq + i).

    * indexer queries N(0,1) bf16, head weights U(0,1) fp32, keys N(0,1);
    * ``key_dtype="fp8_e4m3"`` stores keys as OCP E4M3FN codes with a per-row
      bf16 scale = (row max |k|) / 448, rounded up so no code saturates;
    * ``boost_frac`` > 0 adds, to that seeded fraction of each sequence's
      keys, a vector along the sequence's mean indexer query, sized so the
      mean per-head dot of a boosted key rises by ``boost_sigma`` standard
      deviations of the dot (sqrt(D_I) for unit-variance inputs) -- salient
      tokens with heavy-tailed scores;
    * ``tie_levels`` > 0 makes every indexer key one of ``tie_levels``
      prototype rows with entries in {-4..3}, indexer queries in {-4..3} and
      head weights in {1/8..8/8}: every score of a query takes one of at most
      ``tie_levels`` values, all exact in fp32, so large tie classes straddle
      the k-th rank;
    * absorbed queries N(0, q_abs_std^2) bf16, latent rows N(0, latent_std^2)
      bf16, or with ``latent_dtype="fp8_e4m3"`` e4m3 codes with a float32
      per-row scale (row max |x| / 448).
    """
    st = _streams(seed)
    B = len(seq_lens)
    m = int(tokens_per_seq)
    R = B * m
    seq_lens = [int(s) for s in seq_lens]
    rows = int(sum(seq_lens))
    row_off = _offsets(seq_lens)

    if tie_levels:
        q_f = st["q_idx"].integers(-4, 4, size=(R, H_I, D_I)).astype(np.float32)
        head_w = (st["head_w"].integers(1, 9, size=(R, H_I)) / 8.0).astype(np.float32)
        protos = st["proto"].integers(-4, 4, size=(tie_levels, D_I)).astype(np.float32)
        choice = st["k_idx"].integers(0, tie_levels, size=rows)
        k_f = protos[choice]
        q_idx = f32_to_bf16_bits(q_f)
        k_store = f32_to_bf16_bits(k_f)
        k_scale = None
        if key_dtype != "bf16":
            raise ValueError("tie-class inputs are stored as bf16")
    else:
        q_idx = _normal_bf16(st["q_idx"], (R, H_I, D_I))
        head_w = st["head_w"].random((R, H_I), dtype=np.float32)
        k_scale = None
        if key_dtype == "bf16" and not boost_frac:
            k_store = _normal_bf16(st["k_idx"], (rows, D_I))
        else:
            k_f = st["k_idx"].standard_normal((rows, D_I), dtype=np.float32)
            if boost_frac:
                q_vals = (q_idx.astype(np.uint32) << 16).view(np.float32).reshape(B, m * H_I, D_I)
                rb = st["boost"]
                for b in range(B):
                    mean_q = q_vals[b].mean(axis=0)     # over the heads of the sequence's queries
                    u = mean_q / np.linalg.norm(mean_q)
                    per_head = q_vals[b] @ u            # dot of each head's query with u
                    amp = boost_sigma * math.sqrt(D_I) / float(per_head.mean())
                    nb = seq_lens[b]
                    sel = rb.random(nb) < boost_frac
                    seg = k_f[row_off[b]:row_off[b] + nb]
                    seg[sel] += np.float32(amp) * u.astype(np.float32)
            if key_dtype == "bf16":
                k_store = f32_to_bf16_bits(k_f)
            elif key_dtype == "fp8_e4m3":
                rowmax = np.abs(k_f).max(axis=1)
                rowmax = np.where(rowmax > 0, rowmax, np.float32(1.0))
                k_scale = bf16_bits_round_up(rowmax / np.float32(448.0))
                sc = (k_scale.astype(np.uint32) << 16).view(np.float32)
                k_store = f32_to_e4m3_codes(np.clip(k_f / sc[:, None], -448.0, 448.0))
            else:
                raise ValueError(f"unknown key dtype {key_dtype}")

    q_abs = _normal_bf16(st["q_abs"], (R, H, LATENT_DIM), std=q_abs_std)
    latent_scale = None
    if latent_dtype == "bf16":
        latent = _normal_bf16(st["latent"], (rows, LATENT_DIM), std=latent_std)
    elif latent_dtype == "fp8_e4m3":
        latent, latent_scale = _normal_e4m3_rows(st["latent"], rows, LATENT_DIM, std=latent_std)
    else:
        raise ValueError(f"unknown latent dtype {latent_dtype}")
    seq_len = np.asarray(seq_lens, np.int32)
    return DSAProblem(
        name=name, q_idx=q_idx, head_w=head_w, k_idx=k_store, k_scale=k_scale,
        q_abs=q_abs, latent=latent, row_off=row_off, seq_len=seq_len,
        q_seq=np.arange(R, dtype=np.int32) // m,
        q_pos=(np.repeat(seq_len, m) - m + np.arange(R) % m).astype(np.int32),
        k=k, scale=1.0 / math.sqrt(192.0), act_dtype="bf16", key_dtype=key_dtype,
        meta={"seed": seed, "boost_frac": boost_frac, "tie_levels": tie_levels, "tokens_per_seq": m},
        latent_dtype=None if latent_dtype == "bf16" else latent_dtype, latent_scale=latent_scale,
    )


def prefill_config(T: int = 8192, seed: int = 0, H_I: int = 64, D_I: int = 128,
                   H: int = 64, k: int = 2048, drift: float | None = None,
                   query_rows: Optional[np.ndarray] = None,
                   name: str = "prefill") -> DSAProblem:
    """Causal prefill of one T-token sequence: query t scores keys 0..t.

    Indexer keys N(0,1) plus a linear positional drift ``drift*(s/(T-1))*u``
    along a seeded unit vector u, and every indexer query gets ``+u``, so
    later keys score higher on average (a recency bias). The default drift
    is sqrt(D_I): the mean per-head dot rises by one dot standard deviation
    from the first key to the last. ``query_rows`` restricts the queries to
    those positions (all T when None).
    """
    st = _streams(seed)
    if drift is None:
        drift = math.sqrt(D_I)
    u = st["drift"].standard_normal(D_I).astype(np.float32)
    u /= np.linalg.norm(u)
    pos = np.arange(T, dtype=np.int32) if query_rows is None else np.asarray(query_rows, np.int32)
    R = int(pos.shape[0])
    q_f = st["q_idx"].standard_normal((T, H_I, D_I), dtype=np.float32)[pos] + u
    k_f = st["k_idx"].standard_normal((T, D_I), dtype=np.float32)
    k_f += (np.float32(drift) * (np.arange(T, dtype=np.float32) / max(T - 1, 1)))[:, None] * u
    head_w = st["head_w"].random((T, H_I), dtype=np.float32)[pos]
    q_abs = _normal_bf16(st["q_abs"], (T, H, LATENT_DIM))[pos]
    latent = _normal_bf16(st["latent"], (T, LATENT_DIM), std=0.1)
    return DSAProblem(
        name=name, q_idx=f32_to_bf16_bits(q_f), head_w=head_w,
        k_idx=f32_to_bf16_bits(k_f), k_scale=None, q_abs=q_abs, latent=latent,
        row_off=np.zeros(1, np.int64), seq_len=np.array([T], np.int32),
        q_seq=np.zeros(R, np.int32), q_pos=pos.copy(), k=k,
        scale=1.0 / math.sqrt(192.0), act_dtype="bf16", key_dtype="bf16",
        meta={"seed": seed, "drift": drift},
    )


# Named workloads. The full sizes are the measured shapes; the "small"
# variants keep the structure at sizes the oracle finishes in seconds.
def workload(name: str, seed: int = 0) -> DSAProblem:
    if name == "tiny":
        return tiny_config(seed)
    if name == "tiny-quantized":
        return tiny_config(seed, quantized=True)
    if name == "decode-32k":
        return decode_config([32768] * 4, seed=seed, name=name)
    if name == "decode-128k-fp8":
        return decode_config([131072] * 7 + [200000], seed=seed, key_dtype="fp8_e4m3",
                             boost_frac=0.02, name=name)
    if name == "decode-32k-fp8kv":
        return decode_config([32768] * 4, seed=seed, latent_dtype="fp8_e4m3", name=name)
    if name == "decode-128k-fp8kv":
        return decode_config([131072] * 7 + [200000], seed=seed, key_dtype="fp8_e4m3",
                             boost_frac=0.02, latent_dtype="fp8_e4m3", name=name)
    if name == "decode-32k-mtp4":
        return decode_config([32768] * 4, seed=seed, tokens_per_seq=4, name=name)
    if name == "decode-128k-fp8-mtp4":
        return decode_config([131072] * 7 + [200000], seed=seed, key_dtype="fp8_e4m3", boost_frac=0.02,
                             tokens_per_seq=4, name=name)
    if name == "decode-32k-paged":
        return paged_view(decode_config([32768] * 4, seed=seed, name="decode-32k"), page_size=64, seed=seed)
    if name == "ties-64k":
        return decode_config([65536] * 16, seed=seed, tie_levels=8, name=name)
    if name == "prefill-8k":
        return prefill_config(8192, seed=seed, name=name)
    raise KeyError(name)


def paged_view(prob: DSAProblem, page_size: int = 64, seed: int = 0, spare_pages: int = 3) -> DSAProblem:
    """The same problem with its caches in a paged pool: every sequence's rows
    cut into pages of ``page_size`` rows, the pages placed at seeded random
    slots of a pool with ``spare_pages`` extra pages (filled with other rows),
    and a block table [B, max_pages] naming each sequence's pages in order
    (unused table entries point at slot 0). Storage only: the rows are moved,
    not changed."""
    import dataclasses

    rng = np.random.default_rng(seed)
    B = prob.B
    pages = [(int(n) + page_size - 1) // page_size for n in prob.seq_len]
    total = sum(pages) + spare_pages
    slots = rng.permutation(total)
    max_pages = max(pages)
    table = np.zeros((B, max_pages), np.int32)
    src_rows = rng.integers(0, prob.cache_rows, total * page_size)   # spare and tail rows: other rows
    nxt = 0
    for b in range(B):
        for j in range(pages[b]):
            slot = int(slots[nxt])
            nxt += 1
            table[b, j] = slot
            lo = int(prob.row_off[b]) + j * page_size
            cnt = min(page_size, int(prob.seq_len[b]) - j * page_size)
            src_rows[slot * page_size:slot * page_size + cnt] = np.arange(lo, lo + cnt)

    def move(arr):
        return None if arr is None else np.ascontiguousarray(arr[src_rows])

    return dataclasses.replace(
        prob, name=prob.name + f"-paged{page_size}", k_idx=move(prob.k_idx), k_scale=move(prob.k_scale),
        latent=move(prob.latent), latent_scale=move(prob.latent_scale),
        row_off=np.zeros(B, np.int64), block_table=table, page_size=page_size,
        meta={**prob.meta, "paged_from": prob.name})


def to_torch(prob: DSAProblem, device="cuda"):
    """Copy a problem's arrays to torch tensors on ``device`` (bit-exact:
    bf16 bit patterns become torch.bfloat16, fp8 codes stay uint8)."""
    import types
    import torch

    def t(a, dt):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(device)
        if dt == "fp8_e4m3":
            return torch.from_numpy(a.view(np.uint8)).to(device)
        if dt == "f32":
            return torch.from_numpy(a.astype(np.float32, copy=False)).to(device)
        return torch.from_numpy(a).to(device)

    return types.SimpleNamespace(
        q_idx=t(prob.q_idx, prob.act_dtype), head_w=t(prob.head_w, "f32"),
        k_idx=t(prob.k_idx, prob.key_dtype),
        k_scale=None if prob.k_scale is None else t(prob.k_scale.view(np.int16), None),
        q_abs=t(prob.q_abs, prob.act_dtype), latent=t(prob.latent, prob.kv_dtype),
        latent_scale=None if prob.latent_scale is None else t(prob.latent_scale, "f32"),
        row_off=t(prob.row_off.astype(np.int64), None), seq_len=t(prob.seq_len.astype(np.int32), None),
        q_seq=t(prob.q_seq.astype(np.int32), None), q_pos=t(prob.q_pos.astype(np.int32), None),
        block_table=None if prob.block_table is None else t(prob.block_table.astype(np.int32), None),
    )
