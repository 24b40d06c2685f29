"""Python binding of libdsa.so (include/dsa.h): argument marshalling only.

Each function has the name of the C entry point it calls. Tensors must be
contiguous CUDA (HIP) tensors; the functions pass their ``data_ptr()`` and
torch's current stream, allocate outputs and workspace with torch when the
caller does not pass them, and raise ``DSAError`` on a non-OK status. Every
step of the computation runs in the library's HIP kernels; importing this
module fails if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")

DSA_OK, DSA_ERR_NULL, DSA_ERR_SHAPE, DSA_ERR_DTYPE, DSA_ERR_ALIGN, DSA_ERR_WORKSPACE, \
    DSA_ERR_UNSUPPORTED, DSA_ERR_HIP = range(8)
DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_ENTRY_INDEX_SCORES, DSA_ENTRY_TOPK, DSA_ENTRY_SPARSE_MLA, DSA_ENTRY_DECODE = 0, 1, 2, 3
DSA_LATENT_DIM, DSA_VALUE_DIM, DSA_MAX_TOPK, DSA_MAX_TOKENS_PER_SEQ = 576, 512, 2048, 8

# C signatures, in the order of include/dsa.h.
_P, _I32, _I64, _F32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "dsa_index_scores": (_I32, [_P, _I32, _P, _P, _I32, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _I32,
                                _P, _I64, _P]),
    "dsa_index_scores_decode": (_I32, [_P, _I32, _P, _P, _I32, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                       _P, _I64, _P]),
    "dsa_topk": (_I32, [_P, _I64, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "dsa_sparse_mla_attn": (_I32, [_P, _I32, _P, _I32, _P, _I64, _P, _I32, _P, _P, _I32, _I32, _I32, _F32,
                                   _P, _P, _P, _SZ, _P]),
    "dsa_decode_fused": (_I32, [_P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _I64, _P, _P, _I32, _I32, _I32,
                                _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _P, _SZ, _P]),
    "dsa_decode_fused_noalloc": (_I32, [_P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _I64, _P, _P, _I32, _I32,
                                        _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _P]),
    "dsa_decode_noalloc_limit": (_SZ, []),
    "dsa_sparse_mla_attn_paged": (_I32, [_P, _I32, _P, _I32, _P, _I64, _P, _I32, _I32, _I32, _P, _P, _I32, _I32,
                                         _I32, _F32, _P, _P, _P, _SZ, _P]),
    "dsa_decode_fused_paged": (_I32, [_P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _P, _I64, _P, _I32, _I32, _P,
                                      _I32, _I32, _I32, _I32, _I32, _I32, _I32, _F32, _P, _P, _P, _P, _SZ, _P]),
    "dsa_topk_pairs": (_I32, [_P, _I64, _P, _I32, _I32, _I32, _P, _P, _P]),
    "dsa_topk_merge": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P]),
    "dsa_shard_indices": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _P]),
    "dsa_attn_merge": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P, _P]),
    "dsa_workspace_size": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "dsa_check_indices": (_I32, [_P, _P, _I32, _I32, _P, _P]),
    "dsa_read_probe_blocks": (_I32, []),
    "dsa_read_probe": (_I32, [_P, ctypes.c_uint64, _P, _I32, _P]),
    "dsa_status_string": (ctypes.c_char_p, [_I32]),
    "dsa_last_error": (ctypes.c_char_p, []),
}


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_attention_05_amd.build` "
                          "(the DSA path has no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


class DSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = dsa_status_string(status)
        if status == DSA_ERR_HIP:
            msg += ": " + (lib.dsa_last_error() or b"").decode()
        super().__init__(f"{where}: {msg} (status {status})")
        self.status = status


def _check(status: int, where: str) -> None:
    if status != DSA_OK:
        raise DSAError(status, where)


def dsa_status_string(status: int) -> str:
    return lib.dsa_status_string(int(status)).decode()


def dsa_workspace_size(entry: int, rows: int, max_len: int, k: int, H: int) -> int:
    return int(lib.dsa_workspace_size(entry, rows, max_len, k, H))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _workspace(nbytes: int, ws: Optional[torch.Tensor], device) -> Optional[torch.Tensor]:
    if nbytes == 0:
        return ws
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError("workspace too small")
    return ws


def dsa_index_scores(q_idx: torch.Tensor, head_w: torch.Tensor, k_idx: torch.Tensor,
                     row_off: torch.Tensor, q_pos: torch.Tensor, max_n: int, *,
                     k_scale: Optional[torch.Tensor] = None, q_seq: Optional[torch.Tensor] = None,
                     scores: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Indexer scores [R, ld] (fp32); entries past q_pos[r] are left untouched."""
    R, H_I, D_I = q_idx.shape
    if scores is None:
        ld = (max_n + 3) // 4 * 4
        scores = torch.empty((R, ld), dtype=torch.float32, device=q_idx.device)
    st = lib.dsa_index_scores(
        _ptr(q_idx), _dtype_code(q_idx), _ptr(head_w), _ptr(k_idx), _dtype_code(k_idx), _ptr(k_scale),
        k_idx.shape[0], _ptr(row_off), row_off.numel(), _ptr(q_seq), _ptr(q_pos), R, H_I, D_I, max_n,
        _ptr(scores), scores.shape[1], _stream(stream))
    _check(st, "dsa_index_scores")
    return scores


def dsa_index_scores_decode(q_idx: torch.Tensor, head_w: torch.Tensor, k_idx: torch.Tensor,
                            row_off: torch.Tensor, seq_len: torch.Tensor, max_len: int, *, q_per_seq: int = 1,
                            k_scale: Optional[torch.Tensor] = None, scores: Optional[torch.Tensor] = None,
                            stream=None) -> torch.Tensor:
    """Decode-form indexer scores [R, ld] (fp32), R = B * q_per_seq rows,
    row b * q_per_seq + i at position seq_len[b] - q_per_seq + i."""
    R, H_I, D_I = q_idx.shape
    B = seq_len.numel()
    if scores is None:
        scores = torch.empty((R, (max_len + 3) // 4 * 4), dtype=torch.float32, device=q_idx.device)
    st = lib.dsa_index_scores_decode(
        _ptr(q_idx), _dtype_code(q_idx), _ptr(head_w), _ptr(k_idx), _dtype_code(k_idx), _ptr(k_scale),
        k_idx.shape[0], _ptr(row_off), _ptr(seq_len), B, q_per_seq, H_I, D_I, max_len, _ptr(scores),
        scores.shape[1], _stream(stream))
    _check(st, "dsa_index_scores_decode")
    return scores


def dsa_topk(scores: torch.Tensor, q_pos: torch.Tensor, max_n: int, k: int, *,
             idx_out: Optional[torch.Tensor] = None, workspace=None, stream=None) -> torch.Tensor:
    """Deterministic top-k indices [R, k] (int32, rank order, -1 padded).

    workspace: None allocates what the library asks for (few long rows are
    then split over several workgroups); False passes none (one workgroup
    per row); a uint8 tensor is used as given."""
    R = scores.shape[0]
    if idx_out is None:
        idx_out = torch.empty((R, k), dtype=torch.int32, device=scores.device)
    if workspace is False:
        workspace = None
    else:
        workspace = _workspace(dsa_workspace_size(DSA_ENTRY_TOPK, R, max_n, k, 1), workspace, scores.device)
    st = lib.dsa_topk(_ptr(scores), scores.shape[1], _ptr(q_pos), R, max_n, k, _ptr(idx_out), _ptr(workspace),
                      0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream))
    _check(st, "dsa_topk")
    return idx_out


def dsa_sparse_mla_attn(q_abs: torch.Tensor, latent: torch.Tensor, row_off: Optional[torch.Tensor],
                        idx: torch.Tensor, scale: float, *, latent_scale: Optional[torch.Tensor] = None,
                        q_seq: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                        page_size: int = 0,
                        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                        want_lse: bool = True, workspace: Optional[torch.Tensor] = None,
                        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Sparse absorbed MLA: (out [R, H, 512] fp32, lse [R, H] fp32). A uint8
    (or float8_e4m3fn) latent holds e4m3 codes scaled by latent_scale [rows].
    With block_table [B, max_pages] (and page_size) the cache is paged and
    row_off is ignored."""
    R, H, _ = q_abs.shape
    k = idx.shape[1]
    dev = q_abs.device
    if out is None:
        out = torch.empty((R, H, DSA_VALUE_DIM), dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    nbytes = dsa_workspace_size(DSA_ENTRY_SPARSE_MLA, R, 0, k, H)
    workspace = _workspace(nbytes, workspace, dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if block_table is not None:
        st = lib.dsa_sparse_mla_attn_paged(
            _ptr(q_abs), _dtype_code(q_abs), _ptr(latent), _dtype_code(latent), _ptr(latent_scale),
            latent.shape[0], _ptr(block_table), block_table.shape[1], int(page_size), block_table.shape[0],
            _ptr(q_seq), _ptr(idx), k, R, H, float(scale), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
            _stream(stream))
        _check(st, "dsa_sparse_mla_attn_paged")
        return out, lse
    st = lib.dsa_sparse_mla_attn(
        _ptr(q_abs), _dtype_code(q_abs), _ptr(latent), _dtype_code(latent), _ptr(latent_scale), latent.shape[0],
        _ptr(row_off), row_off.numel(),
        _ptr(q_seq), _ptr(idx), k, R, H, float(scale), _ptr(out), _ptr(lse), _ptr(workspace), wsb,
        _stream(stream))
    _check(st, "dsa_sparse_mla_attn")
    return out, lse


def dsa_check_indices(idx: torch.Tensor, q_pos: torch.Tensor, *, n_bad: Optional[torch.Tensor] = None,
                      stream=None) -> torch.Tensor:
    """Count of structurally bad entries of idx [R, k] (out of [0, q_pos+1),
    repeated, or bad -1 padding), ADDED to n_bad (a zeroed int32 device
    scalar is allocated when none is passed); returns n_bad."""
    R, k = idx.shape
    if n_bad is None:
        n_bad = torch.zeros(1, dtype=torch.int32, device=idx.device)
    st = lib.dsa_check_indices(_ptr(idx), _ptr(q_pos), R, k, _ptr(n_bad), _stream(stream))
    _check(st, "dsa_check_indices")
    return n_bad


def dsa_read_probe(buf: torch.Tensor, *, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """A plain streaming read of buf's bytes (a measurement aid, no part of
    the method): out[g] = the fp32 sum of the floats workgroup g read, one
    workgroup per CU; returns out."""
    G = lib.dsa_read_probe_blocks()
    if out is None:
        out = torch.empty(G, dtype=torch.float32, device=buf.device)
    st = lib.dsa_read_probe(_ptr(buf), buf.numel() * buf.element_size(), _ptr(out), out.numel(), _stream(stream))
    _check(st, "dsa_read_probe")
    return out


def dsa_topk_pairs(scores: torch.Tensor, idx: torch.Tensor, key_offset: int, *, pair_score=None, pair_idx=None,
                   stream=None):
    """A shard's candidate list: (scores at idx, idx + key_offset), -inf / -1 for -1."""
    R, k = idx.shape
    if pair_score is None:
        pair_score = torch.empty((R, k), dtype=torch.float32, device=idx.device)
    if pair_idx is None:
        pair_idx = torch.empty((R, k), dtype=torch.int32, device=idx.device)
    st = lib.dsa_topk_pairs(_ptr(scores), scores.shape[1], _ptr(idx), R, k, int(key_offset), _ptr(pair_score),
                            _ptr(pair_idx), _stream(stream))
    _check(st, "dsa_topk_pairs")
    return pair_score, pair_idx


def dsa_topk_merge(pair_score: torch.Tensor, pair_idx: torch.Tensor, *, idx_out=None, stream=None) -> torch.Tensor:
    """Global top-k [R, k] from P shards' candidate lists [P, R, k]."""
    P, R, k = pair_idx.shape
    if idx_out is None:
        idx_out = torch.empty((R, k), dtype=torch.int32, device=pair_idx.device)
    st = lib.dsa_topk_merge(_ptr(pair_score), _ptr(pair_idx), P, R, k, _ptr(idx_out), _stream(stream))
    _check(st, "dsa_topk_merge")
    return idx_out


def dsa_shard_indices(idx: torch.Tensor, lo: int, hi: int, *, idx_local=None, stream=None) -> torch.Tensor:
    """Entries of idx in [lo, hi) shifted by -lo, others -1."""
    R, k = idx.shape
    if idx_local is None:
        idx_local = torch.empty_like(idx)
    st = lib.dsa_shard_indices(_ptr(idx), R, k, int(lo), int(hi), _ptr(idx_local), _stream(stream))
    _check(st, "dsa_shard_indices")
    return idx_local


def dsa_attn_merge(o_parts: torch.Tensor, lse_parts: torch.Tensor, *, out=None, lse=None, stream=None):
    """Log-sum-exp merge of P partial attentions [P, R, H, 512] / [P, R, H]."""
    P, R, H, _ = o_parts.shape
    if out is None:
        out = torch.empty((R, H, DSA_VALUE_DIM), dtype=torch.float32, device=o_parts.device)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=o_parts.device)
    st = lib.dsa_attn_merge(_ptr(o_parts), _ptr(lse_parts), P, R, H, _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "dsa_attn_merge")
    return out, lse


class DecodeCall:
    """A pre-marshalled dsa_decode_fused call: validates and allocates once,
    then each ``__call__`` enqueues one decode step with no Python-side
    allocation. Used where per-step host overhead matters."""

    def __init__(self, q_idx, head_w, k_idx, q_abs, latent, row_off, seq_len, max_len: int, k: int,
                 scale: float, *, k_scale=None, latent_scale=None, q_per_seq: int = 1, block_table=None,
                 page_size: int = 0, out=None, lse=None, idx_out=None, want_lse=True, record_idx=True,
                 workspace=None):
        R, H_I, D_I = q_idx.shape
        B = seq_len.numel()
        if R != B * q_per_seq:
            raise ValueError(f"q_idx has {R} rows; {B} sequences x {q_per_seq} tokens expected")
        H = q_abs.shape[1]
        dev = q_idx.device
        self.out = out if out is not None else torch.empty((R, H, DSA_VALUE_DIM), dtype=torch.float32, device=dev)
        self.lse = lse if lse is not None or not want_lse else torch.empty((R, H), dtype=torch.float32, device=dev)
        self.idx = idx_out if idx_out is not None or not record_idx else \
            torch.empty((R, k), dtype=torch.int32, device=dev)
        nbytes = dsa_workspace_size(DSA_ENTRY_DECODE, R, max_len, k, H)
        self.workspace = _workspace(nbytes, workspace, dev)
        if _dtype_code(q_idx) != _dtype_code(q_abs):
            raise TypeError("q_idx and q_abs must share one dtype")
        self._keep = (q_idx, head_w, k_idx, k_scale, q_abs, latent, latent_scale, row_off, seq_len, block_table)
        cache = ((_ptr(block_table), block_table.shape[1], int(page_size)) if block_table is not None
                 else (_ptr(row_off),))
        self._fn = lib.dsa_decode_fused_paged if block_table is not None else lib.dsa_decode_fused
        self._args = (
            _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _dtype_code(k_idx), _ptr(k_scale), _ptr(q_abs), _ptr(latent),
            _dtype_code(q_abs), _dtype_code(latent), _ptr(latent_scale), k_idx.shape[0], *cache,
            _ptr(seq_len), B, q_per_seq, max_len, H_I, D_I, H, k,
            float(scale), _ptr(self.out), _ptr(self.lse), _ptr(self.idx), _ptr(self.workspace),
            self.workspace.numel() * self.workspace.element_size())

    def __call__(self, stream=None):
        st = self._fn(*self._args, _stream(stream))
        _check(st, "dsa_decode_fused")
        return self.out, self.lse, self.idx


def dsa_decode_noalloc_limit() -> int:
    return int(lib.dsa_decode_noalloc_limit())


def dsa_decode_fused_noalloc(q_idx, head_w, k_idx, q_abs, latent, row_off, seq_len, max_len: int, k: int,
                             scale: float, *, k_scale=None, latent_scale=None, q_per_seq: int = 1,
                             out=None, lse=None, idx_out=None, stream=None):
    """dsa_decode_fused with the library's per-device scratch as workspace
    (no device allocation by the library). out/lse/idx_out are allocated here
    when not passed; pass them to keep the call allocation-free."""
    R, H_I, D_I = q_idx.shape
    B = seq_len.numel()
    H = q_abs.shape[1]
    dev = q_idx.device
    if out is None:
        out = torch.empty((R, H, DSA_VALUE_DIM), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((R, H), dtype=torch.float32, device=dev)
    if idx_out is None:
        idx_out = torch.empty((R, k), dtype=torch.int32, device=dev)
    st = lib.dsa_decode_fused_noalloc(
        _ptr(q_idx), _ptr(head_w), _ptr(k_idx), _dtype_code(k_idx), _ptr(k_scale), _ptr(q_abs), _ptr(latent),
        _dtype_code(q_abs), _dtype_code(latent), _ptr(latent_scale), k_idx.shape[0], _ptr(row_off),
        _ptr(seq_len), B, q_per_seq, max_len, H_I, D_I, H, k, float(scale), _ptr(out), _ptr(lse), _ptr(idx_out),
        _stream(stream))
    if st == DSA_ERR_WORKSPACE:
        raise DSAError(st, "dsa_decode_fused_noalloc: " + (lib.dsa_last_error() or b"").decode())
    _check(st, "dsa_decode_fused_noalloc")
    return out, lse, idx_out


def dsa_decode_fused(q_idx, head_w, k_idx, q_abs, latent, row_off, seq_len, max_len: int, k: int,
                     scale: float, *, k_scale=None, latent_scale=None, q_per_seq: int = 1, block_table=None,
                     page_size: int = 0, out=None, lse=None, idx_out=None, want_lse=True, record_idx=True,
                     workspace=None, stream=None):
    """One decode step for q_per_seq new tokens per sequence (R = B * q_per_seq
    rows, sequence-major); returns (out [R,H,512], lse [R,H] or None, idx [R,k] or None)."""
    call = DecodeCall(q_idx, head_w, k_idx, q_abs, latent, row_off, seq_len, max_len, k, scale,
                      k_scale=k_scale, latent_scale=latent_scale, q_per_seq=q_per_seq, block_table=block_table,
                      page_size=page_size, out=out, lse=lse, idx_out=idx_out, want_lse=want_lse,
                      record_idx=record_idx, workspace=workspace)
    return call(stream)
