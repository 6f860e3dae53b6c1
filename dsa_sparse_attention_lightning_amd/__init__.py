"""MI355X (gfx950) DSA draft-and-verify hot path: thin binding of libdsa.so.

Functions take torch tensors (device memory only) and forward them, with the
current HIP stream, to the C ABI of include/dsa.h.  Every step of the path
runs in the library's HIP kernels; this module only checks and marshals
arguments and allocates outputs and workspaces with torch when the caller
does not pass them.  bf16 tensors may be torch.bfloat16 or int16/uint16 bit
patterns.
"""

from __future__ import annotations

import math

import torch

from . import _lib

__all__ = [
    "index_scores", "topk", "sparse_attn", "sparse_attn_noalloc", "spec_verify", "NOALLOC_SCRATCH_BYTES",
    "topk_workspace_size", "sparse_attn_workspace_size", "spec_verify_workspace_size",
    "spec_verify_greedy", "spec_verify_greedy_workspace_size",
    "abi_version", "DSAError",
]

DSAError = _lib.DSAError
NOALLOC_SCRATCH_BYTES = _lib.NOALLOC_SCRATCH_BYTES

_BF16_LIKE = (torch.bfloat16, torch.int16, torch.uint16)


def _ptr(t):
    return None if t is None else ctypes_ptr(t)


def ctypes_ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(t, name, dtypes):
    _need(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _need(t.is_cuda, f"{name} must be a device tensor")
    _need(t.dtype in dtypes, f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    _need(t.is_contiguous(), f"{name} must be contiguous")


def abi_version() -> int:
    return _lib.load().dsa_abi_version()


def topk_workspace_size(B, R, ld, k) -> int:
    return int(_lib.load().dsa_topk_workspace_size(B, R, ld, k))


def sparse_attn_workspace_size(B, S_q, H_q, H_kv, D_qk, D_v, k) -> int:
    return int(_lib.load().dsa_sparse_attn_workspace_size(B, S_q, H_q, H_kv, D_qk, D_v, k))


def spec_verify_workspace_size(B, G, V) -> int:
    return int(_lib.load().spec_verify_workspace_size(B, G, V))


def spec_verify_greedy_workspace_size(B, G, V) -> int:
    return int(_lib.load().spec_verify_greedy_workspace_size(B, G, V))


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return ws
    if ws is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    _need(isinstance(ws, torch.Tensor) and ws.is_cuda and ws.is_contiguous(),
          "workspace must be a contiguous device tensor")
    _need(ws.numel() * ws.element_size() >= nbytes, f"workspace needs {nbytes} bytes")
    return ws


def _outputs(accepted_len, emitted, B, G, device):
    if accepted_len is None:
        accepted_len = torch.empty(B, dtype=torch.int32, device=device)
    if emitted is None:
        emitted = torch.empty((B, G + 1), dtype=torch.int32, device=device)
    _dev(accepted_len, "accepted_len", (torch.int32,))
    _dev(emitted, "emitted", (torch.int32,))
    _need(accepted_len.shape == (B,), "accepted_len must be [B]")
    _need(emitted.shape == (B, G + 1), "emitted must be [B, G+1]")
    return accepted_len, emitted


def index_scores(q, w, k_index, block_table, row_len, *, page, ld=None, out=None, stream=None):
    """Lightning-indexer scores: s[b,r,t] = sum_h w[b,r,h] * ReLU(q[b,r,h,:] . k[t,:]).

    q [B, R, H_I, D_I] bf16; w [B, R, H_I] fp32; k_index [pages, page, D_I] bf16;
    block_table [B, max_pages] int32; row_len [B, R] int32.
    Returns fp32 [B, R, ld] (entries at t >= row_len untouched).
    """
    lib = _lib.load()
    _dev(q, "q", _BF16_LIKE)
    _dev(w, "w", (torch.float32,))
    _dev(k_index, "k_index", _BF16_LIKE)
    _dev(block_table, "block_table", (torch.int32,))
    _dev(row_len, "row_len", (torch.int32,))
    B, R, H, D = q.shape
    _need(w.shape == (B, R, H), "w must be [B, R, H_I]")
    _need(k_index.dim() == 3 and k_index.shape[1] == page and k_index.shape[2] == D,
          "k_index must be [pages, page, D_I]")
    _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_pages]")
    _need(row_len.shape == (B, R), "row_len must be [B, R]")
    if ld is None:
        ld = out.shape[-1] if out is not None else page * block_table.shape[1]
    if out is None:
        out = torch.empty((B, R, ld), dtype=torch.float32, device=q.device)
    _dev(out, "out", (torch.float32,))
    _need(out.shape == (B, R, ld), "out must be [B, R, ld]")
    st = lib.dsa_index_scores(_ptr(q), _ptr(w), _ptr(k_index), _ptr(block_table), _ptr(row_len),
                              _ptr(out), B, R, H, D, page, block_table.shape[1], ld, _stream(stream))
    _lib.check("dsa_index_scores", st)
    return out


def topk(scores, row_len, k, *, out=None, workspace=None, stream=None):
    """Top-k positions of each score row (score desc, position asc), ascending, -1 padded.

    scores [B, R, ld] fp32; row_len [B, R] int32.  Returns int32 [B, R, k].
    """
    lib = _lib.load()
    _dev(scores, "scores", (torch.float32,))
    _dev(row_len, "row_len", (torch.int32,))
    B, R, ld = scores.shape
    _need(row_len.shape == (B, R), "row_len must be [B, R]")
    if out is None:
        out = torch.empty((B, R, k), dtype=torch.int32, device=scores.device)
    _dev(out, "out", (torch.int32,))
    _need(out.shape == (B, R, k), "out must be [B, R, k]")
    nbytes = int(lib.dsa_topk_workspace_size(B, R, ld, k))
    ws = _workspace(nbytes, scores.device, workspace)
    st = lib.dsa_topk(_ptr(scores), _ptr(row_len), B, R, ld, k, _ptr(out), _ptr(ws), nbytes,
                      _stream(stream))
    _lib.check("dsa_topk", st)
    return out


def _attn_args(q, k_cache, v_cache, block_table, idx, page, D_v, sm_scale, out, lse):
    """Checks and marshals the arguments shared by sparse_attn and
    sparse_attn_noalloc; returns (C arguments before out, out, lse, shape)."""
    _dev(q, "q", _BF16_LIKE)
    _dev(k_cache, "k_cache", _BF16_LIKE)
    _dev(v_cache, "v_cache", _BF16_LIKE)
    _dev(block_table, "block_table", (torch.int32,))
    _dev(idx, "idx", (torch.int32,))
    B, S_q, H_q, D_qk = q.shape
    latent = k_cache.dim() == 3
    if latent:
        _need(v_cache.data_ptr() == k_cache.data_ptr(), "a latent cache is passed as both k_cache and v_cache")
        H_kv = 1
        _need(k_cache.shape[1] == page and k_cache.shape[2] == D_qk, "latent cache must be [pages, page, D_qk]")
        D_v = D_v if D_v is not None else D_qk
        strides = (page * D_qk, D_qk, 0)
    else:
        _need(k_cache.dim() == 4 and k_cache.shape[1] == page and k_cache.shape[3] == D_qk,
              "k_cache must be [pages, page, H_kv, D_qk]")
        H_kv = k_cache.shape[2]
        D_v = v_cache.shape[3]
        _need(v_cache.shape[:3] == k_cache.shape[:3], "v_cache must match k_cache in [pages, page, H_kv]")
        _need(D_v == D_qk, "separate K/V caches need D_v == D_qk (shared strides)")
        strides = (page * H_kv * D_qk, H_kv * D_qk, D_qk)
    _need(block_table.dim() == 2 and block_table.shape[0] == B, "block_table must be [B, max_pages]")
    if idx.dim() == 2:
        idx_rows, k = 1, idx.shape[1]
        _need(idx.shape[0] == B, "idx must be [B, k]")
    else:
        _need(idx.dim() == 3 and idx.shape[:2] == (B, S_q), "idx must be [B, k] or [B, S_q, k]")
        idx_rows, k = S_q, idx.shape[2]
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D_qk)
    if out is None:
        out = torch.empty((B, S_q, H_q, D_v), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, S_q, H_q), dtype=torch.float32, device=q.device)
    _dev(out, "out", (torch.float32,))
    _dev(lse, "lse", (torch.float32,))
    _need(out.shape == (B, S_q, H_q, D_v), "out must be [B, S_q, H_q, D_v]")
    _need(lse.shape == (B, S_q, H_q), "lse must be [B, S_q, H_q]")
    cargs = (_ptr(q), _ptr(k_cache), _ptr(v_cache), strides[0], strides[1], strides[2], _ptr(block_table),
             _ptr(idx), idx_rows, B, S_q, H_q, H_kv, D_qk, D_v, page, block_table.shape[1], k, float(sm_scale),
             _ptr(out), _ptr(lse))
    return cargs, out, lse, (B, S_q, H_q, H_kv, D_qk, D_v, k)


def sparse_attn(q, k_cache, v_cache, block_table, idx, *, page, D_v=None, sm_scale=None,
                out=None, lse=None, workspace=None, stream=None):
    """Attention over the selected positions idx (shared by all heads).

    q [B, S_q, H_q, D_qk] bf16.  k_cache [pages, page, H_kv, D_qk] bf16 and
    v_cache [pages, page, H_kv, D_v], or a latent cache [pages, page, D_qk]
    passed as both k_cache and v_cache (V = first D_v dims).
    idx [B, k] or [B, S_q, k] int32 (-1 ignored).  Returns (out fp32
    [B, S_q, H_q, D_v], lse fp32 [B, S_q, H_q]).
    """
    lib = _lib.load()
    cargs, out, lse, shape = _attn_args(q, k_cache, v_cache, block_table, idx, page, D_v, sm_scale, out, lse)
    nbytes = int(lib.dsa_sparse_attn_workspace_size(*shape))
    ws = _workspace(nbytes, q.device, workspace)
    st = lib.dsa_sparse_attn(*cargs, _ptr(ws), nbytes, _stream(stream))
    _lib.check("dsa_sparse_attn", st)
    return out, lse


def sparse_attn_noalloc(q, k_cache, v_cache, block_table, idx, *, page, D_v=None, sm_scale=None,
                        out, lse, stream=None):
    """sparse_attn for callers that cannot allocate: out and lse are the
    caller's, and the split-k partials go to the library's fixed per-GPU
    scratch of NOALLOC_SCRATCH_BYTES (shapes needing more are refused).
    Calls that may overlap on one GPU race on that scratch."""
    lib = _lib.load()
    _need(out is not None and lse is not None, "sparse_attn_noalloc takes caller-allocated out and lse")
    cargs, out, lse, _ = _attn_args(q, k_cache, v_cache, block_table, idx, page, D_v, sm_scale, out, lse)
    st = lib.dsa_sparse_attn_noalloc(*cargs, _stream(stream))
    _lib.check("dsa_sparse_attn_noalloc", st)
    return out, lse


def spec_verify(target_logits, draft_logits, draft_tokens, *, uniforms=None, seed=0, offset=0,
                accepted_len=None, emitted=None, diag=None, workspace=None, stream=None):
    """Rejection-sampling verification of drafted chains.

    target_logits [B, G+1, V] fp32; draft_logits [B, G, V] fp32; draft_tokens
    [B, G] int32; uniforms [B, G+1, 2] fp32 or None (in-kernel Philox4x64-10
    with key (seed, 0), counter (offset, b, j, stream)).
    Returns (accepted_len int32 [B], emitted int32 [B, G+1]).
    """
    lib = _lib.load()
    _dev(target_logits, "target_logits", (torch.float32,))
    _dev(draft_logits, "draft_logits", (torch.float32,))
    _dev(draft_tokens, "draft_tokens", (torch.int32,))
    B, G, V = draft_logits.shape
    _need(target_logits.shape == (B, G + 1, V), "target_logits must be [B, G+1, V]")
    _need(draft_tokens.shape == (B, G), "draft_tokens must be [B, G]")
    if uniforms is not None:
        _dev(uniforms, "uniforms", (torch.float32,))
        _need(uniforms.shape == (B, G + 1, 2), "uniforms must be [B, G+1, 2]")
    accepted_len, emitted = _outputs(accepted_len, emitted, B, G, target_logits.device)
    if diag is not None:
        _dev(diag, "diag", (torch.float32,))
        _need(diag.shape == (B, G + 1, 4), "diag must be [B, G+1, 4]")
    nbytes = int(lib.spec_verify_workspace_size(B, G, V))
    ws = _workspace(nbytes, target_logits.device, workspace)
    st = lib.spec_verify(_ptr(target_logits), _ptr(draft_logits), _ptr(draft_tokens), B, G, V,
                         _ptr(uniforms), int(seed) & (2**64 - 1), int(offset) & (2**64 - 1),
                         _ptr(accepted_len), _ptr(emitted), _ptr(diag), _ptr(ws), nbytes,
                         _stream(stream))
    _lib.check("spec_verify", st)
    return accepted_len, emitted


def spec_verify_greedy(target_logits, draft_tokens, *, accepted_len=None, emitted=None, workspace=None,
                       stream=None):
    """Greedy verification: d_j accepted iff it is the argmax of target row j
    (ties to the lower token id); the first mismatch, or the bonus row, emits
    the argmax.  target_logits [B, G+1, V] fp32; draft_tokens [B, G] int32.
    Returns (accepted_len int32 [B], emitted int32 [B, G+1])."""
    lib = _lib.load()
    _dev(target_logits, "target_logits", (torch.float32,))
    _dev(draft_tokens, "draft_tokens", (torch.int32,))
    B, G1, V = target_logits.shape
    G = G1 - 1
    _need(G >= 1, "target_logits needs G+1 >= 2 rows")
    _need(draft_tokens.shape == (B, G), "draft_tokens must be [B, G]")
    accepted_len, emitted = _outputs(accepted_len, emitted, B, G, target_logits.device)
    nbytes = int(lib.spec_verify_greedy_workspace_size(B, G, V))
    ws = _workspace(nbytes, target_logits.device, workspace)
    st = lib.spec_verify_greedy(_ptr(target_logits), _ptr(draft_tokens), B, G, V, _ptr(accepted_len),
                                _ptr(emitted), _ptr(ws), nbytes, _stream(stream))
    _lib.check("spec_verify_greedy", st)
    return accepted_len, emitted
