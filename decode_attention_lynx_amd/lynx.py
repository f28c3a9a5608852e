"""Thin ctypes binding of liblynx.so (C ABI declared in include/lynx.h).

Argument marshalling only: tensors are passed as device pointers with the
current HIP stream; every step of the codec and the attention runs in the
library's HIP kernels.  Before a call, each tensor is checked to be contiguous,
on the right device, of the right dtype and large enough for what the kernels
read or write (ValueError otherwise), since the C ABI sees only pointers.
Loading fails loudly when the library is missing.
"""
from __future__ import annotations

import ctypes
import os

LYNX_OK = 0
LYNX_EINVAL = -1
LYNX_EALIGN = -2
LYNX_EUNSUPPORTED = -3
LYNX_ENOSPACE = -4
LYNX_ELAUNCH = -5
SEL_ANCHOR = 1
SEL_RESIDUAL = 2
OUT_BF16 = 0
OUT_F32 = 1

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblynx.so")
EXPORTS = ("lynx_strerror", "lynx_stream_sizes", "lynx_encode", "lynx_decode_anchor", "lynx_decode_full",
           "lynx_attn_workspace_bytes", "lynx_attn_anchor", "lynx_attn_verify_workspace_bytes", "lynx_attn_verify",
           "lynx_attn_anchor_paged", "lynx_encode_to_host_staging_bytes", "lynx_encode_to_host",
           "lynx_attn_verify_paged", "lynx_attn_anchor_noalloc")
ATTN_SCRATCH_BYTES = 32 << 20    # LYNX_ATTN_SCRATCH_BYTES

_lib = None


class LynxError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {strerror(status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load liblynx.so once; raise if it was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"liblynx.so not found at {LIB_PATH}; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        c_int, c_float, c_uint, c_size, c_void = (ctypes.c_int, ctypes.c_float, ctypes.c_uint, ctypes.c_size_t,
                                                   ctypes.c_void_p)
        L.lynx_strerror.restype = ctypes.c_char_p
        L.lynx_strerror.argtypes = [c_int]
        L.lynx_stream_sizes.restype = c_int
        L.lynx_stream_sizes.argtypes = [c_int, c_int, c_int, c_int, ctypes.POINTER(c_size), ctypes.POINTER(c_size)]
        L.lynx_encode.restype = c_int
        L.lynx_encode.argtypes = [c_void, c_int, c_int, c_int, c_int, c_int, c_float, c_uint, c_void, c_void, c_void]
        L.lynx_decode_anchor.restype = c_int
        L.lynx_decode_anchor.argtypes = [c_void, c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_void, c_void]
        L.lynx_decode_full.restype = c_int
        L.lynx_decode_full.argtypes = [c_void, c_void, c_int, c_int, c_int, c_int, c_int, c_float, c_int, c_void,
                                       c_void]
        L.lynx_attn_workspace_bytes.restype = c_size
        L.lynx_attn_workspace_bytes.argtypes = [c_int, c_int, c_int, c_int, c_int, c_int, c_int]
        L.lynx_attn_anchor.restype = c_int
        L.lynx_attn_anchor.argtypes = [c_void, c_void, c_void, c_int, c_int, c_int, c_int, c_int, c_int, c_int,
                                       c_float, c_float, c_void, c_size, c_int, c_void, c_void]
        L.lynx_encode_to_host_staging_bytes.restype = c_size
        L.lynx_encode_to_host_staging_bytes.argtypes = [c_int] * 5
        L.lynx_encode_to_host.restype = c_int
        L.lynx_encode_to_host.argtypes = [c_void] + [c_int] * 5 + [c_float, c_int, c_void, c_size, c_void, c_void,
                                                                 c_void, c_void]
        L.lynx_attn_anchor_noalloc.restype = c_int
        L.lynx_attn_anchor_noalloc.argtypes = [c_void, c_void, c_void] + [c_int] * 7 + [c_float, c_float, c_int,
                                                                                        c_void, c_void]
        L.lynx_attn_anchor_paged.restype = c_int
        L.lynx_attn_anchor_paged.argtypes = [c_void, c_void, c_void, c_int, c_void, c_void] + [c_int] * 7 + [
            c_float, c_float, c_void, c_size, c_int, c_void, c_void]
        L.lynx_attn_verify_paged.restype = c_int
        L.lynx_attn_verify_paged.argtypes = [c_void] * 5 + [c_int, c_void, c_void] + [c_int] * 8 + [
            c_float, c_float, c_void, c_size, c_int, c_void, c_void, c_void]
        L.lynx_attn_verify_workspace_bytes.restype = c_size
        L.lynx_attn_verify_workspace_bytes.argtypes = [c_int] * 8
        L.lynx_attn_verify.restype = c_int
        L.lynx_attn_verify.argtypes = [c_void, c_void, c_void, c_void, c_void] + [c_int] * 8 + [
            c_float, c_float, c_void, c_size, c_int, c_void, c_void, c_void]
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().lynx_strerror(int(status)).decode()


def _check(status: int, where: str):
    if status != LYNX_OK:
        raise LynxError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need(t, name: str, nbytes: int, dtypes=None, device: str = "cuda"):
    """Refuse, before any launch, a buffer the kernels would misread or overrun: it must be a
    contiguous tensor on `device` ("cuda" or "cpu"), of one of `dtypes`, holding >= nbytes bytes."""
    if t is None:
        raise ValueError(f"{name}: a tensor is required")
    if (device == "cuda") != bool(t.is_cuda):
        raise ValueError(f"{name}: must be a {'CUDA' if device == 'cuda' else 'host'} tensor")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name}: dtype {t.dtype}, expected one of {tuple(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError(f"{name}: {have} bytes, {nbytes} needed")
    return t


def _out_code(out):
    import torch
    _need(out, "out", 0, (torch.bfloat16, torch.float32))
    return OUT_F32 if out.dtype == torch.float32 else OUT_BF16


def _pages(T: int, page_tokens: int) -> int:
    if page_tokens <= 0 or T % page_tokens != 0:
        raise ValueError(f"{T} tokens are not a whole number of {page_tokens}-token pages")
    return T // page_tokens


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def stream_sizes(page_tokens: int, kv_heads: int, head_dim: int, chunk: int):
    """(anchor segment bytes, residual segment bytes) of one page."""
    a, r = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(lib().lynx_stream_sizes(page_tokens, kv_heads, head_dim, chunk, ctypes.byref(a), ctypes.byref(r)),
           "lynx_stream_sizes")
    return a.value, r.value


def encode(kv, page_tokens: int, chunk: int, alpha: float, residual: bool = True, anchor_out=None,
           residual_out=None, stream=None):
    """kv: CUDA bfloat16 [n_pages*P, Hkv, D].  Returns (anchor uint8 [n_pages, a_seg], residual or None)."""
    import torch
    T, Hkv, D = kv.shape
    n_pages = _pages(T, page_tokens)
    _need(kv, "kv", 0, (torch.bfloat16,))
    a_sz, r_sz = stream_sizes(page_tokens, Hkv, D, chunk)
    if anchor_out is None:
        anchor_out = torch.empty((n_pages, a_sz), dtype=torch.uint8, device=kv.device)
    if residual and residual_out is None:
        residual_out = torch.empty((n_pages, r_sz), dtype=torch.uint8, device=kv.device)
    _need(anchor_out, "anchor_out", n_pages * a_sz)
    if residual:
        _need(residual_out, "residual_out", n_pages * r_sz)
    sel = SEL_ANCHOR | (SEL_RESIDUAL if residual else 0)
    _check(lib().lynx_encode(_ptr(kv), n_pages, page_tokens, Hkv, D, chunk, alpha, sel, _ptr(anchor_out),
                             _ptr(residual_out) if residual else None, _stream(stream)), "lynx_encode")
    return anchor_out, (residual_out if residual else None)


def encode_to_host(kv, page_tokens: int, chunk: int, alpha: float, group_pages: int, anchor_host=None,
                   residual_host=None, staging=None, compute_stream=None, copy_stream=None):
    """Encode kv (CUDA bfloat16 [n_pages*P, Hkv, D]) group by group into pinned host tensors
    (uint8 [n_pages, a_seg] and [n_pages, r_seg]), each group's copy overlapping the next group's
    encode.  Asynchronous: the host tensors are complete once copy_stream has drained.  copy_stream
    defaults to the compute stream (no overlap); pass a second stream to overlap."""
    import torch
    T, Hkv, D = kv.shape
    n_pages = _pages(T, page_tokens)
    _need(kv, "kv", 0, (torch.bfloat16,))
    a_sz, r_sz = stream_sizes(page_tokens, Hkv, D, chunk)
    if anchor_host is None:
        anchor_host = torch.empty((n_pages, a_sz), dtype=torch.uint8, pin_memory=True)
    if residual_host is None:
        residual_host = torch.empty((n_pages, r_sz), dtype=torch.uint8, pin_memory=True)
    _need(anchor_host, "anchor_host", n_pages * a_sz, device="cpu")
    _need(residual_host, "residual_host", n_pages * r_sz, device="cpu")
    gp = max(1, min(group_pages, n_pages))
    need = int(lib().lynx_encode_to_host_staging_bytes(gp, page_tokens, Hkv, D, chunk))
    if staging is None:
        staging = torch.empty(max(need, 16), dtype=torch.uint8, device=kv.device)
    _need(staging, "staging", 0)
    cs = _stream(compute_stream)
    xs = _stream(copy_stream) if copy_stream is not None else cs
    _check(lib().lynx_encode_to_host(_ptr(kv), n_pages, page_tokens, Hkv, D, chunk, alpha, group_pages,
                                     _ptr(staging), staging.numel(), ctypes.c_void_p(anchor_host.data_ptr()),
                                     ctypes.c_void_p(residual_host.data_ptr()), cs, xs), "lynx_encode_to_host")
    return anchor_host, residual_host


def decode_anchor(anchor, n_pages: int, page_tokens: int, kv_heads: int, head_dim: int, chunk: int, alpha: float,
                  out_dtype=None, out=None, stream=None):
    """Anchor segments -> [n_pages*P, Hkv, D] tensor (bfloat16 by default, or float32)."""
    import torch
    a_sz, _ = stream_sizes(page_tokens, kv_heads, head_dim, chunk)
    _need(anchor, "anchor", n_pages * a_sz)
    dt = torch.bfloat16 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((n_pages * page_tokens, kv_heads, head_dim), dtype=dt, device=anchor.device)
    code = _out_code(out)
    _need(out, "out", n_pages * page_tokens * kv_heads * head_dim * out.element_size())
    _check(lib().lynx_decode_anchor(_ptr(anchor), n_pages, page_tokens, kv_heads, head_dim, chunk, alpha, code,
                                    _ptr(out), _stream(stream)), "lynx_decode_anchor")
    return out


def decode_full(anchor, residual, n_pages: int, page_tokens: int, kv_heads: int, head_dim: int, chunk: int,
                alpha: float, out_dtype=None, out=None, stream=None):
    """Anchor + residual segments -> [n_pages*P, Hkv, D] tensor (bfloat16 by default, or float32)."""
    import torch
    a_sz, r_sz = stream_sizes(page_tokens, kv_heads, head_dim, chunk)
    _need(anchor, "anchor", n_pages * a_sz)
    _need(residual, "residual", n_pages * r_sz)
    dt = torch.bfloat16 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((n_pages * page_tokens, kv_heads, head_dim), dtype=dt, device=anchor.device)
    code = _out_code(out)
    _need(out, "out", n_pages * page_tokens * kv_heads * head_dim * out.element_size())
    _check(lib().lynx_decode_full(_ptr(anchor), _ptr(residual), n_pages, page_tokens, kv_heads, head_dim, chunk,
                                  alpha, code, _ptr(out), _stream(stream)), "lynx_decode_full")
    return out


def attn_workspace_bytes(batch: int, ctx_tokens: int, q_heads: int, kv_heads: int, head_dim: int,
                         page_tokens: int, chunk: int) -> int:
    return int(lib().lynx_attn_workspace_bytes(batch, ctx_tokens, q_heads, kv_heads, head_dim, page_tokens, chunk))


def attn_anchor(q, k_anchor, v_anchor, ctx_tokens: int, kv_heads: int, page_tokens: int, chunk: int, alpha: float,
                sm_scale: float = 0.0, out_dtype=None, workspace=None, out=None, stream=None):
    """q: CUDA bfloat16 [B, Hq, D]; k_anchor/v_anchor: B*ctx/P anchor segments.  Returns O [B, Hq, D]."""
    import torch
    B, Hq, D = q.shape
    _need(q, "q", 0, (torch.bfloat16,))
    a_sz, _ = stream_sizes(page_tokens, kv_heads, D, chunk)
    seg = B * _pages(ctx_tokens, page_tokens) * a_sz
    _need(k_anchor, "k_anchor", seg)
    _need(v_anchor, "v_anchor", seg)
    ws = attn_workspace_bytes(B, ctx_tokens, Hq, kv_heads, D, page_tokens, chunk)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", 0)
    dt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dt, device=q.device)
    code = _out_code(out)
    _need(out, "out", B * Hq * D * out.element_size())
    _check(lib().lynx_attn_anchor(_ptr(q), _ptr(k_anchor), _ptr(v_anchor), B, ctx_tokens, Hq, kv_heads, D,
                                  page_tokens, chunk, alpha, sm_scale, _ptr(workspace), workspace.numel(), code,
                                  _ptr(out), _stream(stream)), "lynx_attn_anchor")
    return out


def attn_anchor_noalloc(q, k_anchor, v_anchor, ctx_tokens: int, kv_heads: int, page_tokens: int, chunk: int,
                        alpha: float, sm_scale: float = 0.0, out_dtype=None, out=None, stream=None):
    """attn_anchor without a workspace: the library's per-GPU buffer holds the partial results
    (no device allocation by the library; `out` is allocated here when not given)."""
    import torch
    B, Hq, D = q.shape
    _need(q, "q", 0, (torch.bfloat16,))
    a_sz, _ = stream_sizes(page_tokens, kv_heads, D, chunk)
    seg = B * _pages(ctx_tokens, page_tokens) * a_sz
    _need(k_anchor, "k_anchor", seg)
    _need(v_anchor, "v_anchor", seg)
    dt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dt, device=q.device)
    code = _out_code(out)
    _need(out, "out", B * Hq * D * out.element_size())
    _check(lib().lynx_attn_anchor_noalloc(_ptr(q), _ptr(k_anchor), _ptr(v_anchor), B, ctx_tokens, Hq, kv_heads, D,
                                          page_tokens, chunk, alpha, sm_scale, code, _ptr(out), _stream(stream)),
           "lynx_attn_anchor_noalloc")
    return out


def attn_anchor_paged(q, k_pool, v_pool, block_table, seq_lens, kv_heads: int, page_tokens: int, chunk: int,
                      alpha: float, sm_scale: float = 0.0, out_dtype=None, workspace=None, out=None, stream=None):
    """q: CUDA bfloat16 [B, Hq, D]; k_pool / v_pool: [n_pool, anchor_seg] uint8; block_table: CUDA int32
    [B, max_pages]; seq_lens: CUDA int32 [B].  Returns O [B, Hq, D]."""
    import torch
    B, Hq, D = q.shape
    _need(q, "q", 0, (torch.bfloat16,))
    n_pool = k_pool.shape[0]
    max_pages = block_table.shape[1]
    a_sz, _ = stream_sizes(page_tokens, kv_heads, D, chunk)
    _need(k_pool, "k_pool", n_pool * a_sz)
    _need(v_pool, "v_pool", n_pool * a_sz)
    _need(block_table, "block_table", B * max_pages * 4, (torch.int32,))
    _need(seq_lens, "seq_lens", B * 4, (torch.int32,))
    ws = attn_workspace_bytes(B, max_pages * page_tokens, Hq, kv_heads, D, page_tokens, chunk)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", 0)
    dt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, Hq, D), dtype=dt, device=q.device)
    code = _out_code(out)
    _need(out, "out", B * Hq * D * out.element_size())
    _check(lib().lynx_attn_anchor_paged(_ptr(q), _ptr(k_pool), _ptr(v_pool), n_pool, _ptr(block_table),
                                        _ptr(seq_lens), B, max_pages, Hq, kv_heads, D, page_tokens, chunk, alpha,
                                        sm_scale, _ptr(workspace), workspace.numel(), code, _ptr(out),
                                        _stream(stream)), "lynx_attn_anchor_paged")
    return out


def attn_verify_workspace_bytes(batch: int, n_query: int, ctx_tokens: int, q_heads: int, kv_heads: int,
                                head_dim: int, page_tokens: int, chunk: int) -> int:
    return int(lib().lynx_attn_verify_workspace_bytes(batch, n_query, ctx_tokens, q_heads, kv_heads, head_dim,
                                                      page_tokens, chunk))


def attn_verify(q, k_anchor, k_residual, v_anchor, v_residual, ctx_tokens: int, kv_heads: int, page_tokens: int,
                chunk: int, alpha: float, sm_scale: float = 0.0, out_dtype=None, want_lse: bool = True,
                workspace=None, out=None, lse=None, stream=None):
    """q: CUDA bfloat16 [B, M, Hq, D]; K/V anchor and residual: B*ctx/P segments each.

    Returns (O [B, M, Hq, D], lse float32 [B, M, Hq] natural log, or None when want_lse is False)."""
    import torch
    B, M, Hq, D = q.shape
    _need(q, "q", 0, (torch.bfloat16,))
    a_sz, r_sz = stream_sizes(page_tokens, kv_heads, D, chunk)
    n_seg = B * _pages(ctx_tokens, page_tokens)
    for t, name, sz in ((k_anchor, "k_anchor", a_sz), (v_anchor, "v_anchor", a_sz), (k_residual, "k_residual", r_sz),
                        (v_residual, "v_residual", r_sz)):
        _need(t, name, n_seg * sz)
    ws = attn_verify_workspace_bytes(B, M, ctx_tokens, Hq, kv_heads, D, page_tokens, chunk)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", 0)
    dt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, M, Hq, D), dtype=dt, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, M, Hq), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    code = _out_code(out)
    _need(out, "out", B * M * Hq * D * out.element_size())
    if lse is not None:
        _need(lse, "lse", B * M * Hq * 4, (torch.float32,))
    _check(lib().lynx_attn_verify(_ptr(q), _ptr(k_anchor), _ptr(k_residual), _ptr(v_anchor), _ptr(v_residual), B, M,
                                  ctx_tokens, Hq, kv_heads, D, page_tokens, chunk, alpha, sm_scale, _ptr(workspace),
                                  workspace.numel(), code, _ptr(out), _ptr(lse), _stream(stream)),
           "lynx_attn_verify")
    return out, lse


def attn_verify_paged(q, k_anchor_pool, k_residual_pool, v_anchor_pool, v_residual_pool, block_table, seq_lens,
                      kv_heads: int, page_tokens: int, chunk: int, alpha: float, sm_scale: float = 0.0,
                      out_dtype=None, want_lse: bool = True, workspace=None, out=None, lse=None, stream=None):
    """q: CUDA bfloat16 [B, M, Hq, D]; pools: [n_pool, seg] uint8 each; block_table: CUDA int32 [B, max_pages];
    seq_lens: CUDA int32 [B].  Returns (O [B, M, Hq, D], lse [B, M, Hq] or None)."""
    import torch
    B, M, Hq, D = q.shape
    _need(q, "q", 0, (torch.bfloat16,))
    n_pool = k_anchor_pool.shape[0]
    max_pages = block_table.shape[1]
    a_sz, r_sz = stream_sizes(page_tokens, kv_heads, D, chunk)
    for t, name, sz in ((k_anchor_pool, "k_anchor_pool", a_sz), (v_anchor_pool, "v_anchor_pool", a_sz),
                        (k_residual_pool, "k_residual_pool", r_sz), (v_residual_pool, "v_residual_pool", r_sz)):
        _need(t, name, n_pool * sz)
    _need(block_table, "block_table", B * max_pages * 4, (torch.int32,))
    _need(seq_lens, "seq_lens", B * 4, (torch.int32,))
    ws = attn_verify_workspace_bytes(B, M, max_pages * page_tokens, Hq, kv_heads, D, page_tokens, chunk)
    if workspace is None:
        workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", 0)
    dt = torch.float32 if out_dtype is None else out_dtype
    if out is None:
        out = torch.empty((B, M, Hq, D), dtype=dt, device=q.device)
    if want_lse and lse is None:
        lse = torch.empty((B, M, Hq), dtype=torch.float32, device=q.device)
    if not want_lse:
        lse = None
    code = _out_code(out)
    _need(out, "out", B * M * Hq * D * out.element_size())
    if lse is not None:
        _need(lse, "lse", B * M * Hq * 4, (torch.float32,))
    _check(lib().lynx_attn_verify_paged(_ptr(q), _ptr(k_anchor_pool), _ptr(k_residual_pool), _ptr(v_anchor_pool),
                                        _ptr(v_residual_pool), n_pool, _ptr(block_table), _ptr(seq_lens), B, M,
                                        max_pages, Hq, kv_heads, D, page_tokens, chunk, alpha, sm_scale,
                                        _ptr(workspace), workspace.numel(), code, _ptr(out), _ptr(lse),
                                        _stream(stream)), "lynx_attn_verify_paged")
    return out, lse
