"""Exact attention forward and backward passes for MI355X (gfx950): Python binding.

Every step of the computation runs in the HIP kernels of ``libfa_fwd.so``
behind the C ABI of ``include/fa.h``; this package only marshals torch tensors
(device memory and the current stream) into that call. There is no CPU
fallback: a missing library raises.
"""
from __future__ import annotations

import math

from ._lib import (  # noqa: F401
    FA_BF16, FA_ERR_INVALID_ARG, FA_ERR_LAUNCH, FA_ERR_TOO_LARGE, FA_ERR_UNSUPPORTED, FA_F16,
    FA_FP8_E4M3, FA_NOALLOC_SCRATCH_BYTES, FA_OK, FaError, fa_bwd, fa_fwd, fa_fwd_fp8,
    fa_fwd_fp8_block, fa_fwd_kv, fa_fwd_kv_noalloc, fa_fwd_kv_workspace,
    fa_fwd_varlen, fa_fwd_varlen_workspace, fa_quantize_fp8, fa_varlen_order, lib, strerror,
    version,
)

__all__ = ["forward", "forward_fp8", "forward_fp8_block", "quantize_fp8", "forward_kv",
           "forward_kv_noalloc", "forward_varlen", "backward", "fa_fwd", "fa_fwd_fp8",
           "fa_fwd_fp8_block", "fa_quantize_fp8", "fa_fwd_kv", "fa_fwd_kv_noalloc",
           "fa_fwd_varlen", "fa_varlen_order", "varlen_order",
           "fa_bwd", "FaError", "strerror", "version"]


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"q/k/v must be float16 or bfloat16, got {t.dtype}")


def _check(q, k, v):
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    for t in (k, v):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must share shape, dtype and device")
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous [B, H, N, d]")
    if q.device.type != "cuda":
        raise ValueError("q, k, v must be on a GPU")


def _check_buf(t, shape, dtype, device, name):
    """A caller-supplied output or work buffer must be exactly what the kernel
    writes: the kernels see only its address, so a short, strided, mistyped or
    host tensor would be written out of bounds or through a host pointer."""
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _check_workspace(t, need_bytes, device):
    """A float32 work buffer of at least ``need_bytes`` bytes on ``device``."""
    torch = _torch()
    if t.device != device or t.dtype != torch.float32 or not t.is_contiguous() \
            or t.numel() * 4 < need_bytes:
        raise ValueError(f"workspace must be a contiguous float32 tensor on {device} with at "
                         f"least {need_bytes // 4} elements")


def _check_fp8(q8, k8, v8):
    if q8.dim() != 4:
        raise ValueError("fp8 q, k, v must be [B, H, N, d]")
    for t in (k8, v8):
        if t.shape != q8.shape or t.device != q8.device:
            raise ValueError("q, k, v must share shape and device")
    for t in (q8, k8, v8):
        if t.element_size() != 1 or not t.is_contiguous():
            raise ValueError("fp8 inputs must be contiguous 1-byte tensors")
    if q8.device.type != "cuda":
        raise ValueError("fp8 q, k, v must be on a GPU")


def forward(q, k, v, causal: bool = False, scale: float | None = None, out=None, lse=None):
    """O, LSE = attention(q, k, v) for f16/bf16 tensors [B, H, N, d] on the GPU.

    Returns ``(o, lse)``: ``o`` has q's dtype and shape, ``lse`` is float32
    [B, H, N] (natural log). The launch is queued on the current stream.
    """
    torch = _torch()
    _check(q, k, v)
    B, H, N, d = q.shape
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_buf(out, q.shape, q.dtype, q.device, "out")
    _check_buf(lse, (B, H, N), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                B, H, N, d, scale, int(bool(causal)), dt, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd")
    return out, lse


def forward_fp8(q8, k8, v8, descale, causal: bool = False, scale: float | None = None,
                out=None, lse=None):
    """Attention for e4m3fn codes (uint8 or float8_e4m3fn tensors [B, H, N, d])
    with per-tensor descales ``(s_q, s_k, s_v)``; returns bf16 O and fp32 LSE."""
    torch = _torch()
    _check_fp8(q8, k8, v8)
    B, H, N, d = q8.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check_buf(out, (B, H, N, d), torch.bfloat16, q8.device, "out")
    _check_buf(lse, (B, H, N), torch.float32, q8.device, "lse")
    stream = torch.cuda.current_stream(q8.device).cuda_stream
    sq, sk, sv = (float(x) for x in descale)
    rc = fa_fwd_fp8(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(), lse.data_ptr(),
                    sq, sk, sv, B, H, N, d, scale, int(bool(causal)), stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_fp8")
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, scale: float | None = None,
             dq=None, dk=None, dv=None, workspace=None):
    """dQ, dK, dV of attention for f16/bf16 tensors [B, H, N, d] on the GPU,
    given the forward's ``o`` and ``lse`` and the upstream gradient ``dout``.

    Returns ``(dq, dk, dv)`` in q's dtype. ``workspace`` (float32, at least
    2*B*H*N elements) is allocated when not given; on return its first B*H*N
    values hold -D = -rowsum(dout * o). Queued on the current stream.
    """
    torch = _torch()
    _check(q, k, v)
    for t in (o, dout):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device or not t.is_contiguous():
            raise ValueError("o and dout must match q (shape, dtype, device, contiguous)")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if lse.device != q.device:
        raise ValueError("lse must be on q's device")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(q) if dk is None else dk
    dv = torch.empty_like(q) if dv is None else dv
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        _check_buf(t, q.shape, q.dtype, q.device, name)
    if workspace is None:
        workspace = torch.empty(2 * B * H * N, dtype=torch.float32, device=q.device)
    else:
        _check_workspace(workspace, 8 * B * H * N, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                B, H, N, d, scale, int(bool(causal)), dt, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_bwd")
    return dq, dk, dv


def default_splits(B, H, Hkv, Nq, Nk) -> int:
    """Key ranges for fa_fwd_kv when the query tiles alone cannot fill the chip.

    Two workgroups per CU (512 on 256 CUs) give the most bytes in flight, and
    a workgroup should stream at least 4096 keys to amortise its prologue
    (Q load, LDS set-up, the first copies' latency) and its partial write.
    Take 512 workgroups if each still gets 4096 keys, else 256 if that does,
    else 512 with at least 256 keys per range (short histories).
    """
    base = B * Hkv * (-(-(H // Hkv) * Nq // 128))
    base = max(base, 1)
    two, one = -(-512 // base), -(-256 // base)
    for s in (two, one):
        if Nk // s >= 4096:
            return int(max(1, min(s, 1024)))
    return int(max(1, min(two, Nk // 256, 1024)))


def forward_kv(q, k, v, causal: bool = False, scale: float | None = None,
               num_splits: int | None = None, out=None, lse=None, workspace=None):
    """Grouped-query attention over a key/value history: q [B, H, Nq, d], k and
    v [B, Hkv, Nk, d] (H a multiple of Hkv, f16/bf16, contiguous, on the GPU).
    The queries are the last Nq of the Nk positions (causal: query i sees keys
    j <= i + Nk - Nq). ``num_splits`` key ranges are computed in parallel and
    merged (``None`` picks one). Returns ``(o, lse)`` like ``forward``."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Nq, d]; k and v [B, Hkv, Nk, d]")
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous, of one dtype, on one device")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must match q's batch and head dimension")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_splits(B, H, max(Hkv, 1), Nq, Nk)
    if q.device.type != "cuda":
        raise ValueError("q, k, v must be on a GPU")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_buf(out, q.shape, q.dtype, q.device, "out")
    _check_buf(lse, (B, H, Nq), torch.float32, q.device, "lse")
    ws_ptr = 0
    need = fa_fwd_kv_workspace(B, H, Nq, d, num_splits)
    if need:
        if workspace is None:
            workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        else:
            _check_workspace(workspace, need, q.device)
        ws_ptr = workspace.data_ptr()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   B, H, Hkv, Nq, Nk, d, scale, int(bool(causal)), dt, num_splits, ws_ptr or None,
                   stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_kv")
    return out, lse


def forward_kv_noalloc(q, k, v, causal: bool = False, scale: float | None = None,
                       num_splits: int | None = None, out=None, lse=None):
    """``forward_kv`` through the allocation-free entry point: the key-range
    partials live in the library's static per-device scratch
    (FA_NOALLOC_SCRATCH_BYTES), so the library allocates nothing; pass ``out``
    and ``lse`` to allocate nothing here either. ``num_splits`` None picks
    ``default_splits``, lowered to what the scratch holds; an explicit count
    whose partials do not fit raises FaError(FA_ERR_TOO_LARGE). Calls that can
    overlap in time on one GPU share the scratch and must not run
    concurrently."""
    torch = _torch()
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, H, Nq, d]; k and v [B, Hkv, Nk, d]")
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous, of one dtype, on one device")
    if q.device.type != "cuda":
        raise ValueError("q, k, v must be on a GPU")
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != d:
        raise ValueError("k and v must match q's batch and head dimension")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if num_splits is None:
        num_splits = default_splits(B, H, max(Hkv, 1), Nq, Nk)
        per_split = fa_fwd_kv_workspace(B, H, Nq, d, 2) // 2 if B * H * Nq else 0
        if per_split:
            num_splits = max(1, min(num_splits, FA_NOALLOC_SCRATCH_BYTES // per_split))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check_buf(out, q.shape, q.dtype, q.device, "out")
    _check_buf(lse, (B, H, Nq), torch.float32, q.device, "lse")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_fwd_kv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                           lse.data_ptr(), B, H, Hkv, Nq, Nk, d, scale, int(bool(causal)), dt,
                           num_splits, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_kv_noalloc")
    return out, lse


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                   causal: bool = False, scale: float | None = None, num_splits: int = 1,
                   out=None, lse=None, workspace=None, order=None):
    """Attention over B sequences of different lengths packed token-major:
    q [total_q, H, d], k and v [total_k, Hkv, d] (f16/bf16, contiguous, on the
    GPU), cu_seqlens_q / cu_seqlens_k int32 device tensors of B+1 offsets.
    Sequence b is queries cu_seqlens_q[b]:cu_seqlens_q[b+1] against keys
    cu_seqlens_k[b]:cu_seqlens_k[b+1]; causal is bottom-right within each
    sequence. ``order`` (int32 [B] on the GPU, from :func:`varlen_order`) makes
    the kernel run the sequences in that order; the results do not change.
    Returns ``(o, lse)`` with o like q and lse float32 [total_q, H]."""
    torch = _torch()
    if q.dim() != 3 or k.dim() != 3 or k.shape != v.shape:
        raise ValueError("q must be [total_q, H, d]; k and v [total_k, Hkv, d]")
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous, of one dtype, on one device")
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous() or c.device != q.device:
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors on q's device")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B+1 offsets")
    total_q, H, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    if k.shape[2] != d:
        raise ValueError("k and v must match q's head dimension")
    B = cu_seqlens_q.numel() - 1
    if order is not None and (order.dtype != torch.int32 or order.dim() != 1 or order.numel() != B
                              or not order.is_contiguous() or order.device != q.device):
        raise ValueError("order must be a contiguous 1-D int32 tensor of B entries on q's device")
    dt = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q.device.type != "cuda":
        raise ValueError("q, k, v must be on a GPU")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((total_q, H), dtype=torch.float32, device=q.device)
    _check_buf(out, q.shape, q.dtype, q.device, "out")
    _check_buf(lse, (total_q, H), torch.float32, q.device, "lse")
    ws_ptr = 0
    need = fa_fwd_varlen_workspace(total_q, H, d, num_splits)
    if need:
        if workspace is None:
            workspace = torch.empty(need // 4, dtype=torch.float32, device=q.device)
        else:
            _check_workspace(workspace, need, q.device)
        ws_ptr = workspace.data_ptr()
    stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                       cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(),
                       order.data_ptr() if order is not None else None, B, H, Hkv,
                       int(max_seqlen_q), int(max_seqlen_k), total_q, total_k, d, scale,
                       int(bool(causal)), dt, num_splits, ws_ptr or None, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_varlen")
    return out, lse


def varlen_order(cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                 num_splits: int = 1, total_q: int | None = None, total_k: int | None = None,
                 out=None):
    """Longest-first order of a variable-length batch (int32 [B] on the GPU):
    out[v] is the sequence the kernel runs as virtual sequence v, heaviest
    work tile first, for the ``order`` argument of :func:`forward_varlen` with
    the same lengths and ``num_splits``. ``total_q`` / ``total_k`` default to
    the last offsets, which the kernel reads on the device: pass the token
    counts of q and k to avoid that read on the host."""
    torch = _torch()
    for c in (cu_seqlens_q, cu_seqlens_k):
        if c.dtype != torch.int32 or c.dim() != 1 or not c.is_contiguous() or c.device.type != "cuda":
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors on the GPU")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B+1 offsets")
    if cu_seqlens_k.device != cu_seqlens_q.device:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be on one device")
    B = cu_seqlens_q.numel() - 1
    if total_q is None:
        total_q = int(cu_seqlens_q[-1])
    if total_k is None:
        total_k = int(cu_seqlens_k[-1])
    if out is None:
        out = torch.empty(B, dtype=torch.int32, device=cu_seqlens_q.device)
    elif out.dtype != torch.int32 or out.numel() != B or not out.is_contiguous() \
            or out.device != cu_seqlens_q.device:
        raise ValueError("out must be a contiguous int32 tensor of B entries on the offsets' device")
    stream = torch.cuda.current_stream(cu_seqlens_q.device).cuda_stream
    rc = fa_varlen_order(cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, int(max_seqlen_q),
                         int(max_seqlen_k), int(total_q), int(total_k), int(num_splits),
                         out.data_ptr() if B else None, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_varlen_order")
    return out


def quantize_fp8(x, block_rows: int, signs=None, out=None, scales=None):
    """e4m3 codes of x ([B, H, N, d] f16/bf16 on the GPU) with one float32
    scale per block of ``block_rows`` rows (64 or 128), after the random-sign
    Hadamard transform when ``signs`` (float32 [d] of +-1 on the GPU) is given.
    Returns ``(codes uint8 [B, H, N, d], scales float32 [B, H, ceil(N/block_rows)])``."""
    torch = _torch()
    if x.dim() != 4 or not x.is_contiguous() or x.device.type != "cuda":
        raise ValueError("x must be a contiguous [B, H, N, d] tensor on the GPU")
    B, H, N, d = x.shape
    dt = _dtype_code(x)
    nb = -(-N // block_rows) if block_rows > 0 else 0
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((B, H, nb), dtype=torch.float32, device=x.device)
    if out.device != x.device or out.element_size() != 1 or tuple(out.shape) != (B, H, N, d) \
            or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous 1-byte tensor {(B, H, N, d)} on {x.device}")
    _check_buf(scales, (B, H, nb), torch.float32, x.device, "scales")
    sp = None
    if signs is not None:
        if signs.dtype != torch.float32 or signs.numel() != d or not signs.is_contiguous() \
                or signs.device != x.device:
            raise ValueError("signs must be a contiguous float32 tensor of d values on x's device")
        sp = signs.data_ptr()
    stream = torch.cuda.current_stream(x.device).cuda_stream
    rc = fa_quantize_fp8(x.data_ptr(), out.data_ptr(), scales.data_ptr(), sp, B, H, N, d,
                         block_rows, dt, stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_quantize_fp8")
    return out, scales


def forward_fp8_block(q8, k8, v8, q_scale, k_scale, v_scale, causal: bool = False,
                      scale: float | None = None, out=None, lse=None):
    """Attention for e4m3 codes [B, H, N, d] with block scales: q_scale
    [B, H, ceil(N/128)], k_scale and v_scale [B, H, ceil(N/64)] (float32, on
    the GPU). Returns bf16 O and fp32 LSE."""
    torch = _torch()
    _check_fp8(q8, k8, v8)
    B, H, N, d = q8.shape
    for t, rows in ((q_scale, 128), (k_scale, 64), (v_scale, 64)):
        if t.dtype != torch.float32 or not t.is_contiguous() or t.numel() != B * H * -(-N // rows) \
                or t.device != q8.device:
            raise ValueError("scales must be contiguous float32 [B, H, ceil(N/rows)] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    _check_buf(out, (B, H, N, d), torch.bfloat16, q8.device, "out")
    _check_buf(lse, (B, H, N), torch.float32, q8.device, "lse")
    stream = torch.cuda.current_stream(q8.device).cuda_stream
    rc = fa_fwd_fp8_block(q8.data_ptr(), k8.data_ptr(), v8.data_ptr(), out.data_ptr(),
                          lse.data_ptr(), q_scale.data_ptr(), k_scale.data_ptr(),
                          v_scale.data_ptr(), B, H, N, d, scale, int(bool(causal)), stream)
    if rc != FA_OK:
        raise FaError(rc, "fa_fwd_fp8_block")
    return out, lse
