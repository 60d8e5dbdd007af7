"""PyTorch-facing binding of the C ABI (same names as include/mha_fwd.h).

PyTorch supplies device memory and the current stream; the tensors' data
pointers go straight to the library, which does all of the computation.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from . import _native as nat


def _dtype_code(q: torch.Tensor) -> int:
    if q.dtype == torch.float32:
        return nat.MHA_DTYPE_F32
    if q.dtype == torch.bfloat16:
        return nat.MHA_DTYPE_BF16
    if q.dtype in (torch.float8_e4m3fn, torch.uint8):
        return nat.MHA_DTYPE_FP8_E4M3
    raise ValueError(f"unsupported q dtype {q.dtype}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _need(t: Optional[torch.Tensor], name: str, device, dtype=None, shape=None):
    if t is None:
        return
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def mha_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
            causal: bool = False,
            cu_seqlens: Optional[torch.Tensor] = None,
            max_seqlen: Optional[int] = None,
            q_rope: Optional[torch.Tensor] = None,
            k_rope: Optional[torch.Tensor] = None,
            q_scale: Optional[torch.Tensor] = None,
            k_scale: Optional[torch.Tensor] = None,
            softmax_scale: Optional[float] = None,
            out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None,
            num_splits: int = 1,
            o_partial: Optional[torch.Tensor] = None,
            lse_partial: Optional[torch.Tensor] = None,
            fp8_fast_accum: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """Fused attention forward; returns (o, lse).

    fp8_fast_accum (fp8 inputs only) selects MHA_DTYPE_FP8_E4M3_FASTACC: Q K^T
    on the fp8 matrix instruction (twice the rate of the exact default, which
    decodes the codes to bfloat16), whose accumulation keeps about 13 bits
    below the largest product, so the LSE of rows with large scores can be
    off by more than 1e-3.

    num_splits > 1 runs mha_fwd_splitkv: the keys of every query tile are cut
    into that many ranges run as separate work items, then merged
    (mha_combine_splits); o_partial [num_splits, T, Hq, Dv] and lse_partial
    [num_splits, Hq, T] float32 are its scratch (allocated when not given;
    they hold the per-split partial results afterwards).

    q [T, Hq, Dn], k [T, Hkv, Dn], v [T, Hkv, Dv] with cu_seqlens (int32
    [B+1], on the device) and max_seqlen; or q [B, S, Hq, Dn] etc. for a dense
    batch (no cu_seqlens).  o has q's leading shape with Dv columns; lse is
    [Hq, T] float32 (natural log).  fp8: q, k as float8_e4m3fn (or uint8
    codes) with q_scale [T, Hq] and k_scale [T, Hkv] float32; v bf16.
    """
    if fp8_fast_accum and q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError("fp8_fast_accum applies to fp8 inputs only")
    dense = q.dim() == 4
    if dense:
        if cu_seqlens is not None:
            raise ValueError("cu_seqlens is for packed [T, H, D] inputs")
        B, S = q.shape[0], q.shape[1]
        flat = lambda t: None if t is None else t.reshape(B * S, *t.shape[2:])
        qf, kf, vf = flat(q), flat(k), flat(v)
        qrf, krf = flat(q_rope), flat(k_rope)
        qsf, ksf = flat(q_scale), flat(k_scale)
        cu = torch.arange(0, (B + 1) * S, S, dtype=torch.int32, device=q.device)
        max_seqlen = S
    else:
        if cu_seqlens is None or max_seqlen is None:
            raise ValueError("packed inputs need cu_seqlens and max_seqlen")
        qf, kf, vf, qrf, krf, qsf, ksf = q, k, v, q_rope, k_rope, q_scale, k_scale
        cu = cu_seqlens
        B = cu.numel() - 1
    if qf.dim() != 3 or kf.dim() != 3 or vf.dim() != 3:
        raise ValueError("q, k, v must be [T, H, D] (or [B, S, H, D])")
    dev = qf.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    code = _dtype_code(qf)
    if fp8_fast_accum:
        code = nat.MHA_DTYPE_FP8_E4M3_FASTACC
    T, Hq, Dn = qf.shape
    Hkv, Dv = kf.shape[1], vf.shape[2]
    Dr = 0 if qrf is None else qrf.shape[2]
    vdt = torch.float32 if code == nat.MHA_DTYPE_F32 else torch.bfloat16
    _need(qf, "q", dev)
    _need(kf, "k", dev, qf.dtype, (T, Hkv, Dn))
    _need(vf, "v", dev, vdt, (T, Hkv, Dv))
    _need(qrf, "q_rope", dev, vdt, (T, Hq, Dr) if Dr else None)
    _need(krf, "k_rope", dev, vdt, (T, Hkv, Dr) if Dr else None)
    _need(qsf, "q_scale", dev, torch.float32, (T, Hq) if qsf is not None else None)
    _need(ksf, "k_scale", dev, torch.float32, (T, Hkv) if ksf is not None else None)
    _need(cu, "cu_seqlens", dev, torch.int32, (B + 1,))
    o = out if out is not None else torch.empty((T, Hq, Dv), dtype=vdt, device=dev)
    _need(o, "out", dev, vdt, (T, Hq, Dv))
    lse_t = lse if lse is not None else torch.empty((Hq, T), dtype=torch.float32, device=dev)
    _need(lse_t, "lse", dev, torch.float32, (Hq, T))
    stream = torch.cuda.current_stream(dev).cuda_stream
    lib = nat.load()
    scale_arg = float(softmax_scale) if softmax_scale is not None else 0.0
    with torch.cuda.device(dev):
        if num_splits == 1 and o_partial is None and lse_partial is None:
            st = lib.mha_fwd(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(o), _ptr(lse_t),
                             _ptr(cu), int(B), int(max_seqlen), int(Hq), int(Hkv),
                             int(Dn), int(Dr), int(Dv), _ptr(qrf), _ptr(krf),
                             int(bool(causal)), scale_arg, code, _ptr(qsf), _ptr(ksf), stream)
        else:
            op = o_partial if o_partial is not None else torch.empty(
                (num_splits, T, Hq, Dv), dtype=torch.float32, device=dev)
            lp = lse_partial if lse_partial is not None else torch.empty(
                (num_splits, Hq, T), dtype=torch.float32, device=dev)
            _need(op, "o_partial", dev, torch.float32, (num_splits, T, Hq, Dv))
            _need(lp, "lse_partial", dev, torch.float32, (num_splits, Hq, T))
            st = lib.mha_fwd_splitkv(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(o), _ptr(lse_t),
                                     _ptr(cu), int(B), int(max_seqlen), int(Hq), int(Hkv),
                                     int(Dn), int(Dr), int(Dv), _ptr(qrf), _ptr(krf),
                                     int(bool(causal)), scale_arg, code, _ptr(qsf), _ptr(ksf),
                                     int(T), int(num_splits), _ptr(op), _ptr(lp), stream)
    nat.check(st)
    if dense:
        o = o.view(B, S, Hq, Dv)
    return o, lse_t


def mha_fwd_noalloc(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                    out: torch.Tensor, lse: torch.Tensor, cu_seqlens: torch.Tensor,
                    max_seqlen: int, causal: bool = False,
                    q_rope: Optional[torch.Tensor] = None,
                    k_rope: Optional[torch.Tensor] = None,
                    q_scale: Optional[torch.Tensor] = None,
                    k_scale: Optional[torch.Tensor] = None,
                    softmax_scale: Optional[float] = None,
                    fp8_fast_accum: bool = False) -> Tuple[torch.Tensor, torch.Tensor]:
    """mha_fwd_noalloc of the C ABI: mha_fwd on the library's fixed workspace,
    allocating nothing on the device (packed [T, H, D] inputs only; out [T,
    Hq, Dv] and lse [Hq, T] must be given).  Returns (out, lse)."""
    if fp8_fast_accum and q.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise ValueError("fp8_fast_accum applies to fp8 inputs only")
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, H, D]")
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    code = nat.MHA_DTYPE_FP8_E4M3_FASTACC if fp8_fast_accum else _dtype_code(q)
    T, Hq, Dn = q.shape
    Hkv, Dv = k.shape[1], v.shape[2]
    Dr = 0 if q_rope is None else q_rope.shape[2]
    vdt = torch.float32 if code == nat.MHA_DTYPE_F32 else torch.bfloat16
    B = cu_seqlens.numel() - 1
    _need(q, "q", dev)
    _need(k, "k", dev, q.dtype, (T, Hkv, Dn))
    _need(v, "v", dev, vdt, (T, Hkv, Dv))
    _need(q_rope, "q_rope", dev, vdt, (T, Hq, Dr) if Dr else None)
    _need(k_rope, "k_rope", dev, vdt, (T, Hkv, Dr) if Dr else None)
    _need(q_scale, "q_scale", dev, torch.float32, (T, Hq) if q_scale is not None else None)
    _need(k_scale, "k_scale", dev, torch.float32, (T, Hkv) if k_scale is not None else None)
    _need(cu_seqlens, "cu_seqlens", dev, torch.int32, (B + 1,))
    _need(out, "out", dev, vdt, (T, Hq, Dv))
    _need(lse, "lse", dev, torch.float32, (Hq, T))
    stream = torch.cuda.current_stream(dev).cuda_stream
    scale_arg = float(softmax_scale) if softmax_scale is not None else 0.0
    with torch.cuda.device(dev):
        st = nat.load().mha_fwd_noalloc(
            _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(cu_seqlens), int(B),
            int(max_seqlen), int(Hq), int(Hkv), int(Dn), int(Dr), int(Dv), _ptr(q_rope),
            _ptr(k_rope), int(bool(causal)), scale_arg, code, _ptr(q_scale), _ptr(k_scale),
            stream)
    nat.check(st)
    return out, lse


def mha_fwd_supported(dtype_code: int, head_dim_nope: int, head_dim_rope: int, v_dim: int) -> bool:
    return bool(nat.load().mha_fwd_supported(dtype_code, head_dim_nope, head_dim_rope, v_dim))


def mha_fwd_kernel_info(dtype_code: int, head_dim_nope: int, head_dim_rope: int,
                        v_dim: int) -> dict:
    """Launch facts of the kernel mha_fwd uses for this shape on the current device."""
    import ctypes
    vals = [ctypes.c_int32(0) for _ in range(4)]
    st = nat.load().mha_fwd_kernel_info(dtype_code, head_dim_nope, head_dim_rope, v_dim,
                                        *[ctypes.byref(v) for v in vals])
    nat.check(st)
    return dict(zip(("block_m", "blocks_per_cu", "grid", "lds_bytes"), (v.value for v in vals)))


def mha_sched_visit(cu_seqlens: torch.Tensor, max_seqlen: int, num_heads: int,
                    num_kv_heads: int, causal: bool, block_m: int = 256,
                    grid: int = 0, protocol: int = 1) -> torch.Tensor:
    """Runs the scheduler alone; returns visit counts [Hq, B, tiles] (int32).
    protocol 0: next item reserved when an item starts and read after the
    item's work, as the float32 kernel does; 1: reserved and read near the end
    of an item, as the matrix-core kernel does."""
    B = cu_seqlens.numel() - 1
    tiles = (max_seqlen + block_m - 1) // block_m
    visits = torch.zeros((num_heads, B, max(tiles, 1)), dtype=torch.int32,
                         device=cu_seqlens.device)
    stream = torch.cuda.current_stream(cu_seqlens.device).cuda_stream
    with torch.cuda.device(cu_seqlens.device):
        st = nat.load().mha_sched_visit(_ptr(cu_seqlens), int(B), int(max_seqlen),
                                        int(num_heads), int(num_kv_heads), int(bool(causal)),
                                        int(block_m), int(grid), int(protocol), _ptr(visits),
                                        stream)
    nat.check(st)
    return visits


def mha_quantize_fp8(x: torch.Tensor, *, codes: Optional[torch.Tensor] = None,
                     scales: Optional[torch.Tensor] = None):
    """Per-row fp8 quantisation on the GPU (mha_quantize_fp8 of the C ABI).

    x: [..., D] float32 or bfloat16, contiguous, on a GPU.  Returns (codes,
    scales): codes uint8 [..., D] (OCP E4M3 bit patterns; view them as
    torch.float8_e4m3fn if wanted), scales float32 [...], one per row of D
    elements; a [T, H, D] Q or K gives the q / k and q_scale / k_scale
    arguments of mha_fwd's FP8_E4M3 path.
    """
    if x.device.type != "cuda":
        raise ValueError("x must be on a GPU device")
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("x must be float32 or bfloat16")
    if x.dim() < 1 or not x.is_contiguous():
        raise ValueError("x must be contiguous with at least one dimension")
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    c = codes if codes is not None else torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    s = scales if scales is not None else torch.empty(x.shape[:-1], dtype=torch.float32,
                                                      device=x.device)
    _need(c, "codes", x.device, torch.uint8, tuple(x.shape))
    _need(s, "scales", x.device, torch.float32, tuple(x.shape[:-1]))
    code = nat.MHA_DTYPE_BF16 if x.dtype == torch.bfloat16 else nat.MHA_DTYPE_F32
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        st = nat.load().mha_quantize_fp8(_ptr(x), code, int(rows), int(D), _ptr(c), _ptr(s),
                                         stream)
    nat.check(st)
    return c, s


def mha_combine_splits(o_partial: torch.Tensor, lse_partial: torch.Tensor, *,
                       out_dtype: torch.dtype = torch.bfloat16,
                       out: Optional[torch.Tensor] = None,
                       lse: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Log-sum-exp merge of partial results (mha_combine_splits of the C ABI).

    o_partial [n, T, H, Dv] and lse_partial [n, H, T] float32 on a GPU;
    returns o [T, H, Dv] (out_dtype: bfloat16 or float32) and lse [H, T].
    """
    if o_partial.dim() != 4 or lse_partial.dim() != 3:
        raise ValueError("o_partial must be [n, T, H, Dv] and lse_partial [n, H, T]")
    n, T, H, Dv = o_partial.shape
    dev = o_partial.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("out_dtype must be bfloat16 or float32")
    _need(o_partial, "o_partial", dev, torch.float32)
    _need(lse_partial, "lse_partial", dev, torch.float32, (n, H, T))
    o = out if out is not None else torch.empty((T, H, Dv), dtype=out_dtype, device=dev)
    _need(o, "out", dev, out_dtype, (T, H, Dv))
    lse_t = lse if lse is not None else torch.empty((H, T), dtype=torch.float32, device=dev)
    _need(lse_t, "lse", dev, torch.float32, (H, T))
    code = nat.MHA_DTYPE_BF16 if out_dtype == torch.bfloat16 else nat.MHA_DTYPE_F32
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        st = nat.load().mha_combine_splits(_ptr(o_partial), _ptr(lse_partial), int(n), int(T),
                                           int(H), int(Dv), code, _ptr(o), _ptr(lse_t), stream)
    nat.check(st)
    return o, lse_t


def mha_fwd_auto_splits(batch: int, max_seqlen: int, num_heads: int, causal: bool, v_dim: int,
                        cus: int) -> int:
    """Key splits mha_fwd chooses for a bf16 / fp8 problem on `cus` compute
    units (host arithmetic, no device call)."""
    return int(nat.load().mha_fwd_auto_splits(int(batch), int(max_seqlen), int(num_heads),
                                              int(bool(causal)), int(v_dim), int(cus)))
