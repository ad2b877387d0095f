"""Python binding of libfa.so, the gfx950 exact-attention library.

The C entry points are exposed under their own names (``fa_fwd``, ``fa_bwd``,
``fa_decode_splitkv``, ...) and take torch tensors (or raw integer device
addresses) for pointer arguments.  A few convenience wrappers (``forward``,
``backward``, ``decode``, ``quantize_fp8``, ``forward_fp8``) allocate outputs
with torch and call those entry points.  This module only marshals arguments:
all of the attention arithmetic runs in the library's HIP kernels, and nothing
here falls back to another implementation.  If libfa.so has not been built,
``load()`` raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE, FA_ERR_HIP = range(5)

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_Z = ctypes.c_size_t

# name -> (restype, argtypes), mirroring include/fa.h
_SIGS = {
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_version": (_I, []),
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_f32": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_size": (_Z, [_I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                    _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_pre": (_I, [_P, _P, _P, _Z, _I, _I, _I, _I, _P]),
    "fa_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z,
                         _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _P, _Z,
                       _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dq_delta": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _Z,
                             _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_f32": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                        _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_decode_splitkv_q": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P]),
    "fa_decode_splitkv_paged_q": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                                       _I, _I, _I, _F, _I, _I, _P]),
    "fa_decode_splitkv_paged": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                     _I, _F, _I, _P]),
    "fa_fwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _I, _F, _I,
                           _P]),
    "fa_bwd_block_sparse_workspace_size": (_Z, [_I, _I, _I, _I, _I]),
    "fa_bwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                                 _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I, _P]),
    "fa_bwd_varlen": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _P, _P,
                           _I, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_window": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_bwd_window": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                           _I, _I, _I, _I, _I, _I, _F, _I, _I, _I, _P]),
    "fa_fwd_block_sparse": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P, _P, _I,
                                 _P]),
    "fa_decode_combine": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_decode_workspace_size": (_Z, [_I, _I, _I, _I]),
    "fa_decode_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_quantize_fp8": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_fwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P,
                        _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_quantize_pow2_e4m3": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_bwd_fp8_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "fa_bwd_fp8": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _Z,
                        _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_schedule": (_I, [_I, _I, _I, _I, _I, _I, _P, _P, _P, _I]),
    "fa_persistent_schedule": (_I, [_I, _I, _P, _I]),
}

_lib = None


def load():
    """Load libfa.so (built in-tree by ``exact_attention_83_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m exact_attention_83_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class FAError(RuntimeError):
    def __init__(self, name, code):
        msg = load().fa_status_string(code).decode()
        super().__init__(f"{name}: {msg}")
        self.code = code


class FAArgumentError(FAError, ValueError):
    pass


def _check(name, code):
    if code != FA_OK:
        if code in (FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_WORKSPACE):
            raise FAArgumentError(name, code)
        raise FAError(name, code)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _call(name, *args):
    code = getattr(load(), name)(*args)
    _check(name, code)


# ------------------------------------------------------------------ raw C ABI

def fa_fwd(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream=None):
    _call("fa_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
          scale, int(causal), _stream(stream))


def fa_fwd_f32(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, stream=None):
    _call("fa_fwd_f32", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
          scale, int(causal), _stream(stream))


def fa_bwd_workspace_size(B, Hq, Nq, d):
    return load().fa_bwd_workspace_size(B, Hq, Nq, d)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
           B, Hq, Hkv, Nq, Nk, d, scale, causal, stream=None):
    _call("fa_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale,
          int(causal), _stream(stream))


def fa_bwd_pre(o, dout, workspace, workspace_bytes, B, Hq, Nq, d, stream=None):
    _call("fa_bwd_pre", _ptr(o), _ptr(dout), _ptr(workspace), workspace_bytes, B, Hq, Nq, d,
          _stream(stream))


def fa_bwd_dkdv(q, k, v, dout, lse, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
                scale, causal, stream=None):
    _call("fa_bwd_dkdv", _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dk), _ptr(dv),
          _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
          _stream(stream))


def fa_bwd_dq(q, k, v, dout, lse, dq, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale,
              causal, stream=None):
    _call("fa_bwd_dq", _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
          _stream(stream))


def fa_bwd_dq_delta(q, k, v, o, dout, lse, dq, workspace, workspace_bytes, B, Hq, Hkv, Nq, Nk,
                    d, scale, causal, stream=None):
    _call("fa_bwd_dq_delta", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
          _stream(stream))


def fa_bwd_f32(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
               B, Hq, Hkv, Nq, Nk, d, scale, causal, stream=None):
    _call("fa_bwd_f32", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale,
          int(causal), _stream(stream))


def fa_decode_workspace_size(B, Hq, d, num_splits):
    return load().fa_decode_workspace_size(B, Hq, d, num_splits)


def fa_decode_splitkv(q, k, v, o_part, lse_part, B, Hq, Hkv, Nk, d, scale, num_splits,
                      stream=None):
    _call("fa_decode_splitkv", _ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, Hq,
          Hkv, Nk, d, scale, num_splits, _stream(stream))


def fa_decode_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Nk, d, scale, num_splits,
                              stream=None):
    _call("fa_decode_splitkv_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
          Hkv, Nk, d, scale, num_splits, _stream(stream))


def fa_decode_splitkv_q(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                        num_splits, stream=None):
    _call("fa_decode_splitkv_q", _ptr(q), _ptr(k), _ptr(v), _ptr(o_part), _ptr(lse_part), B, Hq,
          Hkv, Nq, Nk, d, scale, int(causal), num_splits, _stream(stream))


def fa_decode_splitkv_paged(q, k_cache, v_cache, block_table, seqlens, o_part, lse_part, B, Hq,
                            Hkv, num_pages, page_size, max_pages, max_seqlen, d, scale,
                            num_splits, stream=None):
    _call("fa_decode_splitkv_paged", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
          _ptr(seqlens), _ptr(o_part), _ptr(lse_part), B, Hq, Hkv, num_pages, page_size,
          max_pages, max_seqlen, d, scale, num_splits, _stream(stream))


def fa_decode_splitkv_paged_q(q, k_cache, v_cache, block_table, seqlens, o_part, lse_part, B, Hq,
                              Hkv, Nq, num_pages, page_size, max_pages, max_seqlen, d, scale,
                              causal, num_splits, stream=None):
    _call("fa_decode_splitkv_paged_q", _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
          _ptr(seqlens), _ptr(o_part), _ptr(lse_part), B, Hq, Hkv, Nq, num_pages, page_size,
          max_pages, max_seqlen, d, scale, int(causal), num_splits, _stream(stream))


def fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, batch, Hq, Hkv, total_q, total_k, max_seqlen_q,
                  max_seqlen_k, d, scale, causal, stream=None):
    _call("fa_fwd_varlen", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(cu_q), _ptr(cu_k),
          batch, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, scale, int(causal),
          _stream(stream))


def fa_bwd_block_sparse_workspace_size(B, Hq, Nq, Nk, d):
    return load().fa_bwd_block_sparse_workspace_size(B, Hq, Nq, Nk, d)


def fa_bwd_block_sparse(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                        Nq, Nk, d, scale, causal, q_tile_ptr, kv_block_idx, max_blocks_per_tile,
                        stream=None):
    _call("fa_bwd_block_sparse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse),
          _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d,
          scale, int(causal), _ptr(q_tile_ptr), _ptr(kv_block_idx), max_blocks_per_tile,
          _stream(stream))


def fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, cu_q, cu_k,
                  batch, Hq, Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, scale, causal,
                  stream=None):
    _call("fa_bwd_varlen", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, _ptr(cu_q), _ptr(cu_k), batch, Hq,
          Hkv, total_q, total_k, max_seqlen_q, max_seqlen_k, d, scale, int(causal),
          _stream(stream))


def fa_fwd_window(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, window_left,
                  window_right, stream=None):
    _call("fa_fwd_window", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d,
          scale, int(causal), window_left, window_right, _stream(stream))


def fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv, Nq,
                  Nk, d, scale, causal, window_left, window_right, stream=None):
    _call("fa_bwd_window", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale,
          int(causal), window_left, window_right, _stream(stream))


def fa_fwd_block_sparse(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, q_tile_ptr,
                        kv_block_idx, max_blocks_per_tile, stream=None):
    _call("fa_fwd_block_sparse", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk,
          d, scale, int(causal), _ptr(q_tile_ptr), _ptr(kv_block_idx), max_blocks_per_tile,
          _stream(stream))


def fa_decode_combine(o_part, lse_part, o, lse, B, Hq, d, num_splits, stream=None):
    _call("fa_decode_combine", _ptr(o_part), _ptr(lse_part), _ptr(o), _ptr(lse), B, Hq, d,
          num_splits, _stream(stream))


def fa_quantize_fp8(x, signs, x8, scales, B, H, N, d, stream=None):
    _call("fa_quantize_fp8", _ptr(x), _ptr(signs), _ptr(x8), _ptr(scales), B, H, N, d,
          _stream(stream))


def fa_fwd_fp8(q8, k8, v8, q_scale, k_scale, v_scale, o, lse, B, Hq, Hkv, Nq, Nk, d, scale,
               causal, stream=None):
    _call("fa_fwd_fp8", _ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale), _ptr(k_scale),
          _ptr(v_scale), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq, Nk, d, scale, int(causal),
          _stream(stream))


def fa_quantize_pow2_e4m3(x, x8, x_scale, B, H, N, d, stream=None):
    _call("fa_quantize_pow2_e4m3", _ptr(x), _ptr(x8), _ptr(x_scale), B, H, N, d, _stream(stream))


def fa_bwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nk, d):
    return load().fa_bwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nk, d)


def fa_bwd_fp8(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes,
               B, Hq, Hkv, Nq, Nk, d, scale, causal, stream=None):
    _call("fa_bwd_fp8", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
          _ptr(dk), _ptr(dv), _ptr(workspace), workspace_bytes, B, Hq, Hkv, Nq, Nk, d, scale,
          int(causal), _stream(stream))


def fa_fwd_schedule(B, Hq, Nq, Nk, d, causal):
    """Work order of the forward launch as three int lists (bh, q_tile, cost)."""
    lib = load()
    n = lib.fa_fwd_schedule(B, Hq, Nq, Nk, d, int(causal), None, None, None, 0)
    if n < 0:
        raise ValueError("fa_fwd_schedule: invalid arguments")
    arr = [(ctypes.c_int * n)() for _ in range(3)]
    n2 = lib.fa_fwd_schedule(B, Hq, Nq, Nk, d, int(causal), *[ctypes.addressof(a) for a in arr], n)
    assert n2 == n
    return [list(a) for a in arr]


def fa_persistent_schedule(n_units, grid):
    """Workgroup of a persistent grid that takes each position of the
    longest-first unit list (a list of n_units ints)."""
    lib = load()
    arr = (ctypes.c_int * max(n_units, 1))()
    n = lib.fa_persistent_schedule(n_units, grid, ctypes.addressof(arr), n_units)
    if n < 0:
        raise ValueError("fa_persistent_schedule: invalid arguments")
    return list(arr)[:n_units]


# ---------------------------------------------------------- torch conveniences

def _default_scale(d, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal=False, scale=None, out=None, lse=None, stream=None, window=None):
    """O, LSE for bf16 (or fp32) q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d].
    ``window`` = (left, right) selects the sliding-window entry point (bf16)."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device) if lse is None else lse
    if window is not None:
        fa_fwd_window(q, k, v, o, l, B, Hq, Hkv, Nq, Nk, d, s, causal, int(window[0]),
                      int(window[1]), stream)
        return o, l
    fn = fa_fwd_f32 if q.dtype == torch.float32 else fa_fwd
    fn(q, k, v, o, l, B, Hq, Hkv, Nq, Nk, d, s, causal, stream)
    return o, l


def backward(q, k, v, o, lse, dout, causal=False, scale=None, workspace=None, stream=None,
             window=None):
    """dQ, dK, dV for the forward above (same dtype as q; ``window`` as there)."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = fa_bwd_workspace_size(B, Hq, Nq, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    if window is not None:
        fa_bwd_window(q, k, v, o, dout, lse, dq, dk, dv, ws, ws.numel() * ws.element_size(), B,
                      Hq, Hkv, Nq, Nk, d, s, causal, int(window[0]), int(window[1]), stream)
        return dq, dk, dv
    fn = fa_bwd_f32 if q.dtype == torch.float32 else fa_bwd
    fn(q, k, v, o, dout, lse, dq, dk, dv, ws, ws.numel() * ws.element_size(), B, Hq, Hkv, Nq,
       Nk, d, s, causal, stream)
    return dq, dk, dv


def decode(q, k, v, num_splits, scale=None, stream=None, return_partials=False):
    """Split-KV decode: q [B][Hq][1][d], k/v [B][Hkv][Nk][d] -> (O, LSE)."""
    import torch
    B, Hq, _, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    rows = B * Hq * num_splits
    o_part = torch.empty((B, Hq, num_splits, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
    fa_decode_splitkv(q, k, v, o_part, lse_part, B, Hq, Hkv, Nk, d, s, num_splits, stream)
    fa_decode_combine(o_part, lse_part, o, lse, B, Hq, d, num_splits, stream)
    assert rows == o_part.shape[0] * o_part.shape[1] * o_part.shape[2]
    if return_partials:
        return o, lse, o_part, lse_part
    return o, lse


def decode_noalloc(q, k, v, num_splits, scale=None, stream=None, out=None, lse=None):
    """decode() through fa_decode_splitkv_noalloc: the library keeps the split
    partials in its own fixed device scratch.  Outputs are allocated here
    unless ``out`` / ``lse`` are given (then nothing is allocated)."""
    import torch
    B, Hq, _, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device) if lse is None else lse
    fa_decode_splitkv_noalloc(q, k, v, o, l, B, Hq, Hkv, Nk, d, s, num_splits, stream)
    return o, l


def decode_tokens(q, k, v, num_splits, causal=False, scale=None, stream=None,
                  return_partials=False):
    """Split-KV decode of a few query tokens: q [B][Hq][Nq][d] (the newest Nq
    positions), k/v [B][Hkv][Nk][d] -> (O [B][Hq][Nq][d], LSE [B][Hq][Nq])."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    o_part = torch.empty((B, Hq, Nq, num_splits, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, Nq, num_splits), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    fa_decode_splitkv_q(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, s, causal, num_splits,
                        stream)
    fa_decode_combine(o_part, lse_part, o, lse, B, Hq * Nq, d, num_splits, stream)
    if return_partials:
        return o, lse, o_part, lse_part
    return o, lse


def forward_varlen(q, k, v, cu_q, cu_k, max_seqlen_q, max_seqlen_k, causal=False, scale=None,
                   stream=None):
    """Packed variable-length forward: q [total_q][Hq][d], k/v [total_k][Hkv][d]
    (bf16, device), cu_q/cu_k int32 [batch+1] device offsets ->
    (O [total_q][Hq][d], LSE [Hq][total_q])."""
    import torch
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    s = _default_scale(d, scale)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, total_q), dtype=torch.float32, device=q.device)
    fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, cu_q.shape[0] - 1, Hq, Hkv, total_q, total_k,
                  int(max_seqlen_q), int(max_seqlen_k), d, s, causal, stream)
    return o, lse


def backward_varlen(q, k, v, o, lse, dout, cu_q, cu_k, max_seqlen_q, max_seqlen_k, causal=False,
                    scale=None, workspace=None, stream=None):
    """dQ, dK, dV of forward_varlen (packed token-major layouts as there)."""
    import torch
    total_q, Hq, d = q.shape
    total_k, Hkv = k.shape[0], k.shape[1]
    s = _default_scale(d, scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = fa_bwd_workspace_size(1, Hq, total_q, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    fa_bwd_varlen(q, k, v, o, dout, lse, dq, dk, dv, ws, ws.numel() * ws.element_size(), cu_q,
                  cu_k, cu_q.shape[0] - 1, Hq, Hkv, total_q, total_k, int(max_seqlen_q),
                  int(max_seqlen_k), d, s, causal, stream)
    return dq, dk, dv


SPARSE_BLOCK_Q = 256   # query rows per block of a block-sparse pattern
SPARSE_BLOCK_K = 64    # keys per block


def forward_block_sparse(q, k, v, q_tile_ptr, kv_block_idx, causal=False, scale=None,
                         max_blocks_per_tile=None, stream=None):
    """Block-sparse forward: q [B][Hq][Nq][d], k/v [B][Hkv][Nk][d] (bf16), one
    CSR pattern for every (b, head): query tile t (SPARSE_BLOCK_Q rows) sees
    the key blocks (SPARSE_BLOCK_K keys) kv_block_idx[q_tile_ptr[t] ..
    q_tile_ptr[t+1]-1] (int32 device tensors) -> (O, LSE)."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    if max_blocks_per_tile is None:
        max_blocks_per_tile = int((q_tile_ptr[1:] - q_tile_ptr[:-1]).max().item())
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_block_sparse(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, s, causal, q_tile_ptr,
                        kv_block_idx, max_blocks_per_tile, stream)
    return o, lse


def backward_block_sparse(q, k, v, o, lse, dout, q_tile_ptr, kv_block_idx, causal=False,
                          scale=None, max_blocks_per_tile=None, workspace=None, stream=None):
    """dQ, dK, dV of forward_block_sparse for the same inputs and pattern."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    if max_blocks_per_tile is None:
        max_blocks_per_tile = int((q_tile_ptr[1:] - q_tile_ptr[:-1]).max().item())
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = fa_bwd_block_sparse_workspace_size(B, Hq, Nq, Nk, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    fa_bwd_block_sparse(q, k, v, o, dout, lse, dq, dk, dv, ws, ws.numel() * ws.element_size(), B,
                        Hq, Hkv, Nq, Nk, d, s, causal, q_tile_ptr, kv_block_idx,
                        max_blocks_per_tile, stream)
    return dq, dk, dv


def decode_paged(q, k_cache, v_cache, block_table, seqlens, num_splits, max_seqlen=None,
                 scale=None, stream=None, return_partials=False):
    """Split-KV decode over a paged cache: q [B][Hq][1][d], k_cache/v_cache
    [num_pages][page_size][Hkv][d], block_table int32 [B][max_pages], seqlens
    int32 [B] (device tensors) -> (O, LSE).  ``max_seqlen`` defaults to the
    table's capacity (max_pages * page_size)."""
    import torch
    B, Hq, _, d = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    max_pages = block_table.shape[1]
    ms = max_pages * page_size if max_seqlen is None else int(max_seqlen)
    s = _default_scale(d, scale)
    o_part = torch.empty((B, Hq, num_splits, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, num_splits), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
    fa_decode_splitkv_paged(q, k_cache, v_cache, block_table, seqlens, o_part, lse_part, B, Hq,
                            Hkv, num_pages, page_size, max_pages, ms, d, s, num_splits, stream)
    fa_decode_combine(o_part, lse_part, o, lse, B, Hq, d, num_splits, stream)
    if return_partials:
        return o, lse, o_part, lse_part
    return o, lse


def decode_paged_tokens(q, k_cache, v_cache, block_table, seqlens, num_splits, causal=False,
                        max_seqlen=None, scale=None, stream=None):
    """decode_paged for a few query tokens per head: q [B][Hq][Nq][d] (the
    newest Nq positions of each entry) -> (O [B][Hq][Nq][d], LSE [B][Hq][Nq])."""
    import torch
    B, Hq, Nq, d = q.shape
    num_pages, page_size, Hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    max_pages = block_table.shape[1]
    ms = max_pages * page_size if max_seqlen is None else int(max_seqlen)
    s = _default_scale(d, scale)
    o_part = torch.empty((B, Hq, Nq, num_splits, d), dtype=torch.float32, device=q.device)
    lse_part = torch.empty((B, Hq, Nq, num_splits), dtype=torch.float32, device=q.device)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    fa_decode_splitkv_paged_q(q, k_cache, v_cache, block_table, seqlens, o_part, lse_part, B, Hq,
                              Hkv, Nq, num_pages, page_size, max_pages, ms, d, s, causal,
                              num_splits, stream)
    fa_decode_combine(o_part, lse_part, o, lse, B, Hq * Nq, d, num_splits, stream)
    return o, lse


def quantize_fp8(x, signs=None, stream=None):
    """e4m3 codes (uint8, same shape) and per-128-row-block fp32 scales."""
    import torch
    B, H, N, d = x.shape
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    sc = torch.empty((B, H, (N + 127) // 128), dtype=torch.float32, device=x.device)
    fa_quantize_fp8(x, signs, x8, sc, B, H, N, d, stream)
    return x8, sc


def quantize_pow2_e4m3(x, stream=None):
    """e4m3 codes (uint8, same shape) and per-32-row e8m0 scale bytes."""
    import torch
    B, H, N, d = x.shape
    x8 = torch.empty(x.shape, dtype=torch.uint8, device=x.device)
    xe = torch.empty((B, H, (N + 31) // 32), dtype=torch.uint8, device=x.device)
    fa_quantize_pow2_e4m3(x, x8, xe, B, H, N, d, stream)
    return x8, xe


def backward_fp8(q, k, v, o, lse, dout, causal=False, scale=None, workspace=None, stream=None):
    """dQ, dK, dV (bf16) with the fp8 dS product for dQ (fa_bwd_fp8)."""
    import torch
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    s = _default_scale(d, scale)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    ws_bytes = fa_bwd_fp8_workspace_size(B, Hq, Hkv, Nq, Nk, d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device) if workspace is None else workspace
    fa_bwd_fp8(q, k, v, o, dout, lse, dq, dk, dv, ws, ws.numel() * ws.element_size(), B, Hq, Hkv,
               Nq, Nk, d, s, causal, stream)
    return dq, dk, dv


def forward_fp8(q8, k8, v8, qs, ks, vs, causal=False, scale=None, stream=None):
    import torch
    B, Hq, Nq, d = q8.shape
    Hkv, Nk = k8.shape[1], k8.shape[2]
    s = _default_scale(d, scale)
    o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device)
    fa_fwd_fp8(q8, k8, v8, qs, ks, vs, o, lse, B, Hq, Hkv, Nq, Nk, d, s, causal, stream)
    return o, lse
