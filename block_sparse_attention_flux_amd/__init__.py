"""Layer-routed hybrid attention (Flux Attention) for MI355X / gfx950.

Thin Python binding over libflux.so: every function below only checks and
marshals arguments (torch tensors -> device pointers, the current HIP stream)
and calls the C entry point of the same name in include/flux.h.  All the
computation runs in the library's HIP kernels; there is no fallback path, and
importing this package fails if the library has not been built.

    route, logits = route(hidden, cu_seqlens, w1, b1, w2, b2)
    mask, row_ptr, col_idx = build_block_mask(max_seqlen, sa)
    out = attn_prefill(q, k, v, cu_seqlens, max_seqlen, route, layer, row_ptr, col_idx, sa)
    out = attn_decode(q, k_cache, v_cache, seqlens, route, layer, row_ptr, col_idx, sa, ws)
"""

import ctypes
import math
from dataclasses import dataclass

import torch

from . import _lib

_LIB = _lib.load()

__all__ = [
    "SAParams", "FluxError", "route", "route_workspace_size", "mask_blocks", "mask_nnz", "build_block_mask",
    "build_block_mask_dynamic",
    "attn_prefill", "attn_prefill_soft", "prefill_workspace", "decode_workspace_size", "decode_workspace", "attn_decode",
    "attn_decode_append", "attn_decode_noalloc", "status_str",
    "kv_rows", "kv_cache", "kv_store_prefill", "kv_append", "attn_decode_sa_compact",
    "probe_mfma", "probe_read",
]


@dataclass(frozen=True)
class SAParams:
    """Sparse Attention block pattern: ``sink_blocks`` sink blocks plus a
    causal window of ``local_blocks`` blocks (diagonal included), blocks of
    ``block_size`` tokens."""
    block_size: int = 128
    sink_blocks: int = 1
    local_blocks: int = 16

    def c(self):
        return _lib.SAParamsC(self.block_size, self.sink_blocks, self.local_blocks)


class FluxError(RuntimeError):
    """The HIP runtime reported an error inside libflux."""


def status_str(code):
    return _LIB.flux_status_str(int(code)).decode()


def _check(code, what):
    if code == _lib.FLUX_OK:
        return
    msg = f"{what}: {status_str(code)} (status {code})"
    if code == _lib.FLUX_ERR_HIP:
        raise FluxError(msg)
    raise ValueError(msg)


def _ptr(t, dtype=None, name="tensor", device=True):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if device and not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def route_workspace_size(n_req, d_in, h1):
    return int(_LIB.flux_route_workspace_size(n_req, d_in, h1))


def route(hidden, cu_seqlens, w1, b1, w2, b2, route_out=None, logits_out=None, workspace=None):
    """Layer Router (flux_route): returns (route uint8 [n_req][L], logits fp32 or None)."""
    if hidden.dtype == torch.bfloat16:
        dt = _lib.FLUX_BF16
    elif hidden.dtype == torch.float32:
        dt = _lib.FLUX_F32
    else:
        raise ValueError("hidden must be bfloat16 or float32")
    n_req = cu_seqlens.numel() - 1
    h1, d_in = w1.shape
    n_layers = w2.shape[0]
    if route_out is None:
        route_out = torch.empty((n_req, n_layers), dtype=torch.uint8, device=hidden.device)
    if workspace is None:
        workspace = torch.empty(max(route_workspace_size(n_req, d_in, h1), 1), dtype=torch.uint8,
                                device=hidden.device)
    code = _LIB.flux_route(
        _ptr(hidden, None, "hidden"), dt, _ptr(cu_seqlens, torch.int32, "cu_seqlens"), n_req, d_in,
        _ptr(w1, torch.float32, "w1"), _ptr(b1, torch.float32, "b1"), h1,
        _ptr(w2, torch.float32, "w2"), _ptr(b2, torch.float32, "b2"), n_layers,
        _ptr(route_out, torch.uint8, "route_out"), _ptr(logits_out, torch.float32, "logits_out"),
        _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(hidden.device))
    _check(code, "flux_route")
    return route_out, logits_out


def mask_blocks(seqlen, sa):
    n = _LIB.flux_mask_blocks(int(seqlen), sa.c())
    if n < 0:
        _check(int(n), "flux_mask_blocks")
    return int(n)


def mask_nnz(seqlen, sa):
    n = _LIB.flux_mask_nnz(int(seqlen), sa.c())
    if n < 0:
        _check(int(n), "flux_mask_nnz")
    return int(n)


def build_block_mask(seqlen, sa, device="cuda", dense=True):
    """SA block mask (flux_build_block_mask): (mask uint8 [nb][nb] or None,
    row_ptr int32 [nb+1], col_idx int32 [nnz])."""
    nb = mask_blocks(seqlen, sa)
    nnz = mask_nnz(seqlen, sa)
    mask = torch.empty((nb, nb), dtype=torch.uint8, device=device) if dense else None
    row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=device)
    col_idx = torch.empty(max(nnz, 1), dtype=torch.int32, device=device)
    code = _LIB.flux_build_block_mask(int(seqlen), sa.c(), _ptr(mask, torch.uint8, "mask"),
                                      _ptr(row_ptr), _ptr(col_idx), _stream(row_ptr.device))
    _check(code, "flux_build_block_mask")
    return mask, row_ptr, col_idx[:nnz]


def build_block_mask_dynamic(q, k, block_size, sink_blocks, tau, max_blocks=0, softmax_scale=None):
    """Content-aware SA block mask of one sequence (flux_build_block_mask_dynamic):
    (row_ptr int32 [nb+1], col_idx int32 [nb (nb+1) / 2]); the first
    row_ptr[nb] columns are the mask.  q [S][hq][d], k [S][hkv][d] bf16."""
    S, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (S, hkv, d):
        raise ValueError("k must be [S][hkv][head_dim] like q")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    nb = (S + int(block_size) - 1) // int(block_size)
    cap = nb * (nb + 1) // 2
    row_ptr = torch.empty(nb + 1, dtype=torch.int32, device=q.device)
    col_idx = torch.empty(cap, dtype=torch.int32, device=q.device)
    ws_bytes = int(_LIB.flux_dynamic_mask_workspace_size(S, hq, hkv, d, int(block_size)))
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=q.device)
    p = _lib.DynParamsC(int(block_size), int(sink_blocks), float(tau), int(max_blocks))
    code = _LIB.flux_build_block_mask_dynamic(
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), S, hq, hkv, d,
        float(softmax_scale), p, _ptr(row_ptr), _ptr(col_idx), cap, _ptr(ws), ws.numel(),
        _stream(q.device))
    _check(code, "flux_build_block_mask_dynamic")
    return row_ptr, col_idx


def _route_fn(route, hkv, layer_fn, head_fn, what):
    """route [n][L] -> one decision per layer; [n][L][hkv] -> one per kv head."""
    if route.dim() == 2:
        return layer_fn
    if route.dim() == 3 and route.shape[2] == hkv:
        return head_fn
    raise ValueError(f"{what}: route must be [n][n_layers] or [n][n_layers][hkv]")


_PREFILL_WS = {}


def prefill_workspace(device="cuda"):
    """The zero-filled FLUX_PREFILL_WORKSPACE_BYTES workspace of the device's
    current stream: made once per (device, stream) and reused, since every
    prefill call leaves it zero again.  Calls on one stream run one after
    another, so they never use it at the same time."""
    device = torch.device(device)
    if device.index is None:
        device = torch.device(device.type, torch.cuda.current_device())
    key = (device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _PREFILL_WS.get(key)
    if ws is None:
        ws = torch.zeros(_lib.FLUX_PREFILL_WORKSPACE_BYTES // 4, dtype=torch.int32, device=device)
        _PREFILL_WS[key] = ws
    return ws


def _prefill_ws_args(workspace, device):
    """(pointer, bytes) for workspace="auto" (the stream's own), None (the
    fixed work order) or a caller's zero-filled int32 tensor."""
    if workspace is None:
        return None, 0
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError('workspace must be "auto", None or a tensor')
        workspace = prefill_workspace(device)
    return _ptr(workspace, None, "workspace"), workspace.numel() * workspace.element_size()


def attn_prefill(q, k, v, cu_seqlens, max_seqlen, route, layer, row_ptr, col_idx, sa,
                 out=None, softmax_scale=None, workspace="auto"):
    """One routed attention layer over packed prompts (flux_attn_prefill, or
    flux_attn_prefill_heads for a per-kv-head route [n_req][n_layers][hkv]).
    workspace: "auto" (the stream's balancing workspace), None (the fixed
    work order) or a zero-filled int32 tensor of FLUX_PREFILL_WORKSPACE_BYTES;
    per-kv-head routes take none."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, d) or v.shape != (T, hkv, d):
        raise ValueError("k and v must be [T][hkv][head_dim] like q")
    fn = _route_fn(route, hkv, _LIB.flux_attn_prefill, _LIB.flux_attn_prefill_heads, "attn_prefill")
    if out is None:
        out = torch.empty_like(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    args = [
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"),
        _ptr(out, torch.bfloat16, "out"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        cu_seqlens.numel() - 1, int(max_seqlen), hq, hkv, d, float(softmax_scale),
        _ptr(route, torch.uint8, "route"), route.shape[1], int(layer),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"),
        row_ptr.numel() - 1, sa.c()]
    if fn is _LIB.flux_attn_prefill:
        args += list(_prefill_ws_args(workspace, q.device))
    code = fn(*args, _stream(q.device))
    _check(code, "flux_attn_prefill")
    return out


def attn_prefill_soft(q, k, v, cu_seqlens, max_seqlen, r_soft, layer, row_ptr, col_idx, sa,
                      out=None, softmax_scale=None, workspace="auto"):
    """Soft-routed forward r FA + (1 - r) SA of one layer (flux_attn_prefill_soft);
    r_soft float32 [n_req][n_layers]; workspace as for attn_prefill."""
    T, hq, d = q.shape
    hkv = k.shape[1]
    if k.shape != (T, hkv, d) or v.shape != (T, hkv, d):
        raise ValueError("k and v must be [T][hkv][head_dim] like q")
    if out is None:
        out = torch.empty_like(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    code = _LIB.flux_attn_prefill_soft(
        _ptr(q, torch.bfloat16, "q"), _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"),
        _ptr(out, torch.bfloat16, "out"), _ptr(cu_seqlens, torch.int32, "cu_seqlens"),
        cu_seqlens.numel() - 1, int(max_seqlen), hq, hkv, d, float(softmax_scale),
        _ptr(r_soft, torch.float32, "r_soft"), r_soft.shape[1], int(layer),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"),
        row_ptr.numel() - 1, sa.c(), *_prefill_ws_args(workspace, q.device), _stream(q.device))
    _check(code, "flux_attn_prefill_soft")
    return out


def decode_workspace_size(n_seq, hq, hkv, head_dim, max_len):
    return int(_LIB.flux_attn_decode_workspace_size(n_seq, hq, hkv, head_dim, max_len))


def decode_workspace(n_seq, hq, hkv, head_dim, max_len, device="cuda"):
    """A device buffer of flux_attn_decode_workspace_size bytes (its contents
    do not matter; torch's allocations are 16-byte aligned)."""
    return torch.empty(max(decode_workspace_size(n_seq, hq, hkv, head_dim, max_len), 16),
                       dtype=torch.uint8, device=device)


def attn_decode(q, k_cache, v_cache, seqlens, route, layer, row_ptr, col_idx, sa,
                workspace=None, out=None, softmax_scale=None):
    """One split-KV decode step of one layer (flux_attn_decode, or
    flux_attn_decode_heads for a per-kv-head route [n_seq][n_layers][hkv])."""
    n_seq, hq, d = q.shape
    _, hkv, max_len, _ = k_cache.shape
    if k_cache.shape != (n_seq, hkv, max_len, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [n_seq][hkv][max_len][head_dim]")
    fn = _route_fn(route, hkv, _LIB.flux_attn_decode, _LIB.flux_attn_decode_heads, "attn_decode")
    if out is None:
        out = torch.empty_like(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(n_seq, hq, hkv, d, max_len, q.device)
    code = fn(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(out, torch.bfloat16, "out"),
        _ptr(seqlens, torch.int32, "seqlens"), n_seq, max_len, hq, hkv, d, float(softmax_scale),
        _ptr(route, torch.uint8, "route"), route.shape[1], int(layer),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"),
        row_ptr.numel() - 1, sa.c(), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "flux_attn_decode")
    return out


def attn_decode_append(q, k_new, v_new, k_cache, v_cache, seqlens, route, layer, row_ptr, col_idx, sa,
                       workspace=None, out=None, softmax_scale=None):
    """One decode step of one layer with the new K/V row appended in the same
    launch (flux_attn_decode_append): k_new, v_new [n_seq][hkv][head_dim] go to
    position seqlens[b] - 1 of the full caches, which the step reads."""
    n_seq, hq, d = q.shape
    _, hkv, max_len, _ = k_cache.shape
    if k_cache.shape != (n_seq, hkv, max_len, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [n_seq][hkv][max_len][head_dim]")
    if k_new.shape != (n_seq, hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [n_seq][hkv][head_dim]")
    if route.dim() != 2:
        raise ValueError("attn_decode_append: route must be [n_seq][n_layers]")
    if out is None:
        out = torch.empty_like(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(n_seq, hq, hkv, d, max_len, q.device)
    code = _LIB.flux_attn_decode_append(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_new, torch.bfloat16, "k_new"),
        _ptr(v_new, torch.bfloat16, "v_new"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(out, torch.bfloat16, "out"),
        _ptr(seqlens, torch.int32, "seqlens"), n_seq, max_len, hq, hkv, d, float(softmax_scale),
        _ptr(route, torch.uint8, "route"), route.shape[1], int(layer),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"),
        row_ptr.numel() - 1, sa.c(), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "flux_attn_decode_append")
    return out


def attn_decode_noalloc(q, k_cache, v_cache, seqlens, route, layer, row_ptr, col_idx, sa,
                        out=None, softmax_scale=None):
    """flux_attn_decode_noalloc: attn_decode with the library's own device scratch
    in place of a workspace (nothing allocated by the library; ``out`` is still
    the caller's).  Calls that overlap in time on one GPU race on that scratch."""
    n_seq, hq, d = q.shape
    _, hkv, max_len, _ = k_cache.shape
    if k_cache.shape != (n_seq, hkv, max_len, d) or v_cache.shape != k_cache.shape:
        raise ValueError("caches must be [n_seq][hkv][max_len][head_dim]")
    if route.dim() != 2:
        raise ValueError("attn_decode_noalloc: route must be [n_seq][n_layers]")
    if out is None:
        out = torch.empty_like(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    code = _LIB.flux_attn_decode_noalloc(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(out, torch.bfloat16, "out"),
        _ptr(seqlens, torch.int32, "seqlens"), n_seq, max_len, hq, hkv, d, float(softmax_scale),
        _ptr(route, torch.uint8, "route"), route.shape[1], int(layer),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"),
        row_ptr.numel() - 1, sa.c(), _stream(q.device))
    _check(code, "flux_attn_decode_noalloc")
    return out


# ---------------------------------------------------------------- K/V caches


def kv_rows(max_len, sa, compact=False):
    """Rows per (sequence, kv head) of a full or compact cache (flux_kv_rows)."""
    n = _LIB.flux_kv_rows(int(max_len), sa.c(), int(bool(compact)))
    if n < 0:
        _check(int(n), "flux_kv_rows")
    return int(n)


def kv_cache(n_seq, hkv, head_dim, max_len, sa, compact=False, device="cuda"):
    """A zero-filled (K, V) cache pair [n_seq][hkv][rows][head_dim] bf16."""
    shape = (n_seq, hkv, kv_rows(max_len, sa, compact), head_dim)
    return (torch.zeros(shape, dtype=torch.bfloat16, device=device),
            torch.zeros(shape, dtype=torch.bfloat16, device=device))


def _cache_args(k_cache, v_cache, max_len, sa, compact):
    n_seq, hkv, rows, d = k_cache.shape
    if v_cache.shape != k_cache.shape:
        raise ValueError("k_cache and v_cache must have the same shape")
    if rows != kv_rows(max_len, sa, compact):
        raise ValueError(f"cache has {rows} rows per head, the layout needs {kv_rows(max_len, sa, compact)}")
    return n_seq, hkv, d


def kv_store_prefill(k, v, cu_seqlens, max_seqlen, k_cache, v_cache, max_len, sa, compact=False):
    """Prompts' K/V rows into decode caches (flux_kv_store_prefill)."""
    n_seq, hkv, d = _cache_args(k_cache, v_cache, max_len, sa, compact)
    if k.shape[1:] != (hkv, d) or v.shape != k.shape:
        raise ValueError("k and v must be [T][hkv][head_dim] like the caches")
    code = _LIB.flux_kv_store_prefill(
        _ptr(k, torch.bfloat16, "k"), _ptr(v, torch.bfloat16, "v"),
        _ptr(cu_seqlens, torch.int32, "cu_seqlens"), cu_seqlens.numel() - 1, int(max_seqlen), hkv, d,
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        int(max_len), int(bool(compact)), sa.c(), _stream(k.device))
    _check(code, "flux_kv_store_prefill")


def kv_append(k_new, v_new, seqlens, k_cache, v_cache, max_len, sa, compact=False):
    """One new row per sequence at position seqlens[b] - 1 (flux_kv_append)."""
    n_seq, hkv, d = _cache_args(k_cache, v_cache, max_len, sa, compact)
    if k_new.shape != (n_seq, hkv, d) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must be [n_seq][hkv][head_dim]")
    code = _LIB.flux_kv_append(
        _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
        _ptr(seqlens, torch.int32, "seqlens"), n_seq, hkv, d,
        _ptr(k_cache, torch.bfloat16, "k_cache"), _ptr(v_cache, torch.bfloat16, "v_cache"),
        int(max_len), int(bool(compact)), sa.c(), _stream(k_new.device))
    _check(code, "flux_kv_append")


def attn_decode_sa_compact(q, k_cache, v_cache, seqlens, max_len, row_ptr, col_idx, sa,
                           workspace=None, out=None, softmax_scale=None):
    """One SA decode step of one layer over compact caches (flux_attn_decode_sa_compact)."""
    n_seq, hq, d = q.shape
    _, hkv, _ = _cache_args(k_cache, v_cache, max_len, sa, True)
    if out is None:
        out = torch.empty_like(q)
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(n_seq, hq, hkv, d, max_len, q.device)
    code = _LIB.flux_attn_decode_sa_compact(
        _ptr(q, torch.bfloat16, "q"), _ptr(k_cache, torch.bfloat16, "k_cache"),
        _ptr(v_cache, torch.bfloat16, "v_cache"), _ptr(out, torch.bfloat16, "out"),
        _ptr(seqlens, torch.int32, "seqlens"), n_seq, int(max_len), hq, hkv, d, float(softmax_scale),
        _ptr(row_ptr, torch.int32, "row_ptr"), _ptr(col_idx, torch.int32, "col_idx"),
        row_ptr.numel() - 1, sa.c(), _ptr(workspace, None, "workspace"),
        workspace.numel() * workspace.element_size(), _stream(q.device))
    _check(code, "flux_attn_decode_sa_compact")
    return out


# ---------------------------------------------------------------- measurement probes


def probe_mfma(sink, n_workgroups, iters):
    """Dense bf16 MFMA loop (flux_probe_mfma); returns the launch's flops."""
    code = _LIB.flux_probe_mfma(_ptr(sink, torch.float32, "sink"), int(n_workgroups), int(iters),
                                _stream(sink.device))
    _check(code, "flux_probe_mfma")
    return float(_LIB.flux_probe_mfma_flops(int(n_workgroups), int(iters)))


def probe_read(src, sink):
    """Streaming read of every byte of src (flux_probe_read); one word per workgroup in sink."""
    code = _LIB.flux_probe_read(_ptr(src, None, "src"), src.numel() * src.element_size(),
                                _ptr(sink, torch.int32, "sink"), sink.numel(), _stream(src.device))
    _check(code, "flux_probe_read")
