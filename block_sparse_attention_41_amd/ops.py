"""ctypes binding over libs2a.so, with the same names as the C ABI (include/s2a.h).

Argument marshalling only: every step runs in the library's HIP kernels.  Tensors are
torch tensors on the GPU (bfloat16 for Q/K/V/O and their gradients, float32 for LSE and
summaries, int32 for chunk indices); this module checks dtype, device, shape and
contiguity, allocates outputs with torch when they are not given, passes raw pointers
and the current HIP stream, and raises on any non-zero status.  There is no fallback:
if the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libs2a.so")

_lib = None
_lock = threading.Lock()

_P = ctypes.c_void_p
_I = ctypes.c_int
_LL = ctypes.c_longlong
_F = ctypes.c_float
_SZ = ctypes.c_size_t

_SIGNATURES = {
    "s2a_status_string": (ctypes.c_char_p, [_I]),
    "s2attn_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _P]),
    "s2attn_bwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "s2attn_bwd_workspace_bytes_dsq": (_SZ, [_I, _I, _I, _I, _I, _I]),
    "s2attn_bwd": (_I, [_P] * 9 + [_P, _SZ] + [_I] * 7 + [_F, _P]),
    "s2attn_bwd_prep": (_I, [_P, _P, _P, _P, _SZ] + [_I] * 7 + [_F, _P]),
    "s2attn_bwd_dq": (_I, [_P] * 6 + [_SZ] + [_I] * 7 + [_F, _P]),
    "s2attn_bwd_dq_prep": (_I, [_P] * 8 + [_SZ] + [_I] * 7 + [_F, _P]),
    "s2attn_bwd_dkdv": (_I, [_P] * 7 + [_SZ] + [_I] * 7 + [_F, _P]),
    "s2attn_bwd_noalloc": (_I, [_P] * 9 + [_I] * 7 + [_F, _P]),
    "hga_summarize": (_I, [_P, _LL, _P, _LL, _I, _I, _I, _I, _I, _P]),
    "hga_append_history": (_I, [_P, _P, _LL, _P, _P, _LL, _P, _LL] + [_I] * 6 + [_P]),
    "hga_select_topk": (_I, [_P, _P, _LL, _P] + [_I] * 8 + [_P]),
    "hga_fwd": (_I, [_P, _P, _P, _LL, _P, _P, _LL, _P, _P, _P] + [_I] * 9 + [_F, _P]),
    "hga_bwd_workspace_bytes": (_SZ, [_I, _I, _I, _I, _I]),
    "hga_bwd_workspace_bytes_dsq": (_SZ, [_I, _I, _I, _I, _I]),
    "hga_bwd_active": (_I, [_P, _P, _P, _LL, _P, _P, _LL, _P, _P, _P, _P, _P, _P, _P, _P, _SZ]
                       + [_I] * 9 + [_F, _P]),
}
_SIGNATURES["hga_decode_workspace_bytes"] = (ctypes.c_size_t, [_I] * 7)
_SIGNATURES["hga_decode"] = (_I, [_P, _P, _P, _LL, _P, _P, _LL, _P, _P, _P, _P, _SZ] + [_I] * 9 + [_F, _P])
# the variants with one chunk list per kv head take the same arguments
for _name in ("hga_select_topk", "hga_fwd", "hga_bwd_active"):
    _SIGNATURES[_name + "_shared"] = _SIGNATURES[_name]
_SIGNATURES["hga_fwd_select_shared"] = (_I, [_P, _P, _P, _LL, _P, _P, _LL, _P, _LL, _P, _P, _P] + [_I] * 9 + [_F, _P])
_SIGNATURES["hga_detach_segment"] = _SIGNATURES["hga_append_history"]
_SIGNATURES["hga_stage_selected"] = (_I, [_P, _I, _I, _I, _P, _P, _LL, _I, _P, _P, _P, _P, _P, _LL] + [_I] * 5 + [_P])
_SIGNATURES["hga_stage_update"] = (_I, [_P, _I, _I, _I, _P, _P, _LL, _I, _P, _P, _P, _P, _P, _P, _P, _LL] + [_I] * 5
                                    + [_P])
EXPORTED = tuple(_SIGNATURES)


def lib() -> ctypes.CDLL:
    """Load libs2a.so once (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                                   "(there is no fallback path)")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in _SIGNATURES.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
    return _lib


class S2AError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        msg = lib().s2a_status_string(status).decode()
        super().__init__(f"{fn} failed with status {status} ({msg})")


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise S2AError(fn, status)


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _want(t: torch.Tensor, name: str, dtype, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _scale(d: int, scale):
    return float(d ** -0.5 if scale is None else scale)


# ------------------------------------------------------------------ S2-Attn -----------

def s2attn_fwd(q, k, v, G: int, shift: bool = True, scale=None, o=None, lse=None):
    """Shifted short attention forward -> (O [B,N,H,d] bf16, LSE [B,H,N] f32)."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if lse is None else lse
    st = lib().s2attn_fwd(_want(q, "q", torch.bfloat16), _want(k, "k", torch.bfloat16, (B, N, Hkv, d)),
                          _want(v, "v", torch.bfloat16, (B, N, Hkv, d)),
                          _want(o, "o", torch.bfloat16, (B, N, H, d)),
                          _want(lse, "lse", torch.float32, (B, H, N)),
                          B, N, H, Hkv, d, G, int(bool(shift)), _scale(d, scale), _stream())
    _check("s2attn_fwd", st)
    return o, lse


def s2attn_bwd_workspace_bytes(B, N, H, Hkv, d) -> int:
    return int(lib().s2attn_bwd_workspace_bytes(B, N, H, Hkv, d))


def s2attn_bwd_workspace_bytes_dsq(B, N, H, Hkv, d, G) -> int:
    return int(lib().s2attn_bwd_workspace_bytes_dsq(B, N, H, Hkv, d, G))


def s2attn_bwd(q, k, v, o, lse, do, G: int, shift: bool = True, scale=None, workspace=None,
               dq=None, dk=None, dv=None):
    """Shifted short attention backward -> (dQ, dK, dV), all bf16.  Without a workspace
    one of s2attn_bwd_workspace_bytes_dsq bytes is allocated (dQ from stored dS)."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    nbytes = s2attn_bwd_workspace_bytes_dsq(B, N, H, Hkv, d, G)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = lib().s2attn_bwd(_want(q, "q", torch.bfloat16), _want(k, "k", torch.bfloat16, (B, N, Hkv, d)),
                          _want(v, "v", torch.bfloat16, (B, N, Hkv, d)),
                          _want(o, "o", torch.bfloat16, (B, N, H, d)),
                          _want(lse, "lse", torch.float32, (B, H, N)),
                          _want(do, "do", torch.bfloat16, (B, N, H, d)),
                          _want(dq, "dq", torch.bfloat16, (B, N, H, d)),
                          _want(dk, "dk", torch.bfloat16, (B, N, Hkv, d)),
                          _want(dv, "dv", torch.bfloat16, (B, N, Hkv, d)),
                          _want(workspace, "workspace", torch.uint8), workspace.numel(),
                          B, N, H, Hkv, d, G, int(bool(shift)), _scale(d, scale), _stream())
    _check("s2attn_bwd", st)
    return dq, dk, dv


def s2attn_bwd_noalloc(q, k, v, o, lse, do, G: int, shift: bool = True, scale=None, dq=None, dk=None, dv=None):
    """s2attn_bwd with the row statistics in the library's static device array (no
    workspace).  Outputs not given are allocated here; the library call allocates
    nothing.  Calls that may overlap on one GPU race on that array."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    st = lib().s2attn_bwd_noalloc(_want(q, "q", torch.bfloat16), _want(k, "k", torch.bfloat16, (B, N, Hkv, d)),
                                  _want(v, "v", torch.bfloat16, (B, N, Hkv, d)),
                                  _want(o, "o", torch.bfloat16, (B, N, H, d)),
                                  _want(lse, "lse", torch.float32, (B, H, N)),
                                  _want(do, "do", torch.bfloat16, (B, N, H, d)),
                                  _want(dq, "dq", torch.bfloat16, (B, N, H, d)),
                                  _want(dk, "dk", torch.bfloat16, (B, N, Hkv, d)),
                                  _want(dv, "dv", torch.bfloat16, (B, N, Hkv, d)),
                                  B, N, H, Hkv, d, G, int(bool(shift)), _scale(d, scale), _stream())
    _check("s2attn_bwd_noalloc", st)
    return dq, dk, dv


def s2attn_bwd_stage(stage, q, k, v, o, lse, do, G: int, shift: bool = True, scale=None, workspace=None,
                     dq=None, dk=None, dv=None):
    """Run one backward stage ("prep", "dq", "dq_prep" or "dkdv") on the current stream.

    dq and dkdv read the statistics that prep (or dq_prep, which also computes dQ) wrote
    to the same workspace; outputs must be preallocated."""
    B, N, H, d = q.shape
    Hkv = k.shape[2]
    sc = _scale(d, scale)
    ws = _want(workspace, "workspace", torch.uint8)
    nb = workspace.numel()
    if stage == "prep":
        st = lib().s2attn_bwd_prep(_want(o, "o", torch.bfloat16, (B, N, H, d)), _want(lse, "lse", torch.float32, (B, H, N)),
                                   _want(do, "do", torch.bfloat16, (B, N, H, d)), ws, nb, B, N, H, Hkv, d, G,
                                   int(bool(shift)), sc, _stream())
    elif stage == "dq":
        st = lib().s2attn_bwd_dq(_want(q, "q", torch.bfloat16), _want(k, "k", torch.bfloat16, (B, N, Hkv, d)),
                                 _want(v, "v", torch.bfloat16, (B, N, Hkv, d)), _want(do, "do", torch.bfloat16, (B, N, H, d)),
                                 _want(dq, "dq", torch.bfloat16, (B, N, H, d)), ws, nb, B, N, H, Hkv, d, G,
                                 int(bool(shift)), sc, _stream())
    elif stage == "dq_prep":
        st = lib().s2attn_bwd_dq_prep(_want(q, "q", torch.bfloat16), _want(k, "k", torch.bfloat16, (B, N, Hkv, d)),
                                      _want(v, "v", torch.bfloat16, (B, N, Hkv, d)),
                                      _want(o, "o", torch.bfloat16, (B, N, H, d)),
                                      _want(lse, "lse", torch.float32, (B, H, N)),
                                      _want(do, "do", torch.bfloat16, (B, N, H, d)),
                                      _want(dq, "dq", torch.bfloat16, (B, N, H, d)), ws, nb, B, N, H, Hkv, d, G,
                                      int(bool(shift)), sc, _stream())
    elif stage == "dkdv":
        st = lib().s2attn_bwd_dkdv(_want(q, "q", torch.bfloat16), _want(k, "k", torch.bfloat16, (B, N, Hkv, d)),
                                   _want(v, "v", torch.bfloat16, (B, N, Hkv, d)),
                                   _want(do, "do", torch.bfloat16, (B, N, H, d)),
                                   _want(dk, "dk", torch.bfloat16, (B, N, Hkv, d)),
                                   _want(dv, "dv", torch.bfloat16, (B, N, Hkv, d)), ws, nb, B, N, H, Hkv, d, G,
                                   int(bool(shift)), sc, _stream())
    else:
        raise ValueError(stage)
    _check(f"s2attn_bwd_{stage}", st)


# ------------------------------------------------------------------ HGA ---------------

def _bstride(t: torch.Tensor) -> int:
    return t.stride(0)


def _want_rows(t, name, B, L, heads, d):
    """bf16 [B, L, heads, d] whose rows are contiguous (batch stride may be larger)."""
    if not t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bf16 GPU tensor")
    if tuple(t.shape) != (B, L, heads, d):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, L, heads, d)}")
    if L and (t.stride(3) != 1 or t.stride(2) != d or t.stride(1) != heads * d):
        raise ValueError(f"{name} rows must be contiguous")
    return t.data_ptr()


def hga_summarize(k_hist, chunk: int = 128, summ=None):
    """Per-chunk mean keys of the history -> summaries [B, T/chunk, Hkv, d] float32.

    ``summ`` may be a view whose rows are contiguous (e.g. a slice of a larger buffer)."""
    B, T, Hkv, d = k_hist.shape
    C = T // chunk
    if summ is None:
        summ = torch.empty((B, C, Hkv, d), dtype=torch.float32, device=k_hist.device)
    if summ.dtype != torch.float32 or tuple(summ.shape) != (B, C, Hkv, d) or \
            (C and (summ.stride(3) != 1 or summ.stride(2) != d or summ.stride(1) != Hkv * d)):
        raise ValueError("summ must be float32 [B, T/chunk, Hkv, d] with contiguous rows")
    st = lib().hga_summarize(_want_rows(k_hist, "k_hist", B, T, Hkv, d), _bstride(k_hist),
                             summ.data_ptr(), summ.stride(0), B, T, Hkv, d, chunk, _stream())
    _check("hga_summarize", st)
    return summ


def hga_append_history(k_seg, v_seg, k_hist, v_hist, summ, T: int, chunk: int = 128):
    """Detach a finished segment into the history: copy ``k_seg``/``v_seg`` [B, S, Hkv, d]
    to history rows [T, T + S) of ``k_hist``/``v_hist`` [B, >= T + S, Hkv, d] and write the
    summaries of its S/chunk chunks into ``summ`` [B, >= (T + S)/chunk, Hkv, d] float32."""
    B, S, Hkv, d = k_seg.shape
    L = k_hist.shape[1]
    if T + S > L or tuple(v_hist.shape) != tuple(k_hist.shape) or v_hist.stride() != k_hist.stride():
        raise ValueError("history buffers must match and hold T + S tokens")
    if tuple(v_seg.stride()) != tuple(k_seg.stride()):
        raise ValueError("k_seg and v_seg must share a layout")
    C = summ.shape[1]
    if summ.dtype != torch.float32 or (summ.shape[0], summ.shape[2], summ.shape[3]) != (B, Hkv, d) or \
            C * chunk < T + S or (C and (summ.stride(3) != 1 or summ.stride(2) != d or summ.stride(1) != Hkv * d)):
        raise ValueError("summ must be float32 [B, >= (T+S)/chunk, Hkv, d] with contiguous rows")
    st = lib().hga_append_history(_want_rows(k_seg, "k_seg", B, S, Hkv, d), _want_rows(v_seg, "v_seg", B, S, Hkv, d),
                                  _bstride(k_seg), _want_rows(k_hist, "k_hist", B, L, Hkv, d),
                                  _want_rows(v_hist, "v_hist", B, L, Hkv, d), _bstride(k_hist), summ.data_ptr(),
                                  summ.stride(0), B, S, Hkv, d, T, chunk, _stream())
    _check("hga_append_history", st)


# ------------------------------------------------------------- host-tier history ------

def pinned_empty(shape, dtype=torch.bfloat16):
    """A new tensor in pinned host memory (torch allocates it with hipHostMalloc), e.g. a
    host-tier history [B, L, Hkv, d]."""
    return torch.empty(shape, dtype=dtype, pin_memory=True)


def _want_host_rows(t, name, B, L, heads, d):
    """bf16 [B, L, heads, d] in pinned host memory whose rows are contiguous."""
    if not isinstance(t, torch.Tensor) or t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be a bf16 tensor in pinned host memory")
    if tuple(t.shape) != (B, L, heads, d):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(B, L, heads, d)}")
    if L == 0:
        return None                       # an empty history is never read
    if not t.is_pinned():
        raise TypeError(f"{name} must be a bf16 tensor in pinned host memory")
    if t.stride(3) != 1 or t.stride(2) != d or t.stride(1) != heads * d:
        raise ValueError(f"{name} rows must be contiguous")
    return t.data_ptr()


def hga_detach_segment(k_seg, v_seg, k_host, v_host, summ, T: int, chunk: int = 128):
    """hga_append_history into a host-tier history: ``k_host``/``v_host`` [B, >= T + S, Hkv, d]
    pinned host tensors receive rows [T, T + S); the summaries go to ``summ`` (device)."""
    B, S, Hkv, d = k_seg.shape
    L = k_host.shape[1]
    if T + S > L or tuple(v_host.shape) != tuple(k_host.shape) or v_host.stride() != k_host.stride():
        raise ValueError("host history buffers must match and hold T + S tokens")
    if tuple(v_seg.stride()) != tuple(k_seg.stride()):
        raise ValueError("k_seg and v_seg must share a layout")
    C = summ.shape[1]
    if summ.dtype != torch.float32 or not summ.is_cuda or (summ.shape[0], summ.shape[2], summ.shape[3]) != (B, Hkv, d) \
            or C * chunk < T + S or (C and (summ.stride(3) != 1 or summ.stride(2) != d or summ.stride(1) != Hkv * d)):
        raise ValueError("summ must be float32 [B, >= (T+S)/chunk, Hkv, d] on the GPU with contiguous rows")
    st = lib().hga_detach_segment(_want_rows(k_seg, "k_seg", B, S, Hkv, d), _want_rows(v_seg, "v_seg", B, S, Hkv, d),
                                  _bstride(k_seg), _want_host_rows(k_host, "k_host", B, L, Hkv, d),
                                  _want_host_rows(v_host, "v_host", B, L, Hkv, d), _bstride(k_host), summ.data_ptr(),
                                  summ.stride(0), B, S, Hkv, d, T, chunk, _stream())
    _check("hga_detach_segment", st)


def hga_stage_slots(lists: int, Hkv: int, nqb: int, topk: int, C: int) -> int:
    """Staging capacity (chunks per kv head) that any lists of this shape fit in: the most
    chunks one kv head's lists can name (at least 1)."""
    return max(1, min(C, (lists // Hkv) * nqb * topk))


def hga_stage_selected(idx, k_host, v_host, T: int, chunk: int = 128, max_slots=None, k_stage=None, v_stage=None,
                       idx_staged=None, chunk_of=None, count=None):
    """Gather the history chunks that ``idx`` [B, lists, nqb, topk] names from the host-tier
    history (``k_host``/``v_host`` pinned [B, >= T, Hkv, d]) into a device staging history.

    Returns (k_stage, v_stage, idx_staged, chunk_of, count) with k_stage/v_stage
    [B, max_slots * chunk, Hkv, d]: the attention entry points called with these (and
    T = max_slots * chunk) give the results of the call on the full history with idx."""
    B, lists, nqb, topk = idx.shape
    L, Hkv, d = k_host.shape[1], k_host.shape[2], k_host.shape[3]
    if T > L or tuple(v_host.shape) != tuple(k_host.shape) or v_host.stride() != k_host.stride():
        raise ValueError("host history buffers must match and hold T tokens")
    C = T // chunk
    max_slots = hga_stage_slots(lists, Hkv, nqb, topk, C) if max_slots is None else int(max_slots)
    dev = idx.device
    rows = max_slots * chunk
    k_stage = torch.empty((B, rows, Hkv, d), dtype=torch.bfloat16, device=dev) if k_stage is None else k_stage
    v_stage = torch.empty((B, rows, Hkv, d), dtype=torch.bfloat16, device=dev) if v_stage is None else v_stage
    if tuple(v_stage.stride()) != tuple(k_stage.stride()):
        raise ValueError("k_stage and v_stage must share a layout")
    idx_staged = torch.empty_like(idx) if idx_staged is None else idx_staged
    chunk_of = torch.empty((B, Hkv, max_slots), dtype=torch.int32, device=dev) if chunk_of is None else chunk_of
    count = torch.empty((B, Hkv), dtype=torch.int32, device=dev) if count is None else count
    st = lib().hga_stage_selected(
        _want(idx, "idx", torch.int32), lists, nqb, topk, _want_host_rows(k_host, "k_host", B, L, Hkv, d),
        _want_host_rows(v_host, "v_host", B, L, Hkv, d), _bstride(k_host), T,
        _want(chunk_of, "chunk_of", torch.int32, (B, Hkv, max_slots)), _want(count, "count", torch.int32, (B, Hkv)),
        _want(idx_staged, "idx_staged", torch.int32, tuple(idx.shape)),
        _want_rows(k_stage, "k_stage", B, rows, Hkv, d), _want_rows(v_stage, "v_stage", B, rows, Hkv, d),
        _bstride(k_stage), max_slots, B, Hkv, d, chunk, _stream())
    _check("hga_stage_selected", st)
    return k_stage, v_stage, idx_staged, chunk_of, count


def hga_stage_update(idx, k_host, v_host, T: int, chunk: int, chunk_of, k_stage, v_stage, idx_staged=None,
                     count=None, copied=None, copy_list=None):
    """Cached staging: like hga_stage_selected, but ``chunk_of`` [B, Hkv, max_slots] int32
    holds the chunk each slot of ``k_stage``/``v_stage`` already has (-1 = free; all -1 for
    new buffers) and is updated; only chunks the staging does not hold are copied from
    host memory.  Returns (idx_staged, count, copied)."""
    B, lists, nqb, topk = idx.shape
    L, Hkv, d = k_host.shape[1], k_host.shape[2], k_host.shape[3]
    if T > L or tuple(v_host.shape) != tuple(k_host.shape) or v_host.stride() != k_host.stride():
        raise ValueError("host history buffers must match and hold T tokens")
    max_slots = chunk_of.shape[-1]
    rows = max_slots * chunk
    dev = idx.device
    if tuple(v_stage.stride()) != tuple(k_stage.stride()):
        raise ValueError("k_stage and v_stage must share a layout")
    idx_staged = torch.empty_like(idx) if idx_staged is None else idx_staged
    count = torch.empty((B, Hkv), dtype=torch.int32, device=dev) if count is None else count
    copied = torch.empty((B, Hkv), dtype=torch.int32, device=dev) if copied is None else copied
    copy_list = torch.empty((B, Hkv, max_slots), dtype=torch.int32, device=dev) if copy_list is None else copy_list
    st = lib().hga_stage_update(
        _want(idx, "idx", torch.int32), lists, nqb, topk, _want_host_rows(k_host, "k_host", B, L, Hkv, d),
        _want_host_rows(v_host, "v_host", B, L, Hkv, d), _bstride(k_host), T,
        _want(chunk_of, "chunk_of", torch.int32, (B, Hkv, max_slots)), _want(count, "count", torch.int32, (B, Hkv)),
        _want(copied, "copied", torch.int32, (B, Hkv)),
        _want(copy_list, "copy_list", torch.int32, (B, Hkv, max_slots)),
        _want(idx_staged, "idx_staged", torch.int32, tuple(idx.shape)),
        _want_rows(k_stage, "k_stage", B, rows, Hkv, d), _want_rows(v_stage, "v_stage", B, rows, Hkv, d),
        _bstride(k_stage), max_slots, B, Hkv, d, chunk, _stream())
    _check("hga_stage_update", st)
    return idx_staged, count, copied


def _select(fn, q, summ, qblock, topk, idx, lists):
    B, S, H, d = q.shape
    if summ.dim() != 4 or summ.shape[0] != B or summ.shape[3] != d:
        raise ValueError(f"summ has shape {tuple(summ.shape)}, expected ({B}, C, Hkv, {d})")
    C, Hkv = summ.shape[1], summ.shape[2]
    # the kernel reads summary (b, c, j) at b * stride(0) + (c * Hkv + j) * d
    if summ.dtype != torch.float32 or (C and (summ.stride(3) != 1 or summ.stride(2) != d
                                              or summ.stride(1) != Hkv * d)):
        raise ValueError("summ must be float32 [B, C, Hkv, d] with contiguous rows")
    if B > 1 and C and summ.stride(0) < C * Hkv * d:
        raise ValueError("summ batches overlap")
    heads = Hkv if lists == "kv" else H
    if idx is None:
        idx = torch.empty((B, heads, S // qblock, topk), dtype=torch.int32, device=q.device)
    st = getattr(lib(), fn)(_want(q, "q", torch.bfloat16), summ.data_ptr(), summ.stride(0),
                            _want(idx, "idx", torch.int32, (B, heads, S // qblock, topk)),
                            B, S, H, Hkv, d, C, qblock, topk, _stream())
    _check(fn, st)
    return idx


def hga_select_topk(q, summ, qblock: int = 64, topk: int = 8, idx=None):
    """Top-k history chunks per (batch, q head, query block) -> idx int32 [B,H,S/qblock,topk]."""
    return _select("hga_select_topk", q, summ, qblock, topk, idx, "q")


def hga_select_topk_shared(q, summ, qblock: int = 64, topk: int = 8, idx=None):
    """Top-k history chunks per (batch, kv head, query block), scored with the summed block
    means of the kv head's q heads -> idx int32 [B,Hkv,S/qblock,topk]."""
    return _select("hga_select_topk_shared", q, summ, qblock, topk, idx, "kv")


def _fwd(fn, q, k_act, v_act, k_hist, v_hist, idx, chunk, qblock, scale, o, lse):
    B, S, H, d = q.shape
    Hkv = k_act.shape[2]
    T = k_hist.shape[1]
    topk = idx.shape[-1]
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse is None else lse
    st = getattr(lib(), fn)(_want(q, "q", torch.bfloat16), _want_rows(k_act, "k_act", B, S, Hkv, d),
                            _want_rows(v_act, "v_act", B, S, Hkv, d), _bstride(k_act),
                            _want_rows(k_hist, "k_hist", B, T, Hkv, d) if T else None,
                            _want_rows(v_hist, "v_hist", B, T, Hkv, d) if T else None, _bstride(k_hist),
                            _want(idx, "idx", torch.int32, (B, Hkv if fn.endswith("_shared") else H, S // qblock, topk)),
                            _want(o, "o", torch.bfloat16, (B, S, H, d)), _want(lse, "lse", torch.float32, (B, H, S)),
                            B, S, H, Hkv, d, T, chunk, qblock, topk, _scale(d, scale), _stream())
    _check(fn, st)
    return o, lse


def hga_fwd(q, k_act, v_act, k_hist, v_hist, idx, chunk: int = 128, qblock: int = 64, scale=None,
            o=None, lse=None):
    """HGA forward -> (O [B,S,H,d] bf16, LSE [B,H,S] f32); idx [B,H,S/qblock,topk]."""
    return _fwd("hga_fwd", q, k_act, v_act, k_hist, v_hist, idx, chunk, qblock, scale, o, lse)


def hga_fwd_shared(q, k_act, v_act, k_hist, v_hist, idx, chunk: int = 128, qblock: int = 64, scale=None,
                   o=None, lse=None):
    """HGA forward with chunk lists per kv head, idx [B,Hkv,S/qblock,topk]."""
    return _fwd("hga_fwd_shared", q, k_act, v_act, k_hist, v_hist, idx, chunk, qblock, scale, o, lse)


def hga_fwd_select_shared(q, k_act, v_act, k_hist, v_hist, summ, chunk: int = 128, qblock: int = 64, topk: int = 8,
                          scale=None, idx=None, o=None, lse=None):
    """HGA forward that chooses its own chunk lists (one per kv head and query block, as
    hga_select_topk_shared) in the same launch -> (O, LSE, idx [B,Hkv,S/qblock,topk])."""
    B, S, H, d = q.shape
    Hkv = k_act.shape[2]
    T = k_hist.shape[1]
    C = T // chunk
    if summ.dim() != 4 or tuple(summ.shape) != (B, C, Hkv, d) or summ.dtype != torch.float32 or \
            (C and (summ.stride(3) != 1 or summ.stride(2) != d or summ.stride(1) != Hkv * d)):
        raise ValueError(f"summ must be float32 [{B}, {C}, {Hkv}, {d}] with contiguous rows")
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device) if lse is None else lse
    idx = torch.empty((B, Hkv, S // qblock, topk), dtype=torch.int32, device=q.device) if idx is None else idx
    st = lib().hga_fwd_select_shared(
        _want(q, "q", torch.bfloat16), _want_rows(k_act, "k_act", B, S, Hkv, d),
        _want_rows(v_act, "v_act", B, S, Hkv, d), _bstride(k_act),
        _want_rows(k_hist, "k_hist", B, T, Hkv, d) if T else None,
        _want_rows(v_hist, "v_hist", B, T, Hkv, d) if T else None, _bstride(k_hist),
        summ.data_ptr() if C else None, summ.stride(0),
        _want(idx, "idx", torch.int32, (B, Hkv, S // qblock, topk)),
        _want(o, "o", torch.bfloat16, (B, S, H, d)), _want(lse, "lse", torch.float32, (B, H, S)),
        B, S, H, Hkv, d, T, chunk, qblock, topk, _scale(d, scale), _stream())
    _check("hga_fwd_select_shared", st)
    return o, lse, idx


def hga_bwd_workspace_bytes(B, S, H, Hkv, d) -> int:
    return int(lib().hga_bwd_workspace_bytes(B, S, H, Hkv, d))


def hga_bwd_workspace_bytes_dsq(B, S, H, Hkv, d) -> int:
    return int(lib().hga_bwd_workspace_bytes_dsq(B, S, H, Hkv, d))


def _bwd(fn, q, k_act, v_act, k_hist, v_hist, idx, o, lse, do, chunk, qblock, scale, workspace, dq, dk_act,
         dv_act):
    B, S, H, d = q.shape
    Hkv = k_act.shape[2]
    T = k_hist.shape[1]
    topk = idx.shape[-1]
    dq = torch.empty_like(q) if dq is None else dq
    dk_act = torch.empty((B, S, Hkv, d), dtype=torch.bfloat16, device=q.device) if dk_act is None else dk_act
    dv_act = torch.empty((B, S, Hkv, d), dtype=torch.bfloat16, device=q.device) if dv_act is None else dv_act
    nbytes = hga_bwd_workspace_bytes_dsq(B, S, H, Hkv, d)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = getattr(lib(), fn)(
        _want(q, "q", torch.bfloat16), _want_rows(k_act, "k_act", B, S, Hkv, d),
        _want_rows(v_act, "v_act", B, S, Hkv, d), _bstride(k_act),
        _want_rows(k_hist, "k_hist", B, T, Hkv, d) if T else None,
        _want_rows(v_hist, "v_hist", B, T, Hkv, d) if T else None, _bstride(k_hist),
        _want(idx, "idx", torch.int32, (B, Hkv if fn.endswith("_shared") else H, S // qblock, topk)),
        _want(o, "o", torch.bfloat16, (B, S, H, d)), _want(lse, "lse", torch.float32, (B, H, S)),
        _want(do, "do", torch.bfloat16, (B, S, H, d)),
        _want(dq, "dq", torch.bfloat16, (B, S, H, d)), _want(dk_act, "dk_act", torch.bfloat16, (B, S, Hkv, d)),
        _want(dv_act, "dv_act", torch.bfloat16, (B, S, Hkv, d)),
        _want(workspace, "workspace", torch.uint8), workspace.numel(),
        B, S, H, Hkv, d, T, chunk, qblock, topk, _scale(d, scale), _stream())
    _check(fn, st)
    return dq, dk_act, dv_act


def hga_bwd_active(q, k_act, v_act, k_hist, v_hist, idx, o, lse, do, chunk: int = 128, qblock: int = 64,
                   scale=None, workspace=None, dq=None, dk_act=None, dv_act=None):
    """HGA backward to the active segment -> (dQ, dK_act, dV_act) bf16; idx [B,H,S/qblock,topk].
    Without a workspace, one of hga_bwd_workspace_bytes_dsq bytes is allocated (the local
    part of dQ from stored dS)."""
    return _bwd("hga_bwd_active", q, k_act, v_act, k_hist, v_hist, idx, o, lse, do, chunk, qblock, scale,
                workspace, dq, dk_act, dv_act)


def hga_bwd_active_shared(q, k_act, v_act, k_hist, v_hist, idx, o, lse, do, chunk: int = 128, qblock: int = 64,
                          scale=None, workspace=None, dq=None, dk_act=None, dv_act=None):
    """HGA backward with chunk lists per kv head, idx [B,Hkv,S/qblock,topk]."""
    return _bwd("hga_bwd_active_shared", q, k_act, v_act, k_hist, v_hist, idx, o, lse, do, chunk, qblock, scale,
                workspace, dq, dk_act, dv_act)


def hga_decode_workspace_bytes(B, nq, Sa, H, d, chunk=128, topk=8) -> int:
    return int(lib().hga_decode_workspace_bytes(B, nq, Sa, H, d, chunk, topk))


def hga_decode(q, k_act, v_act, k_hist, v_hist, idx, chunk: int = 128, scale=None, workspace=None, o=None,
               lse=None):
    """Generation step: q [B,nq,H,d] are the last nq tokens of the active segment k_act/v_act
    [B,Sa,Hkv,d]; idx [B,H,topk] lists their block's history chunks -> (O [B,nq,H,d] bf16,
    LSE [B,H,nq] f32)."""
    B, nq, H, d = q.shape
    Sa, Hkv = k_act.shape[1], k_act.shape[2]
    T = k_hist.shape[1]
    topk = idx.shape[-1]
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, H, nq), dtype=torch.float32, device=q.device) if lse is None else lse
    nbytes = hga_decode_workspace_bytes(B, nq, Sa, H, d, chunk, topk)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    st = lib().hga_decode(
        _want(q, "q", torch.bfloat16), _want_rows(k_act, "k_act", B, Sa, Hkv, d),
        _want_rows(v_act, "v_act", B, Sa, Hkv, d), _bstride(k_act),
        _want_rows(k_hist, "k_hist", B, T, Hkv, d) if T else None,
        _want_rows(v_hist, "v_hist", B, T, Hkv, d) if T else None, _bstride(k_hist),
        _want(idx, "idx", torch.int32, (B, H, topk)),
        _want(o, "o", torch.bfloat16, (B, nq, H, d)), _want(lse, "lse", torch.float32, (B, H, nq)),
        _want(workspace, "workspace", torch.uint8), workspace.numel(),
        B, nq, Sa, H, Hkv, d, T, chunk, topk, _scale(d, scale), _stream())
    _check("hga_decode", st)
    return o, lse

