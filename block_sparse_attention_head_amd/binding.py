"""ctypes binding of libsparstar.so (include/sparstar.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the path runs in the library's kernels.
There is no fallback: if the library is missing the calls raise.
"""
import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libsparstar.so")

OK, ERR_INVALID_ARGUMENT, ERR_UNSUPPORTED, ERR_HIP = 0, 1, 2, 3
FP32, BF16 = 0, 1
BLOCK = 128
FUSED_MAX_NKB = 2048   # sparstar_select_blocks_from_means holds a row of screened scores in registers

_i64, _f32, _f64, _vp = ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p
_SIGNATURES = {
    "sparstar_block_means": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64, _vp, _vp]),
    "sparstar_block_scores": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _vp, _vp]),
    "sparstar_select_blocks": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _i64, _f64, _vp, _vp, _i64, _vp]),
    "sparstar_select_blocks_from_means": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _i64,
                                                         _f64, _vp, _vp, _i64, _vp, _i64, _vp]),
    "sparstar_select_workspace_bytes": (_i64, [_i64, _i64, _i64, _i64]),
    "sparstar_select_blocks_from_qk": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                      _i64, _f32, _i64, _f64, _vp, _vp, _vp, _vp, _i64,
                                                      _vp, _i64, _vp]),
    "sparstar_select_blocks_from_means_noalloc": (ctypes.c_int, [_vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32,
                                                                 _i64, _f64, _vp, _vp, _i64, _vp]),
    "sparstar_block_sparse_attn_fwd": (ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64,
                                                      _i64, _i64, _vp, _vp, _i64, _f32, _vp, _vp, _vp]),
    "sparstar_retained_mass": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp]),
    "sparstar_token_topk_bound": (ctypes.c_int, [_vp, _vp, ctypes.c_int, _i64, _i64, _i64, _i64, _i64,
                                                 _i64, _i64, _i64, _f32, _vp, _vp]),
    "sparstar_transfer_scores": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _i64,
                                                _i64, _vp, _vp]),
    "sparstar_forced_blocks": (_i64, [_i64, _i64]),
    "sparstar_kept_blocks": (_i64, [_i64, _i64, _f64]),
    "sparstar_last_error": (ctypes.c_char_p, []),
    "sparstar_version": (ctypes.c_int32, []),
}

_lib = None


class SparstarError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"status {status}: {message}")
        self.status = status


def lib():
    """Load libsparstar.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m block_sparse_attention_head_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


def last_error() -> str:
    return lib().sparstar_last_error().decode()


def version() -> int:
    return lib().sparstar_version()


def forced_blocks(n_forced_tokens: int, block: int = BLOCK) -> int:
    return lib().sparstar_forced_blocks(n_forced_tokens, block)


def kept_blocks(nkb: int, n_forced_blocks: int, density: float) -> int:
    return lib().sparstar_kept_blocks(nkb, n_forced_blocks, density)


def _check(status):
    if status != OK:
        raise SparstarError(status, last_error())


# --------------------------------------------------------------------------
# torch-facing wrappers (device memory and stream plumbing only)
# --------------------------------------------------------------------------
def _torch():
    import torch
    return torch


def _stream(stream=None):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _expect(t, name, shape, dtype):
    """Shape and dtype of a caller-supplied tensor, checked before any call:
    the library reads and writes through raw pointers at these strides."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _selection_buffers(lead, n_forced_blocks, density, nkb, max_kept, kv_count, kv_index, device):
    """kv_count [*lead] and kv_index [*lead, max_kept] int32; max_kept defaults
    to the width of a supplied kv_index, else to the kept-block count."""
    torch = _torch()
    if max_kept is None:
        if kv_index is not None:
            max_kept = kv_index.shape[-1]
        else:
            max_kept = kept_blocks(nkb, n_forced_blocks, density)
            if max_kept < 0:
                raise SparstarError(ERR_INVALID_ARGUMENT, "invalid n_forced_blocks or density")
    if kv_index is None:
        # at least one column, and the library writes all of them (-1 padding)
        max_kept = max(1, max_kept)
    if kv_count is None:
        kv_count = torch.empty(lead, dtype=torch.int32, device=device)
    if kv_index is None:
        kv_index = torch.empty((*lead, max_kept), dtype=torch.int32, device=device)
    _expect(kv_count, "kv_count", lead, torch.int32)
    _expect(kv_index, "kv_index", (*lead, max_kept), torch.int32)
    return max_kept, kv_count, kv_index


def block_means(x, block=BLOCK, out=None, stream=None):
    """x [B,H,N,D] bf16/fp32 -> [B,H,ceil(N/block),D] fp32."""
    torch = _torch()
    B, H, N, D = x.shape
    nb = -(-N // block)
    if out is None:
        out = torch.empty((B, H, nb, D), dtype=torch.float32, device=x.device)
    _expect(out, "out", (B, H, nb, D), torch.float32)
    _check(lib().sparstar_block_means(_dev(x, "x"), _dtype_code(x), B, H, N, D, block,
                                      _dev(out, "out"), _stream(stream)))
    return out


def block_scores(qbar, kbar, tau=None, out=None, stream=None):
    """S [B,H,nqb,nkb] fp32 = tau * qbar kbar^T (tau = D^-1/2 by default)."""
    torch = _torch()
    B, H, nqb, D = qbar.shape
    nkb = kbar.shape[2]
    if tau is None:
        tau = 1.0 / math.sqrt(D)
    _expect(qbar, "qbar", (B, H, nqb, D), torch.float32)
    _expect(kbar, "kbar", (B, H, nkb, D), torch.float32)
    if out is None:
        out = torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=qbar.device)
    _expect(out, "S", (B, H, nqb, nkb), torch.float32)
    _check(lib().sparstar_block_scores(_dev(qbar, "qbar"), _dev(kbar, "kbar"), B, H, nqb, nkb, D,
                                       tau, _dev(out, "S"), _stream(stream)))
    return out


def select_blocks(S, n_forced_blocks, density, max_kept=None, kv_count=None, kv_index=None,
                  stream=None):
    """-> (kv_count [B,H,nqb] int32, kv_index [B,H,nqb,max_kept] int32)."""
    torch = _torch()
    B, H, nqb, nkb = S.shape
    _expect(S, "S", S.shape, torch.float32)
    max_kept, kv_count, kv_index = _selection_buffers((B, H, nqb), n_forced_blocks, density, nkb,
                                                      max_kept, kv_count, kv_index, S.device)
    _check(lib().sparstar_select_blocks(_dev(S, "S"), B, H, nqb, nkb, n_forced_blocks, density,
                                        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"),
                                        max_kept, _stream(stream)))
    return kv_count, kv_index


def select_workspace_bytes(B, H, nqb, nkb) -> int:
    return lib().sparstar_select_workspace_bytes(B, H, nqb, nkb)


def select_workspace(B, H, nqb, nkb, device):
    """A workspace for select_blocks_from_means (uint8, 256-byte aligned)."""
    torch = _torch()
    n = select_workspace_bytes(B, H, nqb, nkb)
    if n < 0:
        raise SparstarError(ERR_UNSUPPORTED, f"no screened route for nkb={nkb}")
    return torch.empty(max(1, n), dtype=torch.uint8, device=device)


def select_blocks_from_means(qbar, kbar, n_forced_blocks, density, tau=None, max_kept=None,
                             kv_count=None, kv_index=None, workspace=None, stream=None):
    """Scores and selection without S in float32 (screened scores in a
    workspace, exact scores for the few blocks that decide a row);
    nkb <= FUSED_MAX_NKB.  The selection equals select_blocks(block_scores(...))."""
    torch = _torch()
    B, H, nqb, D = qbar.shape
    nkb = kbar.shape[2]
    _expect(qbar, "qbar", (B, H, nqb, D), torch.float32)
    _expect(kbar, "kbar", (B, H, nkb, D), torch.float32)
    if tau is None:
        tau = 1.0 / math.sqrt(D)
    max_kept, kv_count, kv_index = _selection_buffers((B, H, nqb), n_forced_blocks, density, nkb,
                                                      max_kept, kv_count, kv_index, qbar.device)
    if workspace is None:
        workspace = select_workspace(B, H, nqb, nkb, qbar.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    _check(lib().sparstar_select_blocks_from_means(
        _dev(qbar, "qbar"), _dev(kbar, "kbar"), B, H, nqb, nkb, D, tau, n_forced_blocks, density,
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"), max_kept,
        _dev(workspace, "workspace"), workspace.numel(), _stream(stream)))
    return kv_count, kv_index


def select_blocks_from_qk(q, k, n_forced_blocks, density, block=BLOCK, tau=None, max_kept=None,
                          qbar=None, kbar=None, kv_count=None, kv_index=None, workspace=None,
                          stream=None):
    """The whole selection stage from q [B,H,Nq,D] and k [B,H,Nk,D] (same
    dtype) in one library call: block means of both, then
    select_blocks_from_means on them.  Returns (kv_count, kv_index, qbar, kbar)."""
    torch = _torch()
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    _expect(k, "k", (B, H, Nk, D), q.dtype)
    nqb, nkb = -(-Nq // block), -(-Nk // block)
    if qbar is None:
        qbar = torch.empty((B, H, nqb, D), dtype=torch.float32, device=q.device)
    if kbar is None:
        kbar = torch.empty((B, H, nkb, D), dtype=torch.float32, device=q.device)
    _expect(qbar, "qbar", (B, H, nqb, D), torch.float32)
    _expect(kbar, "kbar", (B, H, nkb, D), torch.float32)
    if tau is None:
        tau = 1.0 / math.sqrt(D)
    max_kept, kv_count, kv_index = _selection_buffers((B, H, nqb), n_forced_blocks, density, nkb,
                                                      max_kept, kv_count, kv_index, q.device)
    if workspace is None:
        workspace = select_workspace(B, H, nqb, nkb, q.device)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1:
        raise TypeError("workspace must be a 1-D uint8 tensor")
    _check(lib().sparstar_select_blocks_from_qk(
        _dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, Nq, Nk, D, block, tau, n_forced_blocks,
        density, _dev(qbar, "qbar"), _dev(kbar, "kbar"), _dev(kv_count, "kv_count"),
        _dev(kv_index, "kv_index"), max_kept, _dev(workspace, "workspace"), workspace.numel(),
        _stream(stream)))
    return kv_count, kv_index, qbar, kbar


def select_blocks_from_means_noalloc(qbar, kbar, n_forced_blocks, density, tau=None,
                                     max_kept=None, kv_count=None, kv_index=None, stream=None):
    """select_blocks_from_means without a workspace: the library's own device
    scratch (64 MiB per GPU) stands in for it, so the call itself allocates
    nothing (pass kv_count and kv_index to keep it that way).  Calls that
    overlap in time on one GPU race on that scratch."""
    torch = _torch()
    B, H, nqb, D = qbar.shape
    nkb = kbar.shape[2]
    _expect(qbar, "qbar", (B, H, nqb, D), torch.float32)
    _expect(kbar, "kbar", (B, H, nkb, D), torch.float32)
    if tau is None:
        tau = 1.0 / math.sqrt(D)
    max_kept, kv_count, kv_index = _selection_buffers((B, H, nqb), n_forced_blocks, density, nkb,
                                                      max_kept, kv_count, kv_index, qbar.device)
    _check(lib().sparstar_select_blocks_from_means_noalloc(
        _dev(qbar, "qbar"), _dev(kbar, "kbar"), B, H, nqb, nkb, D, tau, n_forced_blocks, density,
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"), max_kept, _stream(stream)))
    return kv_count, kv_index


def block_sparse_attn_fwd(q, k, v, kv_count, kv_index, scale=None, block=BLOCK, out=None,
                          lse=None, return_lse=True, stream=None):
    """O [B,H,Nq,D] (dtype of q) and LSE [B,H,Nq] fp32 over the listed key blocks."""
    torch = _torch()
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    _dtype_code(q)
    _expect(k, "k", (B, H, Nk, D), q.dtype)
    _expect(v, "v", (B, H, Nk, D), q.dtype)
    nqb = -(-Nq // block)
    max_kept = kv_index.shape[-1]
    _expect(kv_count, "kv_count", (B, H, nqb), torch.int32)
    _expect(kv_index, "kv_index", (B, H, nqb, max_kept), torch.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _expect(out, "out", q.shape, q.dtype)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _expect(lse, "lse", (B, H, Nq), torch.float32)
    _check(lib().sparstar_block_sparse_attn_fwd(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dtype_code(q), B, H, Nq, Nk, D, block,
        _dev(kv_count, "kv_count"), _dev(kv_index, "kv_index"), max_kept, scale,
        _dev(out, "o"), _dev(lse, "lse") if lse is not None else None, _stream(stream)))
    return out, lse


def retained_mass(lse_sel, lse_dense, out=None, stream=None):
    """exp(lse_sel - lse_dense) per query token (0 where either is -inf)."""
    torch = _torch()
    if out is None:
        out = torch.empty_like(lse_sel)
    _check(lib().sparstar_retained_mass(_dev(lse_sel, "lse_sel"), _dev(lse_dense, "lse_dense"),
                                        lse_sel.numel(), _dev(out, "mass"), _stream(stream)))
    return out


def token_topk_bound(q, k, n_forced_blocks, k_blocks, block=BLOCK, scale=None, out=None,
                     stream=None):
    """Token-wise Top-K upper bound of the retained mass per query token
    [B,H,Nq] at the budget of n_forced_blocks forced + k_blocks ranked blocks."""
    torch = _torch()
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    _check(lib().sparstar_token_topk_bound(_dev(q, "q"), _dev(k, "k"), _dtype_code(q), B, H, Nq, Nk, D,
                                           block, n_forced_blocks, k_blocks, scale, _dev(out, "bound"),
                                           _stream(stream)))
    return out


def transfer_scores(S_src, src_geom, dst_geom, block=BLOCK, out=None, stream=None):
    """Scores of a source scale carried to a target scale (mask reuse).

    src_geom, dst_geom: (n_text, n_ref, n_cur) token counts of the two scales;
    S_src [B,H,ceil(src n_cur/block),ceil(src total/block)] fp32 ->
    S_dst [B,H,ceil(dst n_cur/block),ceil(dst total/block)] fp32."""
    torch = _torch()
    B, H = S_src.shape[:2]
    nqb = -(-int(dst_geom[2]) // block)
    nkb = -(-sum(int(x) for x in dst_geom) // block)
    if out is None:
        out = torch.empty((B, H, nqb, nkb), dtype=torch.float32, device=S_src.device)
    _check(lib().sparstar_transfer_scores(_dev(S_src, "S_src"), B, H, block, *[int(x) for x in src_geom],
                                          *[int(x) for x in dst_geom], _dev(out, "S_dst"),
                                          _stream(stream)))
    return out


def transferred_selection(S_src, src_geom, dst_geom, n_forced_blocks, density, block=BLOCK,
                          max_kept=None, stream=None):
    """The target scale's selection when the source scale's scores are reused:
    transfer_scores, then select_blocks under the target's forced set and budget."""
    S = transfer_scores(S_src, src_geom, dst_geom, block=block, stream=stream)
    return select_blocks(S, n_forced_blocks, density, max_kept=max_kept, stream=stream)


def selection_retained_mass(q, k, v, kv_count, kv_index, block=BLOCK, stream=None):
    """Retained attention mass of a selection, per query token [B,H,Nq]: the
    attention LSE over the listed blocks against the LSE over every block
    (listed by the selector at n_forced_blocks = 0, density = 1)."""
    _, lse_sel = block_sparse_attn_fwd(q, k, v, kv_count, kv_index, block=block, stream=stream)
    qbar = block_means(q, block, stream=stream)
    kbar = block_means(k, block, stream=stream)
    S = block_scores(qbar, kbar, stream=stream)
    d_cnt, d_idx = select_blocks(S, 0, 1.0, stream=stream)
    _, lse_dense = block_sparse_attn_fwd(q, k, v, d_cnt, d_idx, block=block, stream=stream)
    return retained_mass(lse_sel, lse_dense, stream=stream)


def sparse_attention(q, k, v, n_forced_tokens, density, block=BLOCK, return_all=False,
                     fused=False, stream=None):
    """The whole path for one scale: means -> scores -> selection -> attention.

    With ``fused`` (and nkb <= FUSED_MAX_NKB) the selection stage is one
    select_blocks_from_qk call (screened scores) and S is never materialised
    (``return_all`` then gives S = None).
    """
    F = forced_blocks(n_forced_tokens, block)
    if fused and -(-k.shape[2] // block) <= FUSED_MAX_NKB:
        S = None
        kv_count, kv_index, qbar, kbar = select_blocks_from_qk(q, k, F, density, block=block,
                                                               stream=stream)
    else:
        qbar = block_means(q, block, stream=stream)
        kbar = block_means(k, block, stream=stream)
        S = block_scores(qbar, kbar, stream=stream)
        kv_count, kv_index = select_blocks(S, F, density, stream=stream)
    o, lse = block_sparse_attn_fwd(q, k, v, kv_count, kv_index, block=block, stream=stream)
    if return_all:
        return {"qbar": qbar, "kbar": kbar, "S": S, "kv_count": kv_count,
                "kv_index": kv_index, "o": o, "lse": lse}
    return o
