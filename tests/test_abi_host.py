"""The C ABI library: it loads, exports what include/sparstar.h declares, and its
host-side logic (helpers, argument checks) behaves as documented.  No call here
reaches the GPU: every compute call below fails validation first."""
import ctypes
import os
import re
import subprocess

import pytest

import block_sparse_attention_head_amd as sp
from block_sparse_attention_head_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparstar.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparstar_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) == set(binding._SIGNATURES), names
    h = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (sparstar_\w+)", out))
    assert set(names) <= exported


def test_version_and_helpers():
    assert sp.version() == 10400
    assert sp.forced_blocks(0) == 0
    assert sp.forced_blocks(1) == 1
    assert sp.forced_blocks(128) == 1
    assert sp.forced_blocks(129) == 2
    assert sp.forced_blocks(512 + 3600) == 33
    assert sp.forced_blocks(-1) == -1
    assert sp.kept_blocks(16, 1, 0.25) == 5
    assert sp.kept_blocks(286, 4, 0.1875) == 57
    assert sp.kept_blocks(1129, 4, 0.09375) == 110
    assert sp.kept_blocks(595, 33, 0.09375) == 86
    assert sp.kept_blocks(129, 4, 0.625) == 83
    assert sp.kept_blocks(504, 4, 0.1875) == 98
    assert sp.kept_blocks(1129, 4, 1.0) == 1129
    assert sp.kept_blocks(10, 0, 0.0) == 0
    assert sp.kept_blocks(10, 11, 0.5) == -1
    assert sp.kept_blocks(10, 1, 1.5) == -1
    assert sp.kept_blocks(10, 1, float("nan")) == -1


def test_kept_blocks_matches_oracle_budget():
    import oracle
    for nkb in (1, 2, 7, 16, 129, 286, 504, 595, 1129):
        for F in sorted(f for f in {0, 1, 4, nkb // 3, nkb} if f <= nkb):
            for dens in (0.0, 0.09375, 0.1875, 0.625, 1.0, 0.1, 0.3, 0.7):
                assert sp.kept_blocks(nkb, F, dens) == oracle.kept_blocks(nkb, F, dens)


L = None


def _lib():
    return sp.lib()


NULL = ctypes.c_void_p(None)
FAKE = ctypes.c_void_p(4096)     # aligned, never dereferenced: validation fails first


def _err(status, code, needle):
    assert status == code, (status, sp.last_error())
    assert needle in sp.last_error(), sp.last_error()


def test_means_validation():
    f = _lib().sparstar_block_means
    _err(f(NULL, 1, 1, 1, 128, 128, 128, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(f(FAKE, 1, 1, 1, 128, 96, 128, FAKE, NULL), sp.ERR_UNSUPPORTED, "D must be")
    _err(f(FAKE, 1, 1, 1, 128, 128, 96, FAKE, NULL), sp.ERR_UNSUPPORTED, "block")
    _err(f(FAKE, 1, 1, 1, 128, 128, 16, FAKE, NULL), sp.ERR_UNSUPPORTED, "block")
    _err(f(FAKE, 1, 0, 1, 128, 128, 128, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "B and H")
    _err(f(FAKE, 1, 1, 1, 0, 128, 128, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "sequence")
    _err(f(FAKE, 7, 1, 1, 128, 128, 128, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "dtype")
    _err(f(ctypes.c_void_p(4098), 1, 1, 1, 128, 128, 128, FAKE, NULL), sp.ERR_INVALID_ARGUMENT,
         "aligned")


def test_scores_validation():
    f = _lib().sparstar_block_scores
    _err(f(FAKE, NULL, 1, 1, 4, 4, 128, 0.1, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(f(FAKE, FAKE, 1, 1, 0, 4, 128, 0.1, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "nqb")
    _err(f(FAKE, FAKE, 1, 1, 4, 4, 32, 0.1, FAKE, NULL), sp.ERR_UNSUPPORTED, "D must be")
    _err(f(FAKE, FAKE, 1, 1, 4, 4, 128, float("inf"), FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "tau")


def test_select_validation():
    f = _lib().sparstar_select_blocks
    _err(f(NULL, 1, 1, 4, 16, 1, 0.25, FAKE, FAKE, 5, NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(f(FAKE, 1, 1, 4, 16, 17, 0.25, FAKE, FAKE, 5, NULL), sp.ERR_INVALID_ARGUMENT, "n_forced")
    _err(f(FAKE, 1, 1, 4, 16, 1, 1.25, FAKE, FAKE, 5, NULL), sp.ERR_INVALID_ARGUMENT, "density")
    _err(f(FAKE, 1, 1, 4, 16, 1, -0.1, FAKE, FAKE, 5, NULL), sp.ERR_INVALID_ARGUMENT, "density")
    _err(f(FAKE, 1, 1, 4, 16, 1, 0.25, FAKE, FAKE, 4, NULL), sp.ERR_INVALID_ARGUMENT, "max_kept")


def test_fused_select_validation():
    f = _lib().sparstar_select_blocks_from_means
    ws = sp.select_workspace_bytes(1, 1, 4, 16)
    assert ws > 0
    ok = [FAKE, FAKE, 1, 1, 4, 16, 128, 0.088, 1, 0.25, FAKE, FAKE, 5, FAKE, ws, NULL]

    def call(**kw):
        a = list(ok)
        pos = {"qbar": 0, "nqb": 4, "nkb": 5, "D": 6, "tau": 7, "F": 8, "density": 9,
               "cnt": 10, "max_kept": 12, "ws": 13, "ws_bytes": 14}
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    _err(call(qbar=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(cnt=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(qbar=ctypes.c_void_p(4100)), sp.ERR_INVALID_ARGUMENT, "aligned")
    _err(call(nqb=0), sp.ERR_INVALID_ARGUMENT, "nqb")
    _err(call(D=96), sp.ERR_UNSUPPORTED, "D must be")
    _err(call(tau=float("inf")), sp.ERR_INVALID_ARGUMENT, "tau")
    _err(call(F=17), sp.ERR_INVALID_ARGUMENT, "n_forced")
    _err(call(density=1.5), sp.ERR_INVALID_ARGUMENT, "density")
    _err(call(max_kept=4), sp.ERR_INVALID_ARGUMENT, "max_kept")
    _err(call(ws=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(ws=ctypes.c_void_p(4096 + 128)), sp.ERR_INVALID_ARGUMENT, "256-byte")
    _err(call(ws_bytes=ws - 1), sp.ERR_INVALID_ARGUMENT, "workspace_bytes")
    big = sp.FUSED_MAX_NKB + 1
    _err(call(nkb=big, max_kept=big), sp.ERR_UNSUPPORTED, "nkb")
    # workspace sizes: float16 screened scores (128 * ceil(nkb / 128) per row),
    # then one float per (head, 128-block strip) of key norms, 256-byte aligned
    assert sp.select_workspace_bytes(1, 16, 563, 1129) == 16 * 563 * 1152 * 2 + 16 * 9 * 4
    assert sp.select_workspace_bytes(1, 1, 3, 129) == 3 * 256 * 2 + 2 * 4
    assert sp.select_workspace_bytes(1, 1, 4, 2049) == -1
    assert sp.select_workspace_bytes(0, 1, 4, 16) == -1
    # the largest supported row passes validation up to the launch (not made here)
    assert sp.FUSED_MAX_NKB == 2048


def test_select_from_qk_validation():
    """The whole-stage entry point checks the means' and the selection's
    arguments, and the workspace, before anything is enqueued."""
    f = _lib().sparstar_select_blocks_from_qk
    ws = sp.select_workspace_bytes(1, 1, 4, 16)
    BF = sp.BF16
    ok = [FAKE, FAKE, BF, 1, 1, 500, 2000, 128, 128, 0.088, 1, 0.25, FAKE, FAKE, FAKE, FAKE, 5, FAKE,
          ws, NULL]

    def call(**kw):
        a = list(ok)
        pos = {"q": 0, "k": 1, "dtype": 2, "Nq": 5, "Nk": 6, "D": 7, "block": 8, "tau": 9, "F": 10,
               "density": 11, "qbar": 12, "cnt": 14, "max_kept": 16, "ws": 17, "ws_bytes": 18}
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    _err(call(q=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(k=ctypes.c_void_p(4100)), sp.ERR_INVALID_ARGUMENT, "aligned")
    _err(call(dtype=7), sp.ERR_INVALID_ARGUMENT, "dtype")
    _err(call(Nq=0), sp.ERR_INVALID_ARGUMENT, "sequence length")
    _err(call(Nk=0), sp.ERR_INVALID_ARGUMENT, "sequence length")
    _err(call(D=96), sp.ERR_UNSUPPORTED, "D must be")
    _err(call(block=48), sp.ERR_UNSUPPORTED, "block")
    _err(call(qbar=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(cnt=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(tau=float("nan")), sp.ERR_INVALID_ARGUMENT, "tau")
    _err(call(F=17), sp.ERR_INVALID_ARGUMENT, "n_forced")
    _err(call(density=-0.5), sp.ERR_INVALID_ARGUMENT, "density")
    _err(call(max_kept=4), sp.ERR_INVALID_ARGUMENT, "max_kept")
    # nkb = ceil(Nk / block): 2049 blocks exceed the screened route
    _err(call(Nk=2049 * 128, max_kept=2049), sp.ERR_UNSUPPORTED, "nkb")
    _err(call(ws=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(ws=ctypes.c_void_p(4096 + 64)), sp.ERR_INVALID_ARGUMENT, "256-byte")
    _err(call(ws_bytes=ws - 1), sp.ERR_INVALID_ARGUMENT, "workspace_bytes")


def test_noalloc_validation():
    """The allocation-free route refuses sizes beyond its 64 MiB scratch, and
    bad arguments, before anything is enqueued."""
    f = _lib().sparstar_select_blocks_from_means_noalloc
    assert sp.select_workspace_bytes(1, 64, 1000, 2048) > 64 << 20
    assert sp.select_workspace_bytes(1, 16, 563, 1129) <= 64 << 20
    _err(f(FAKE, FAKE, 1, 64, 1000, 2048, 128, 0.088, 4, 0.1, FAKE, FAKE, 210, NULL),
         sp.ERR_UNSUPPORTED, "scratch")
    _err(f(NULL, FAKE, 1, 1, 4, 16, 128, 0.088, 1, 0.25, FAKE, FAKE, 5, NULL),
         sp.ERR_INVALID_ARGUMENT, "null")
    _err(f(FAKE, FAKE, 1, 1, 4, 16, 128, 0.088, 1, 0.25, FAKE, FAKE, 4, NULL),
         sp.ERR_INVALID_ARGUMENT, "max_kept")
    _err(f(FAKE, FAKE, 1, 1, 4, 2049, 128, 0.088, 1, 0.25, FAKE, FAKE, 600, NULL),
         sp.ERR_UNSUPPORTED, "nkb")


def test_retained_mass_validation():
    f = _lib().sparstar_retained_mass
    _err(f(FAKE, FAKE, -1, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "n must be")
    _err(f(NULL, FAKE, 10, FAKE, NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(f(FAKE, FAKE, 10, NULL, NULL), sp.ERR_INVALID_ARGUMENT, "null")
    assert f(NULL, NULL, 0, NULL, NULL) == sp.OK   # nothing to do, nothing touched


def test_token_bound_validation():
    f = _lib().sparstar_token_topk_bound
    args = [FAKE, FAKE, 1, 1, 2, 300, 700, 128, 128, 2, 1, 0.088, FAKE, NULL]

    def call(**kw):
        a = list(args)
        pos = {"q": 0, "k": 1, "dtype": 2, "B": 3, "Nq": 5, "Nk": 6, "D": 7, "block": 8, "F": 9,
               "kb": 10, "scale": 11, "out": 12}
        for key, v in kw.items():
            a[pos[key]] = v
        return f(*a)

    _err(call(q=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(out=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(dtype=0), sp.ERR_UNSUPPORTED, "bf16")
    _err(call(dtype=7), sp.ERR_INVALID_ARGUMENT, "dtype")
    _err(call(q=ctypes.c_void_p(4100)), sp.ERR_INVALID_ARGUMENT, "aligned")
    _err(call(Nk=0), sp.ERR_INVALID_ARGUMENT, "sequence")
    _err(call(D=96), sp.ERR_UNSUPPORTED, "D must be")
    _err(call(block=96), sp.ERR_UNSUPPORTED, "block")
    _err(call(F=-1), sp.ERR_INVALID_ARGUMENT, "block counts")
    _err(call(kb=-2), sp.ERR_INVALID_ARGUMENT, "block counts")
    _err(call(scale=0.0), sp.ERR_INVALID_ARGUMENT, "scale")
    _err(call(scale=float("inf")), sp.ERR_INVALID_ARGUMENT, "scale")


def test_transfer_validation():
    f = _lib().sparstar_transfer_scores
    FAKE2 = ctypes.c_void_p(8192)
    args = [FAKE, 1, 16, 128, 512, 32000, 32000, 512, 72000, 72000, FAKE2, NULL]

    def call(**kw):
        a = list(args)
        pos = {"src": 0, "B": 1, "H": 2, "block": 3, "st": 4, "sr": 5, "sc": 6, "dt": 7, "dr": 8,
               "dc": 9, "dst": 10}
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    _err(call(src=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(dst=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(dst=FAKE), sp.ERR_INVALID_ARGUMENT, "overlap")
    _err(call(B=0), sp.ERR_INVALID_ARGUMENT, "B and H")
    _err(call(block=256), sp.ERR_UNSUPPORTED, "block")
    _err(call(block=96), sp.ERR_UNSUPPORTED, "block")
    _err(call(sr=-1), sp.ERR_INVALID_ARGUMENT, ">= 0")
    _err(call(sr=0), sp.ERR_INVALID_ARGUMENT, "empty source segment")
    _err(call(st=0), sp.ERR_INVALID_ARGUMENT, "empty source segment")
    _err(call(sc=0), sp.ERR_INVALID_ARGUMENT, "empty source segment")
    _err(call(sc=0, dc=0, st=1, sr=1), sp.ERR_INVALID_ARGUMENT, "n_cur")
    _err(call(dr=1 << 30), sp.ERR_INVALID_ARGUMENT, "2^30")
    _err(call(dr=600_000_000, dc=600_000_000), sp.ERR_INVALID_ARGUMENT, "2^30")
    _err(call(block=32, dr=400_000_000, dc=400_000_000), sp.ERR_INVALID_ARGUMENT, "int32")


def test_attn_validation():
    f = _lib().sparstar_block_sparse_attn_fwd
    args = [FAKE, FAKE, FAKE, 1, 1, 1, 256, 256, 128, 128, FAKE, FAKE, 2, 0.088, FAKE, NULL, NULL]

    def call(**kw):
        a = list(args)
        pos = {"q": 0, "dtype": 3, "B": 4, "Nq": 6, "Nk": 7, "D": 8, "block": 9, "idx": 11,
               "max_kept": 12, "scale": 13, "o": 14}
        for k, v in kw.items():
            a[pos[k]] = v
        return f(*a)

    _err(call(q=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(o=NULL), sp.ERR_INVALID_ARGUMENT, "null")
    _err(call(idx=NULL), sp.ERR_INVALID_ARGUMENT, "kv_index")
    _err(call(D=80), sp.ERR_UNSUPPORTED, "D must be")
    _err(call(block=256), sp.ERR_UNSUPPORTED, "block")
    _err(call(block=48), sp.ERR_UNSUPPORTED, "block")
    _err(call(Nk=0), sp.ERR_INVALID_ARGUMENT, "sequence")
    _err(call(scale=0.0), sp.ERR_INVALID_ARGUMENT, "scale")
    _err(call(scale=float("nan")), sp.ERR_INVALID_ARGUMENT, "scale")
    _err(call(max_kept=-1), sp.ERR_INVALID_ARGUMENT, "max_kept")
    _err(call(dtype=5), sp.ERR_INVALID_ARGUMENT, "dtype")
    # the stated per-head limit N * D < 2^31 (byte offsets inside one head's
    # bf16 K/V slab then fit the unsigned 32-bit buffer offsets)
    _err(call(Nk=1 << 24), sp.ERR_INVALID_ARGUMENT, "N*D")
    _err(call(Nq=1 << 24), sp.ERR_INVALID_ARGUMENT, "N*D")
    _err(call(Nk=1 << 25, D=64), sp.ERR_INVALID_ARGUMENT, "N*D")


def test_error_cleared_on_next_call():
    f = _lib().sparstar_block_means
    f(NULL, 1, 1, 1, 128, 128, 128, FAKE, NULL)
    assert sp.last_error() != ""
    f(FAKE, 1, 1, 1, 128, 96, 128, FAKE, NULL)
    assert "D must be" in sp.last_error()


def test_product_path_does_not_import_oracle():
    """The binding and the build script never reference the oracle."""
    pkg = os.path.join(ROOT, "block_sparse_attention_head_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "oracle" not in text.lower(), fn


@pytest.mark.skipif(__import__("torch").cuda.is_available(),
                    reason="only where no GPU is visible: the call must fail at the launch")
def test_launch_failure_is_reported_without_a_gpu():
    """Valid arguments but no GPU: the launch fails, the call returns
    SPARSTAR_ERR_HIP with a message, and the next call clears it."""
    st = _lib().sparstar_block_means(FAKE, 1, 1, 1, 256, 128, 128, FAKE, NULL)
    assert st == sp.ERR_HIP, (st, sp.last_error())
    assert "sparstar_block_means" in sp.last_error()
    st = _lib().sparstar_block_scores(FAKE, FAKE, 1, 1, 4, 4, 128, 0.1, FAKE, NULL)
    assert st == sp.ERR_HIP, (st, sp.last_error())
    assert sp.last_error() != ""
    # the largest key length the API admits at D = 128 passes validation
    st = _lib().sparstar_block_sparse_attn_fwd(FAKE, FAKE, FAKE, 1, 1, 1, 256, (1 << 24) - 1, 128,
                                               128, FAKE, FAKE, 2, 0.088, FAKE, NULL, NULL)
    assert st == sp.ERR_HIP, (st, sp.last_error())
    _err(_lib().sparstar_block_means(NULL, 1, 1, 1, 128, 128, 128, FAKE, NULL),
         sp.ERR_INVALID_ARGUMENT, "null")


def test_binding_checks_shapes_and_dtypes_before_calling():
    """The binding refuses tensors whose dtype or shape does not match what
    the library will read and write through raw pointers (host tensors here:
    every check fails before any device pointer is taken)."""
    import torch
    bf, f32, i32 = torch.bfloat16, torch.float32, torch.int32
    q = torch.zeros((1, 2, 300, 128), dtype=bf)
    k = torch.zeros((1, 2, 500, 128), dtype=bf)
    cnt = torch.zeros((1, 2, 3), dtype=i32)
    idx = torch.zeros((1, 2, 3, 4), dtype=i32)
    with pytest.raises(TypeError, match="k must be"):
        sp.block_sparse_attn_fwd(q, k.float(), k, cnt, idx)
    with pytest.raises(ValueError, match="v must have shape"):
        sp.block_sparse_attn_fwd(q, k, k[:, :, :400], cnt, idx)
    with pytest.raises(ValueError, match="k must have shape"):
        sp.block_sparse_attn_fwd(q, k[..., :64].contiguous(), k, cnt, idx)
    with pytest.raises(TypeError, match="kv_index must be"):
        sp.block_sparse_attn_fwd(q, k, k, cnt, idx.long())
    with pytest.raises(ValueError, match="kv_count must have shape"):
        sp.block_sparse_attn_fwd(q, k, k, cnt[:, :, :2], idx)
    with pytest.raises(ValueError, match="kv_count must have shape"):
        sp.block_sparse_attn_fwd(q, k, k, cnt, idx, block=64)      # 5 query blocks at 64
    with pytest.raises(ValueError, match="out must have shape"):
        sp.block_sparse_attn_fwd(q, k, k, cnt, idx, out=q[:, :1])
    with pytest.raises(ValueError, match="lse must have shape"):
        sp.block_sparse_attn_fwd(q, k, k, cnt, idx, lse=torch.zeros((1, 2, 299)))
    S = torch.zeros((1, 2, 3, 4), dtype=f32)
    # a supplied kv_index fixes max_kept; a mismatched explicit max_kept is refused
    with pytest.raises(ValueError, match="kv_index must have shape"):
        sp.select_blocks(S, 1, 0.5, max_kept=3, kv_index=idx)
    with pytest.raises(TypeError, match="S must be"):
        sp.select_blocks(S.double(), 1, 0.5)
    with pytest.raises(ValueError, match="kv_count must have shape"):
        sp.select_blocks(S, 1, 0.5, kv_count=cnt[0])
    qbar = torch.zeros((1, 2, 3, 128), dtype=f32)
    with pytest.raises(ValueError, match="kbar must have shape"):
        sp.select_blocks_from_means(qbar, torch.zeros((1, 1, 4, 128)), 1, 0.5)
    with pytest.raises(ValueError, match="S must have shape"):
        sp.block_scores(qbar, torch.zeros((1, 2, 4, 128)), out=torch.zeros((1, 2, 3, 5)))
    with pytest.raises(ValueError, match="out must have shape"):
        sp.block_means(q, out=torch.zeros((1, 2, 2, 128)))
