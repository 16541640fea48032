"""Host-side checks of libfa.so: it loads, exports what include/fa.h declares, and
rejects bad arguments with the documented codes before any device work.  These
calls never reach a kernel launch, so they run without a GPU."""
import ctypes
import os
import re

import pytest

import io_aware_exact_02_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, HEADDIM, DTYPE, SCALE, WORKSPACE, LAUNCH, ALIGN, PHASE = 0, -1, -2, -3, -4, -5, -6, -7, -8, -9
SCRATCH = -10
P = 0x10000          # a fake, 16-byte aligned pointer value: never dereferenced on these paths


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (python -m io_aware_exact_02_amd.build)")
    return fa.library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(fa.EXPORTED_SYMBOLS)
    raw = ctypes.CDLL(fa.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), name


def test_header_documents_every_status_code():
    text = open(HEADER).read()
    for name, val in (("FA_OK", 0), ("FA_ERR_NULL", -1), ("FA_ERR_SHAPE", -2), ("FA_ERR_HEADDIM", -3),
                      ("FA_ERR_DTYPE", -4), ("FA_ERR_SCALE", -5), ("FA_ERR_WORKSPACE", -6),
                      ("FA_ERR_LAUNCH", -7), ("FA_ERR_ALIGN", -8), ("FA_ERR_PHASE", -9),
                      ("FA_ERR_SCRATCH", -10)):
        assert re.search(rf"{name}\s*=\s*{val}\b", text), name


def test_strerror_and_version(lib):
    assert fa.fa_abi_version() == 1
    msgs = {s: fa.fa_strerror(s) for s in (OK, NULL, SHAPE, HEADDIM, DTYPE, SCALE, WORKSPACE, LAUNCH, ALIGN, PHASE,
                                           SCRATCH)}
    assert msgs[OK] == "success"
    assert len(set(msgs.values())) == len(msgs)
    assert "unknown" in fa.fa_strerror(12345)


def _fwd(lib, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Tq=8, Tk=8, d=64, scale=0.125, causal=0, dtype=fa.FA_BF16,
         odtype=None):
    odtype = dtype if odtype is None else odtype
    return lib.fa_fwd(q, k, v, o, lse, B, H, Tq, Tk, d, scale, causal, dtype, odtype, None)


def test_fwd_argument_errors(lib):
    assert _fwd(lib, q=None) == NULL
    assert _fwd(lib, lse=None) == NULL
    for bad in (dict(B=0), dict(H=0), dict(Tq=0), dict(Tk=0), dict(Tk=-3)):
        assert _fwd(lib, **bad) == SHAPE, bad
    for d in (0, 32, 96, 100, 512):
        assert _fwd(lib, d=d) == HEADDIM, d
    assert _fwd(lib, dtype=2) == DTYPE
    assert _fwd(lib, dtype=-1) == DTYPE
    assert _fwd(lib, dtype=fa.FA_F32, odtype=fa.FA_BF16) == DTYPE
    assert _fwd(lib, odtype=3) == DTYPE
    for s in (0.0, -1.0, float("nan"), float("inf")):
        assert _fwd(lib, scale=s) == SCALE, s
    assert _fwd(lib, q=P + 8) == ALIGN
    assert _fwd(lib, lse=P + 4) == ALIGN


def test_bwd_workspace_bytes(lib):
    B, H, Tq, Tk, d = 2, 3, 100, 70, 128
    rows = B * H * Tq
    pad = (rows + 63) // 64 * 64
    # bf16: two row-term arrays (-D and -lse log2 e), for every head width and gradient
    # dtype; float32 inputs: D
    for dd in (64, 128, 256):
        assert fa.fa_bwd_workspace_bytes(B, H, Tq, Tk, dd, fa.FA_BF16, fa.FA_BF16) == 8 * pad
        assert fa.fa_bwd_workspace_bytes(B, H, Tq, Tk, dd, fa.FA_BF16, fa.FA_F32) == 8 * pad
    assert fa.fa_bwd_workspace_bytes(B, H, Tq, Tk, d, fa.FA_F32, fa.FA_F32) == 4 * pad
    assert fa.fa_bwd_workspace_bytes(0, H, Tq, Tk, d, fa.FA_BF16, fa.FA_BF16) == 0
    assert fa.fa_bwd_workspace_bytes(B, H, Tq, Tk, 96, fa.FA_BF16, fa.FA_BF16) == 0


def _bwd(lib, ws=P, ws_bytes=1 << 30, B=1, H=1, Tq=8, Tk=8, d=64, scale=0.125, dtype=fa.FA_BF16,
         gdtype=fa.FA_BF16, odtype=None, null_at=None):
    ptrs = [P] * 9
    if null_at is not None:
        ptrs[null_at] = None
    odtype = dtype if odtype is None else odtype
    return lib.fa_bwd(*ptrs, B, H, Tq, Tk, d, scale, 0, dtype, odtype, gdtype, ws, ws_bytes, None)


def test_bwd_argument_errors(lib):
    for i in range(9):
        assert _bwd(lib, null_at=i) == NULL, i
    assert _bwd(lib, B=0) == SHAPE
    assert _bwd(lib, d=48) == HEADDIM
    assert _bwd(lib, dtype=fa.FA_F32, gdtype=fa.FA_BF16) == DTYPE
    assert _bwd(lib, gdtype=5) == DTYPE
    assert _bwd(lib, dtype=fa.FA_F32, gdtype=fa.FA_F32, odtype=fa.FA_BF16) == DTYPE
    assert _bwd(lib, odtype=7) == DTYPE
    assert _bwd(lib, scale=float("nan")) == SCALE
    assert _bwd(lib, ws=None) == WORKSPACE
    need = fa.fa_bwd_workspace_bytes(1, 1, 8, 8, 64, fa.FA_BF16, fa.FA_BF16)
    assert _bwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert _bwd(lib, ws=P + 8, ws_bytes=need) == ALIGN


def test_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    q = torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.forward(q, q, q)


def test_bwd_phase_mask(lib):
    need = fa.fa_bwd_workspace_bytes(1, 1, 8, 8, 64, fa.FA_BF16, fa.FA_BF16)
    args = [P] * 9 + [1, 1, 8, 8, 64, 0.125, 0, fa.FA_BF16, fa.FA_BF16, fa.FA_BF16, P, need]
    assert lib.fa_bwd_phases(*args, 8, None) == PHASE
    assert lib.fa_bwd_phases(*args, -1, None) == PHASE
    assert lib.fa_bwd_phases(*args, 0, None) == OK          # checks only, launches nothing
    bad = list(args); bad[0] = None
    assert lib.fa_bwd_phases(*bad, 0, None) == NULL


def _dec(lib, ws=P, ws_bytes=1 << 30, B=1, H=1, Tq=1, Tk=100, d=128, scale=0.125, dtype=fa.FA_BF16,
         odtype=fa.FA_BF16, nsplit=0, null_at=None):
    ptrs = [P] * 5
    if null_at is not None:
        ptrs[null_at] = None
    return lib.fa_fwd_splitkv(*ptrs, B, H, Tq, Tk, d, scale, 0, dtype, odtype, nsplit, ws, ws_bytes, None)


def test_splitkv_workspace_and_errors(lib):
    # four partials (one per wave) per key chunk, each d floats of O~ plus 4 statistics per row
    B, H, Tq, Tk, d = 2, 3, 5, 1000, 128
    ns = 3
    assert fa.fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, ns) == 4 * ns * B * H * Tq * (d + 4) * 4
    auto = fa.fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, 0)
    assert auto > 0 and auto % (4 * B * H * Tq * (d + 4) * 4) == 0
    # more chunks than 32-key tiles are clamped to the tile count
    assert fa.fa_fwd_splitkv_workspace_bytes(1, 1, 1, 64, 64, 50) == 4 * 2 * 1 * (64 + 4) * 4
    assert fa.fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, 256, 0) == 0
    assert fa.fa_fwd_splitkv_workspace_bytes(B, H, Tq, Tk, d, -1) == 0
    for i in range(5):
        assert _dec(lib, null_at=i) == NULL, i
    assert _dec(lib, Tk=0) == SHAPE
    assert _dec(lib, nsplit=-2) == SHAPE
    assert _dec(lib, d=256) == HEADDIM
    assert _dec(lib, d=96) == HEADDIM
    assert _dec(lib, dtype=fa.FA_F32, odtype=fa.FA_F32) == DTYPE
    assert _dec(lib, odtype=9) == DTYPE
    assert _dec(lib, scale=0.0) == SCALE
    assert _dec(lib, ws=None) == WORKSPACE
    need = fa.fa_fwd_splitkv_workspace_bytes(1, 1, 1, 100, 128, 0)
    assert _dec(lib, ws_bytes=need - 1) == WORKSPACE
    assert _dec(lib, ws=P + 4, ws_bytes=need) == ALIGN


def _mfwd(lib, mask=P, mheads=1, B=1, H=2, Tq=300, Tk=300, d=128, dtype=fa.FA_BF16, odtype=fa.FA_BF16,
          null_at=None):
    ptrs = [P] * 5
    if null_at is not None:
        ptrs[null_at] = None
    return lib.fa_fwd_masked(*ptrs, B, H, Tq, Tk, d, 0.125, 0, dtype, odtype, mask, mheads, None)


def _mbwd(lib, mask=P, mheads=1, B=1, H=2, Tq=300, Tk=300, d=128, dtype=fa.FA_BF16, ws=P, ws_bytes=1 << 30):
    return lib.fa_bwd_masked(*([P] * 9), B, H, Tq, Tk, d, 0.125, 0, dtype, dtype, dtype, mask, mheads, ws,
                             ws_bytes, None)


def test_masked_argument_errors(lib):
    """The block-sparse entry points: mask presence, its head count, dtype, head
    dimension and block counts are checked before anything is launched."""
    for i in range(5):
        assert _mfwd(lib, null_at=i) == NULL, i
    assert _mfwd(lib, mask=None) == NULL
    assert _mbwd(lib, mask=None) == NULL
    for mh in (0, 3, -1):
        assert _mfwd(lib, mheads=mh) == SHAPE, mh
        assert _mbwd(lib, mheads=mh) == SHAPE, mh
    assert _mfwd(lib, dtype=fa.FA_F32, odtype=fa.FA_F32) == DTYPE
    assert _mbwd(lib, dtype=fa.FA_F32) == DTYPE
    assert _mfwd(lib, odtype=7) == DTYPE
    assert _mbwd(lib, d=96) == HEADDIM
    assert _mfwd(lib, d=96) == HEADDIM
    assert _mfwd(lib, Tq=0) == SHAPE
    assert _mbwd(lib, ws=None) == WORKSPACE
    need = fa.fa_bwd_workspace_bytes(1, 2, 300, 300, 128, fa.FA_BF16, fa.FA_BF16)
    assert _mbwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert _mbwd(lib, ws=P + 8, ws_bytes=need) == ALIGN


def test_masked_phase_mask(lib):
    args = [P] * 9 + [1, 2, 300, 300, 128, 0.125, 0, fa.FA_BF16, fa.FA_BF16, fa.FA_BF16, P, 1, P, 1 << 30]
    assert lib.fa_bwd_masked_phases(*args, 8, None) == PHASE
    assert lib.fa_bwd_masked_phases(*args, 0, None) == OK         # checks only, launches nothing
    bad = list(args)
    bad[19] = None
    assert lib.fa_bwd_masked_phases(*bad, 0, None) == NULL


def test_window_argument_errors(lib):
    def fwd(wl=4, wr=2, dtype=fa.FA_BF16, odtype=fa.FA_BF16, d=128, null_at=None):
        ptrs = [P] * 5
        if null_at is not None:
            ptrs[null_at] = None
        return lib.fa_fwd_window(*ptrs, 1, 2, 300, 300, d, 0.125, wl, wr, dtype, odtype, None)

    def bwd(wl=4, wr=2, dtype=fa.FA_BF16, ws=P, ws_bytes=1 << 30, phases=None):
        args = [P] * 9 + [1, 2, 300, 300, 128, 0.125, wl, wr, dtype, dtype, dtype, ws, ws_bytes]
        if phases is None:
            return lib.fa_bwd_window(*args, None)
        return lib.fa_bwd_window_phases(*args, phases, None)

    for i in range(5):
        assert fwd(null_at=i) == NULL
    for wl, wr in ((-2, 0), (0, -2), (-5, -5)):
        assert fwd(wl, wr) == SHAPE and bwd(wl, wr) == SHAPE
    assert fwd(dtype=fa.FA_F32, odtype=fa.FA_F32) == DTYPE and bwd(dtype=fa.FA_F32) == DTYPE
    assert fwd(d=96) == HEADDIM
    assert bwd(ws=None) == WORKSPACE
    assert bwd(phases=8) == PHASE
    assert bwd(phases=0) == OK              # checks only, launches nothing


def test_docs_argument_errors(lib):
    def fwd(cu=P, nd=3, dtype=fa.FA_BF16, odtype=fa.FA_BF16, d=128, T=300, null_at=None):
        ptrs = [P] * 5
        if null_at is not None:
            ptrs[null_at] = None
        return lib.fa_fwd_docs(*ptrs, 1, 2, T, d, 0.125, 1, cu, nd, dtype, odtype, None)

    def bwd(cu=P, nd=3, dtype=fa.FA_BF16, ws=P, ws_bytes=1 << 30, phases=None):
        args = [P] * 9 + [1, 2, 300, 128, 0.125, 0, cu, nd, dtype, dtype, dtype, ws, ws_bytes]
        if phases is None:
            return lib.fa_bwd_docs(*args, None)
        return lib.fa_bwd_docs_phases(*args, phases, None)

    for i in range(5):
        assert fwd(null_at=i) == NULL
    assert fwd(cu=None) == NULL and bwd(cu=None) == NULL
    for nd in (0, -1):
        assert fwd(nd=nd) == SHAPE and bwd(nd=nd) == SHAPE
    assert fwd(T=0) == SHAPE
    assert fwd(cu=P + 2) == ALIGN and bwd(cu=P + 2) == ALIGN
    assert fwd(dtype=fa.FA_F32, odtype=fa.FA_F32) == DTYPE and bwd(dtype=fa.FA_F32) == DTYPE
    assert fwd(d=96) == HEADDIM
    assert bwd(ws=None) == WORKSPACE
    assert bwd(phases=8) == PHASE
    assert bwd(phases=0) == OK              # checks only, launches nothing


def _bwd_noalloc(lib, B=1, H=1, Tq=8, Tk=8, d=64, scale=0.125, dtype=fa.FA_BF16, gdtype=fa.FA_BF16, odtype=None,
                 null_at=None, misalign_at=None):
    ptrs = [P] * 9
    if null_at is not None:
        ptrs[null_at] = None
    if misalign_at is not None:
        ptrs[misalign_at] = P + 8
    odtype = dtype if odtype is None else odtype
    return lib.fa_bwd_noalloc(*ptrs, B, H, Tq, Tk, d, scale, 0, dtype, odtype, gdtype, None)


def test_bwd_noalloc_argument_errors(lib):
    """fa_bwd_noalloc checks its arguments as fa_bwd does, and rejects problems whose
    workspace exceeds the fixed scratch with FA_ERR_SCRATCH, all before any HIP call."""
    for i in range(9):
        assert _bwd_noalloc(lib, null_at=i) == NULL, i
        assert _bwd_noalloc(lib, misalign_at=i) == ALIGN, i
    assert _bwd_noalloc(lib, B=0) == SHAPE
    assert _bwd_noalloc(lib, d=48) == HEADDIM
    assert _bwd_noalloc(lib, dtype=fa.FA_F32, gdtype=fa.FA_BF16) == DTYPE
    assert _bwd_noalloc(lib, odtype=7) == DTYPE
    assert _bwd_noalloc(lib, scale=0.0) == SCALE
    # bf16: 8 bytes per (padded) query row; the scratch holds 2^21 rows
    rows_max = fa.NOALLOC_SCRATCH_BYTES // 8
    assert fa.fa_bwd_workspace_bytes(1, 32, rows_max // 32, 64, 128, fa.FA_BF16, fa.FA_BF16) \
        == fa.NOALLOC_SCRATCH_BYTES
    assert _bwd_noalloc(lib, B=1, H=32, Tq=rows_max // 32 + 1, Tk=64, d=128) == SCRATCH
    assert _bwd_noalloc(lib, B=2, H=32, Tq=rows_max // 32, Tk=64, d=128) == SCRATCH
    # float32: 4 bytes per row, twice the rows
    assert _bwd_noalloc(lib, B=1, H=64, Tq=rows_max // 32 + 64, Tk=64, d=64, dtype=fa.FA_F32,
                        gdtype=fa.FA_F32) == SCRATCH
