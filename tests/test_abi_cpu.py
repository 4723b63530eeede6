"""CPU-side checks of the C-ABI library: it loads, exports every declared symbol,
and rejects bad arguments before launching anything (no GPU needed for these paths)."""
import ctypes
import os
import re

import pytest

import dsa_lightning_indexer_scores_amd as ic

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "indexcache.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ic_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ic.LIB_PATH):
        pytest.fail(f"{ic.LIB_PATH} missing: run the build first")
    return ic.lib()


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in indexcache.h but not exported"


def test_version_and_empty_error(L):
    assert ic.version() >= 100


def _shape(**kw):
    base = dict(B=1, Lq=512, Lk=512, k=64, H=4, d=64, H_I=4, d_I=32, idx_dtype=ic.IC_BF16)
    base.update(kw)
    return ic.make_shape(**base)


FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation first


def _layers(pattern):
    arr = (ic.Layer * len(pattern))()
    for i, c in enumerate(pattern):
        full = c in "F1"
        arr[i] = ic.Layer(FAKE if full else None, FAKE if full else None, FAKE if full else None, FAKE, FAKE, FAKE)
    return arr


def _stack(pattern, n_layers=None, shape=None, ws_bytes=1 << 30):
    s = shape or _shape()
    n = len(pattern) if n_layers is None else n_layers
    return ic.lib().ic_run_stack(pattern.encode(), n, _layers(pattern.ljust(n, "S")[:n] if n else pattern),
                                 ctypes.byref(s), FAKE, ctypes.c_void_p(0x10000), ws_bytes, None, None)


def test_pattern_errors(L):
    assert _stack("SFSS") == ic.IC_ERR_NO_CACHED_INDICES
    assert "no cached indices" in ic.last_error()
    assert _stack("0100") == ic.IC_ERR_NO_CACHED_INDICES
    assert _stack("FXSS") == ic.IC_ERR_PATTERN
    assert _stack("FSS", n_layers=4) == ic.IC_ERR_PATTERN


def test_shape_and_workspace_errors(L):
    assert _stack("FSSS", shape=_shape(d=96)) == ic.IC_ERR_SHAPE
    assert _stack("FSSS", shape=_shape(d_I=48)) == ic.IC_ERR_SHAPE
    assert _stack("FSSS", shape=_shape(H_I=65)) == ic.IC_ERR_SHAPE
    assert _stack("FSSS", shape=_shape(k=0)) == ic.IC_ERR_SHAPE
    assert _stack("FSSS", shape=_shape(Lq=600)) == ic.IC_ERR_SHAPE        # pos0 + Lq > Lk
    assert _stack("FSSS", shape=_shape(idx_dtype=7)) == ic.IC_ERR_DTYPE
    assert _stack("FSSS", shape=_shape(chunk=100)) == ic.IC_ERR_SHAPE
    assert _stack("FSSS", shape=_shape(Lk=1 << 24, d=64)) == ic.IC_ERR_SHAPE   # 4 GiB of KV rows
    assert "4 GiB" in ic.last_error()
    assert _stack("FSSS", ws_bytes=16) == ic.IC_ERR_WORKSPACE
    need = ic.workspace_size(_shape(), ic.IC_OP_RUN_STACK)
    assert need >= 512 * 512 * 4                                           # one chunk x visible keys, fp32
    assert ic.workspace_size(_shape(d=96), ic.IC_OP_RUN_STACK) == 0


def test_missing_pointers(L):
    arr = _layers("FSSS")
    arr[0].k_I = None
    s = _shape()
    r = L.ic_run_stack(b"FSSS", 4, arr, ctypes.byref(s), FAKE, ctypes.c_void_p(0x10000), 1 << 30, None, None)
    assert r == ic.IC_ERR_ARG
    dec = _shape(Lq=2)
    r = L.ic_decode_step(b"FSSS", 4, _layers("FSSS"), ctypes.byref(dec), FAKE, FAKE, ctypes.c_void_p(0x10000),
                         1 << 30, None, None)
    assert r == ic.IC_ERR_SHAPE                                            # decode needs Lq == 1


def test_workspace_sizes_scale_with_chunk(L):
    s_full = _shape(Lq=8192, Lk=8192, chunk=0)
    s_small = _shape(Lq=8192, Lk=8192, chunk=1024)
    assert ic.workspace_size(s_full, ic.IC_OP_INDEXER_TOPK) == 4096 * 8192 * 4
    assert ic.workspace_size(s_small, ic.IC_OP_INDEXER_TOPK) == 1024 * 8192 * 4
    dec = _shape(B=32, Lq=1, Lk=65600, k=2048, H=16, d=128, H_I=64, d_I=128, idx_dtype=ic.IC_FP8_E4M3)
    assert ic.workspace_size(dec, ic.IC_OP_DECODE_STEP) >= 32 * 65600 * 4


def test_topk_rows_seq_validation(L):
    ws = ctypes.c_void_p(0x10000)
    # NULL seq_len, bad k, max_len beyond the row stride: rejected before any launch
    assert L.ic_topk_rows_seq(FAKE, 100, 4, None, 100, 8, FAKE, None, 0, None) == 1
    assert L.ic_topk_rows_seq(FAKE, 100, 4, FAKE, 100, 0, FAKE, None, 0, None) == 2
    assert L.ic_topk_rows_seq(FAKE, 100, 4, FAKE, 101, 8, FAKE, None, 0, None) == 2
    # a workspace that is given must be large enough and 256-byte aligned
    need = ic.topk_rows_seq_ws(32, 65600, 2048)
    assert L.ic_topk_rows_seq(FAKE, 65600, 32, FAKE, 65600, 2048, FAKE, ws, need - 1, None) == 6
    assert L.ic_topk_rows_seq(FAKE, 65600, 32, FAKE, 65600, 2048, FAKE, ctypes.c_void_p(0x10010), need, None) == 6


def test_topk_rows_seq_workspace_sizes():
    # short rows, or many rows, need none; few long rows keep k candidates (position and
    # key) per 16384-key segment
    assert ic.topk_rows_seq_ws(32, 32768, 2048) == 0
    assert ic.topk_rows_seq_ws(4096, 65600, 2048) == 0
    assert ic.topk_rows_seq_ws(32, 65600, 2048) == 2 * 32 * 5 * 2048 * 4
    assert ic.topk_rows_seq_ws(3, 40000, 100) == 2 * 3 * 3 * 100 * 4
    assert ic.topk_rows_seq_ws(8, 131072, 2048) == 2 * 8 * 8 * 2048 * 4
    # a candidate list longer than one register-resident 1024 x 16 block (16384 keys)
    # falls back to streaming
    assert ic.topk_rows_seq_ws(8, 131073, 2048) == 0
    assert ic.topk_rows_seq_ws(8, 65536, 4096) == 2 * 8 * 4 * 4096 * 4
    assert ic.topk_rows_seq_ws(8, 65537, 4096) == 0


def test_mfma_probe_library_exports_its_entry():
    path = os.path.join(os.path.dirname(ic.LIB_PATH), "libicprobe.so")
    assert os.path.exists(path), "libicprobe.so missing: run the build first"
    P = ctypes.CDLL(path)
    assert hasattr(P, "icp_mfma_stream")
    P.icp_mfma_stream.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert P.icp_mfma_stream(1, 0, 1, None, None) != 0   # rejected before any launch


def test_index_overlap_validation(L):
    # NULL inputs, k out of range, means without the per-row outputs: rejected before any launch
    assert L.ic_index_overlap(None, FAKE, 4, 8, None, None, None, None, None) == 1
    assert L.ic_index_overlap(FAKE, FAKE, 4, 0, None, None, None, None, None) == 2
    assert L.ic_index_overlap(FAKE, FAKE, 4, 5000, None, None, None, None, None) == 2
    assert L.ic_index_overlap(FAKE, FAKE, 4, 8, None, None, None, FAKE, None) == 1


def test_run_stack_varlen_validation(L):
    s = _shape(B=2, Lq=30, Lk=100)
    ql = (ctypes.c_int32 * 2)(10, 20)
    p0 = (ctypes.c_int32 * 2)(0, 50)
    run = lambda pat, shape, q, p: L.ic_run_stack_varlen(pat.encode(), len(pat), _layers(pat), ctypes.byref(shape),
                                                         q, p, FAKE, ctypes.c_void_p(0x10000), 1 << 30, None, None)
    assert run("FS", s, None, p0) == 1                                    # host arrays are required
    assert run("SF", s, ql, p0) == 5                                      # S first
    bad = (ctypes.c_int32 * 2)(10, 21)
    assert run("FS", s, bad, p0) == 2                                     # q_len does not sum to Lq
    far = (ctypes.c_int32 * 2)(0, 90)
    assert run("FS", s, ql, far) == 2                                     # pos0 + q_len beyond Lk
    s2 = _shape(B=2, Lq=30, Lk=100, pos0=5)
    assert run("FS", s2, ql, p0) == 2                                     # per-sequence pos0 only


def test_distill_kl_validation(L):
    s = _shape()
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)
    holes = (ctypes.c_void_p * 2)(FAKE, None)
    ws = ctypes.c_void_p(0x10000)
    need = ic.workspace_size(s, ic.IC_OP_DISTILL_KL)
    assert need == ic.workspace_size(s, ic.IC_OP_INDEXER_TOPK) > 0     # one score tile
    call = lambda shape, n, q, kv, kl=FAKE, wsb=1 << 30: L.ic_distill_kl(
        ctypes.byref(shape), FAKE, FAKE, FAKE, FAKE, n, q, kv, kl, None, ws, wsb, None)
    assert call(s, 0, ptrs, ptrs) == ic.IC_ERR_ARG                      # no served layer
    assert call(s, 17, ptrs, ptrs) == ic.IC_ERR_ARG                     # more than 16
    assert call(s, 2, None, ptrs) == ic.IC_ERR_ARG                      # host pointer arrays required
    assert call(s, 2, ptrs, holes) == ic.IC_ERR_ARG                     # a NULL layer pointer
    assert call(s, 2, ptrs, ptrs, kl=None) == ic.IC_ERR_ARG
    assert call(_shape(d=96), 2, ptrs, ptrs) == ic.IC_ERR_SHAPE
    assert call(_shape(idx_dtype=7), 2, ptrs, ptrs) == ic.IC_ERR_DTYPE
    assert call(s, 2, ptrs, ptrs, wsb=16) == ic.IC_ERR_WORKSPACE


def test_run_stack_dynamic_validation(L):
    s = _shape()
    ws = ctypes.c_void_p(0x10000)
    run = lambda pat, stride=16, tau=0.5, layers=None, wsb=1 << 30: L.ic_run_stack_dynamic(
        pat.encode(), len(pat), layers if layers is not None else _layers(pat), ctypes.byref(s), stride, tau,
        FAKE, None, None, ws, wsb, None, None)
    assert run("SFSS") == ic.IC_ERR_NO_CACHED_INDICES
    assert run("FSSS", stride=0) == ic.IC_ERR_ARG
    assert run("FSSS", tau=-0.1) == ic.IC_ERR_ARG
    assert run("FSSS", tau=float("nan")) == ic.IC_ERR_ARG
    half = _layers("FSSS")
    half[1].q_I = FAKE                                                    # q_I without w and k_I
    assert run("FSSS", layers=half) == ic.IC_ERR_ARG
    assert run("FSSS", wsb=16) == ic.IC_ERR_WORKSPACE
    need = L.ic_run_stack_dynamic_ws(ctypes.byref(s), 16)
    assert need > ic.workspace_size(s, ic.IC_OP_INDEXER_TOPK)            # one tile + probe region
    assert L.ic_run_stack_dynamic_ws(ctypes.byref(s), 1) > need          # more probe rows
    assert L.ic_run_stack_dynamic_ws(ctypes.byref(s), 0) == 0


@pytest.mark.skipif(__import__("torch").cuda.device_count() > 0,
                    reason="launches with placeholder pointers: only where no GPU can run them")
def test_hip_failure_after_validation_is_reported(L):
    """With arguments that pass validation, a HIP runtime failure (here: no device) comes
    back as IC_ERR_HIP naming the launch that failed, from a one-layer call and from the
    middle of a stack call, never as a crash."""
    s = _shape()
    r = L.ic_indexer_scores(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 512, None)
    assert r == ic.IC_ERR_HIP and "indexer launch" in ic.last_error()
    assert _stack("FSSS") == ic.IC_ERR_HIP and "launch" in ic.last_error()
