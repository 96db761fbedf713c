"""CPU checks of the C ABI: the library loads, exports every declared symbol,
rejects bad arguments before launching anything, and its host-side Hilbert
order agrees with the oracle's.  No test here touches a GPU."""
import ctypes
import math
import os
import re
import shutil
import subprocess

import numpy as np
import pytest

import free_block_sparse_mask_amd as fb
from oracle import sparge_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparge.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fb.LIB_PATH), reason="libsparge.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sparge_[a-z_0-9]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    L = fb.lib()
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(L, n), n
        assert n in fb._SIGNATURES, f"binding lacks {n}"


def test_constants_agree_with_the_oracle():
    assert fb.lib().sparge_version() >= 10000
    assert fb.rows_per_wave() == O.ROWS_PER_GROUP
    text = open(HEADER).read()
    assert f"#define SPARGE_BQ {O.BQ}" in text and f"#define SPARGE_BK {O.BK}" in text


def _t(B, H, N, d, contiguous=True):
    return fb.SpargeTensor(B, H, N, d, H * N * d, N * d, d)


FAKE = ctypes.c_void_p(1 << 20)   # never dereferenced: every call below fails its host checks


def _attn(q, k, v, o, qk=fb.BF16, pv=fb.BF16, lam=-5.0, causal=0, mg=FAKE, cnt=None, idx=None,
          counts=FAKE, ws=None, ws_bytes=0, scales=(None, None), od=None):
    L = fb.lib()
    return L.sparge_attn(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), FAKE, ctypes.byref(v), FAKE,
                         ctypes.byref(o), qk, pv, pv if od is None else od, scales[0], scales[1], mg,
                         cnt, idx, lam, causal, counts, None, ws, ws_bytes, None)


def test_attn_rejects_bad_arguments_before_launch():
    q, k = _t(1, 4, 256, 128), _t(1, 2, 256, 128)
    assert _attn(q, k, k, q, lam=0.0) == fb.SPARGE_EINVAL              # lambda must be < 0
    assert _attn(q, k, k, q, lam=float("nan")) == fb.SPARGE_EINVAL
    assert _attn(q, k, k, q, lam=1.0) == fb.SPARGE_EINVAL
    assert _attn(q, k, k, q, causal=2) == fb.SPARGE_EINVAL
    assert _attn(q, k, k, q, qk=fb.F16, pv=fb.BF16) == fb.SPARGE_EINVAL  # dtype pair
    assert _attn(q, k, k, q, od=fb.F16) == fb.SPARGE_EINVAL              # o dtype
    o_odd = fb.SpargeTensor(1, 4, 256, 128, 4 * 256 * 130, 256 * 130, 130)
    assert _attn(q, k, k, o_odd, od=fb.F32) == fb.SPARGE_EINVAL          # 520-byte rows
    assert _attn(q, _t(1, 3, 256, 128), _t(1, 3, 256, 128), q) == fb.SPARGE_EINVAL  # H % H_kv
    assert _attn(q, _t(1, 2, 255, 128), k, q) == fb.SPARGE_EINVAL       # N differs
    assert _attn(q, k, k, _t(1, 4, 256, 64)) == fb.SPARGE_EINVAL        # o shape
    q96, k96 = _t(1, 4, 256, 96), _t(1, 2, 256, 96)
    assert _attn(q96, k96, k96, q96) == fb.SPARGE_EUNSUPPORTED          # d not 64 / 128
    big_q, big_k = _t(1, 1, 64 * 4096 + 1, 128), _t(1, 1, 64 * 4096 + 1, 128)
    assert _attn(big_q, big_k, big_k, big_q) == fb.SPARGE_EUNSUPPORTED  # Tn > SPARGE_MAX_TN
    assert _attn(q, k, k, q, mg=None) == fb.SPARGE_EINVAL               # M_g required
    assert _attn(q, k, k, q, counts=None) == fb.SPARGE_EINVAL
    assert _attn(q, k, k, q, cnt=FAKE) == fb.SPARGE_EINVAL              # lists come in pairs
    assert _attn(q, k, k, q) == fb.SPARGE_EWORKSPACE                    # V^T and lists in workspace
    assert _attn(q, k, k, q, cnt=FAKE, idx=FAKE) == fb.SPARGE_EWORKSPACE
    assert _attn(q, k, k, q, qk=fb.I8, pv=fb.F16) == fb.SPARGE_EINVAL   # int8 needs scales
    strided = fb.SpargeTensor(1, 4, 256, 128, 4 * 256 * 136, 256 * 136, 136)
    assert _attn(strided, k, k, q, qk=fb.I8, pv=fb.F16, scales=(FAKE, FAKE)) == fb.SPARGE_EINVAL
    odd = fb.SpargeTensor(1, 4, 256, 128, 4 * 256 * 129, 256 * 129, 129)
    assert _attn(odd, k, k, q) == fb.SPARGE_EINVAL                      # 16-byte strides
    neg = fb.SpargeTensor(1, 4, -1, 128, 0, 0, 128)
    assert _attn(neg, k, k, q) == fb.SPARGE_EINVAL
    msg = fb.lib().sparge_last_error().decode()
    assert "negative" in msg


def test_predict_and_quant_reject_bad_arguments():
    L = fb.lib()
    q, k = _t(1, 4, 256, 128), _t(1, 2, 256, 128)
    for tau in (0.0, -0.1, 1.5, float("nan")):
        rc = L.sparge_predict_mask(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.BF16, tau, 0.5, 0,
                                   FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
        assert rc == fb.SPARGE_EINVAL, tau
    for theta in (float("nan"), float("inf")):
        rc = L.sparge_predict_mask(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.BF16, 0.9, theta, 0,
                                   FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
        assert rc == fb.SPARGE_EINVAL
    rc = L.sparge_predict_mask(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.I8, 0.9, 0.5, 0,
                               FAKE, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert rc == fb.SPARGE_EINVAL
    rc = L.sparge_predict_mask(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.BF16, 0.9, 0.5, 0,
                               None, FAKE, FAKE, None, None, FAKE, 1 << 40, None)
    assert rc == fb.SPARGE_EINVAL
    need = L.sparge_workspace_size(ctypes.byref(q), ctypes.byref(k))
    rc = L.sparge_predict_mask(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.BF16, 0.9, 0.5, 0,
                               FAKE, FAKE, FAKE, None, None, FAKE, need - 1, None)
    assert rc == fb.SPARGE_EWORKSPACE
    rc = L.sparge_quant_qk_int8(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.BF16, None, FAKE,
                                FAKE, FAKE, FAKE, need, None)
    assert rc == fb.SPARGE_EINVAL
    rc = L.sparge_quant_qk_int8(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), fb.BF16, FAKE, FAKE,
                                FAKE, FAKE, FAKE, need - 1, None)
    assert rc == fb.SPARGE_EWORKSPACE


def test_empty_problems_launch_nothing():
    L = fb.lib()
    for q, k in ((_t(1, 2, 0, 64), _t(1, 2, 0, 64)), (_t(0, 2, 128, 64), _t(0, 2, 128, 64))):
        assert L.sparge_predict_mask(None, ctypes.byref(q), None, ctypes.byref(k), fb.F16, 0.9, 0.5, 1,
                                     None, None, None, None, None, None, 0, None) == fb.SPARGE_OK
        assert L.sparge_quant_qk_int8(None, ctypes.byref(q), None, ctypes.byref(k), fb.F16, None, None,
                                      None, None, None, 0, None) == fb.SPARGE_OK
        assert L.sparge_hilbert_permute(None, ctypes.byref(q), None, ctypes.byref(q), fb.F16, None, 0,
                                        None) == fb.SPARGE_OK


def test_permute_rejects_bad_arguments():
    L = fb.lib()
    x = _t(1, 2, 100, 64)
    assert L.sparge_hilbert_permute(FAKE, ctypes.byref(x), FAKE, ctypes.byref(_t(1, 2, 99, 64)),
                                    fb.BF16, FAKE, 0, None) == fb.SPARGE_EINVAL
    assert L.sparge_hilbert_permute(FAKE, ctypes.byref(x), FAKE, ctypes.byref(x), 7, FAKE, 0,
                                    None) == fb.SPARGE_EINVAL
    assert L.sparge_hilbert_permute(FAKE, ctypes.byref(x), FAKE, ctypes.byref(x), fb.BF16, FAKE, 2,
                                    None) == fb.SPARGE_EINVAL
    assert L.sparge_hilbert_permute(FAKE, ctypes.byref(x), FAKE, ctypes.byref(x), fb.BF16, FAKE, 0,
                                    None) == fb.SPARGE_EINVAL           # x == y
    # x spans 1 * 2 * 100 * 64 bf16 = 25600 bytes: a y that starts inside it overlaps,
    # one that starts at its end does not (the launch is never reached: perm is null)
    base = 1 << 20
    for off, rc in ((25600 - 16, fb.SPARGE_EINVAL), (16, fb.SPARGE_EINVAL), (-16, fb.SPARGE_EINVAL),
                    (25600, fb.SPARGE_EINVAL), (-25600, fb.SPARGE_EINVAL)):
        got = L.sparge_hilbert_permute(ctypes.c_void_p(base), ctypes.byref(x), ctypes.c_void_p(base + off),
                                       ctypes.byref(x), fb.BF16, None, 0, None)
        assert got == rc
        msg = L.sparge_last_error().decode()
        assert ("overlap" in msg) == (abs(off) < 25600), (off, msg)
    y8 =fb.SpargeTensor(1, 2, 100, 8, 2 * 100 * 16, 100 * 16, 16)   # 8-byte rows, 16-byte stride
    assert L.sparge_hilbert_permute(FAKE, ctypes.byref(y8), ctypes.c_void_p(1 << 21), ctypes.byref(y8),
                                    fb.I8, FAKE, 0, None) == fb.SPARGE_EUNSUPPORTED  # 8-byte rows


def test_workspace_size_grows_with_the_problem():
    L = fb.lib()
    small = L.sparge_workspace_size(ctypes.byref(_t(1, 2, 1024, 64)), ctypes.byref(_t(1, 2, 1024, 64)))
    big = L.sparge_workspace_size(ctypes.byref(_t(1, 32, 131072, 128)), ctypes.byref(_t(1, 8, 131072, 128)))
    assert 0 < small < big
    # the float64 compressed map [B, H, Tm, Tn] dominates
    assert big >= 8 * 32 * 1024 * 2048


@pytest.mark.parametrize("grid", [(12, 48, 80), (1, 6, 6), (4, 16, 16), (3, 5, 7), (1, 1, 1), (2, 64, 1)])
def test_hilbert_index_matches_oracle(grid):
    perm, inv = fb.hilbert_index(*grid)
    p_ref, i_ref = O.hilbert_permutation(*grid)
    assert np.array_equal(perm, p_ref) and np.array_equal(inv, i_ref)


def test_hilbert_index_rejects_bad_grids():
    L = fb.lib()
    buf = np.zeros(4, dtype=np.int32)
    assert L.sparge_hilbert_index(0, 2, 2, buf.ctypes.data, buf.ctypes.data) == fb.SPARGE_EINVAL
    assert L.sparge_hilbert_index(2, 2, 2, None, buf.ctypes.data) == fb.SPARGE_EINVAL
    assert L.sparge_hilbert_index(1 << 11, 1 << 11, 1 << 10, buf.ctypes.data,
                                  buf.ctypes.data) == fb.SPARGE_EUNSUPPORTED


@pytest.mark.parametrize("grid", [(12, 48, 80), (1, 6, 6), (3, 5, 7), (2, 64, 1), (5, 1, 1)])
def test_grid_orders_match_oracle(grid):
    T, Hg, Wg = grid
    refs = {fb.ORDER_HILBERT: O.hilbert_permutation(T, Hg, Wg)[0],
            fb.ORDER_ROWMAJOR: O.raster_order(T, Hg, Wg),
            fb.ORDER_TIMEMAJOR: O.time_major_order(T, Hg, Wg)}
    for order, ref in refs.items():
        perm, inv = fb.grid_order(T, Hg, Wg, order)
        assert np.array_equal(perm, ref), order
        assert np.array_equal(inv[perm], np.arange(perm.size)), order


def test_grid_order_and_l1_reject_bad_arguments():
    L = fb.lib()
    buf = np.zeros(8, dtype=np.int32)
    assert L.sparge_grid_order(2, 2, 2, 3, buf.ctypes.data, buf.ctypes.data) == fb.SPARGE_EINVAL
    assert L.sparge_grid_order(2, 0, 2, 1, buf.ctypes.data, buf.ctypes.data) == fb.SPARGE_EINVAL
    assert L.sparge_grid_order(2, 2, 2, 1, None, buf.ctypes.data) == fb.SPARGE_EINVAL
    x = _t(1, 2, 10, 64)
    FAKE = ctypes.c_void_p(1 << 20)
    ws = L.sparge_l1_workspace_size()
    assert ws >= 16 * 1024
    assert L.sparge_l1_sums(FAKE, ctypes.byref(x), fb.I8, FAKE, ctypes.byref(x), fb.F16, FAKE, FAKE, ws,
                            None) == fb.SPARGE_EINVAL
    assert L.sparge_l1_sums(FAKE, ctypes.byref(x), fb.F16, FAKE, ctypes.byref(_t(1, 2, 11, 64)), fb.F16, FAKE,
                            FAKE, ws, None) == fb.SPARGE_EINVAL
    assert L.sparge_l1_sums(FAKE, ctypes.byref(x), fb.F16, FAKE, ctypes.byref(x), fb.F16, None, FAKE, ws,
                            None) == fb.SPARGE_EINVAL
    assert L.sparge_l1_sums(FAKE, ctypes.byref(x), fb.F16, FAKE, ctypes.byref(x), fb.F16, FAKE, FAKE, ws - 1,
                            None) == fb.SPARGE_EWORKSPACE


def test_noalloc_rejects_problems_beyond_its_scratch():
    """The static scratch of sparge_attn_noalloc holds 64 MiB: at B = 1,
    H = 8, H_kv = 2, d = 128 that is N up to 65536.  A larger problem is
    refused on the host, before any device call, naming both sizes."""
    L = fb.lib()
    text = open(HEADER).read()
    assert "#define SPARGE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)" in text
    q, k = _t(1, 8, 70000, 128), _t(1, 2, 70000, 128)
    rc = L.sparge_attn_noalloc(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), FAKE, ctypes.byref(k), FAKE,
                               ctypes.byref(q), fb.BF16, fb.BF16, fb.BF16, None, None, FAKE, None, None,
                               -5.0, 1, FAKE, None, None)
    assert rc == fb.SPARGE_EWORKSPACE
    msg = L.sparge_last_error().decode()
    assert "scratch" in msg and str(64 << 20) in msg, msg
    # the scratch formula of the header, evaluated here, agrees on both sides of the limit
    def need(H, Hkv, N, d):
        Tm, Tn = -(-N // 128), -(-N // 64)
        return 2 * Hkv * d * 64 * Tn + 8 * H * N + 6 * H * Tm * Tn + 8 * Hkv * d * -(-N // 1024)
    assert need(8, 2, 70000, 128) > 64 << 20 > need(8, 2, 65536, 128)
    # the other argument checks are sparge_attn's
    assert L.sparge_attn_noalloc(FAKE, ctypes.byref(q), FAKE, ctypes.byref(k), FAKE, ctypes.byref(k), FAKE,
                                 ctypes.byref(q), fb.BF16, fb.BF16, fb.BF16, None, None, FAKE, None, None,
                                 0.5, 1, FAKE, None, None) == fb.SPARGE_EINVAL


def test_header_and_library_from_c(tmp_path):
    """include/sparge.h compiles as C99 with every warning an error, a C
    program links against libsparge.so, and its host-only calls (version,
    rows per wavefront, the path setting, Hilbert and grid orders, workspace
    sizes, the error codes and messages) behave as the header states
    (tests/c/abi_from_c.c)."""
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    libdir = os.path.dirname(fb.LIB_PATH)
    exe = str(tmp_path / "abi_from_c")
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_from_c.c"), "-o", exe, f"-L{libdir}", "-lsparge",
           f"-Wl,-rpath,{libdir}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
