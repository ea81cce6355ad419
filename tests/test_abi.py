"""The C-ABI library loads and exports every entry point include/fa.h
declares, and argument errors come back as status codes before any GPU work
(CPU only: these calls never reach the HIP runtime)."""
import ctypes
import os
import re

import pytest

from exact_tiled_attention_fwd_amd import _native

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
           if f.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*"
                             r"([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return names


@pytest.fixture(scope="module")
def lib():
    _native.ensure_built()
    return _native.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string"} <= names
    for n in names:
        assert hasattr(lib, n), f"libfa.so does not export {n}"


def test_status_strings(lib):
    for code, name in _native.STATUS_NAMES.items():
        assert _native.fa_status_string(code).startswith(name)
    assert "unknown" in _native.fa_status_string(99)


FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced: validation fails first


def fwd(lib, q=FAKE, k=FAKE, v=FAKE, o=ctypes.c_void_p(0x200000), lse=ctypes.c_void_p(0x900000),
        B=1, H=1, N=8, d=64, dtype=1, scale=0.125, mask=0, window=0):
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, d, dtype, scale, mask, window, None)


def test_fwd_argument_errors(lib):
    assert fwd(lib, q=None) == 1                      # FA_ERR_NULL
    assert fwd(lib, N=0) == 2 and fwd(lib, B=-1) == 2  # FA_ERR_SHAPE
    assert fwd(lib, dtype=7) == 3                     # FA_ERR_DTYPE
    assert fwd(lib, d=96) == 4 and fwd(lib, d=32) == 4  # bf16 needs d in {64, 128}
    assert fwd(lib, dtype=0, d=129) == 4 and fwd(lib, dtype=0, d=0) == 4
    assert fwd(lib, mask=3) == 5 and fwd(lib, mask=2, window=-1) == 5
    assert fwd(lib, scale=float("inf")) == 6 and fwd(lib, scale=float("nan")) == 6
    assert fwd(lib, q=ctypes.c_void_p(0x100004)) == 7  # FA_ERR_ALIGN
    assert fwd(lib, o=FAKE) == 10                     # output aliases an input
    assert fwd(lib, N=1 << 30, d=128) == 2           # N * d beyond 2^31 - 1
    assert fwd(lib, dtype=0, d=1, N=(1 << 29) + 1) == 2  # N beyond 2^29


def test_bwd_argument_errors(lib):
    ws_need = lib.fa_bwd_workspace_bytes(2, 3, 100, 64, 1)
    assert ws_need >= 2 * 3 * 100 * 4 and ws_need % 256 == 0
    assert lib.fa_bwd_workspace_bytes(0, 3, 100, 64, 1) == 0
    assert lib.fa_bwd_workspace_bytes(1, 1, 100, 96, 1) == 0
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]

    def bwd(ws=p[9], wsb=ws_need, scale=0.1, mask=0, window=0, d=64, q=p[0]):
        return lib.fa_bwd(q, p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], ws, wsb,
                          2, 3, 100, d, 1, scale, mask, window, None)
    assert bwd(q=None) == 1
    assert bwd(ws=None) == 8 and bwd(wsb=ws_need - 1) == 8
    assert bwd(mask=2, window=-2) == 5
    assert bwd(scale=float("nan")) == 6
    assert bwd(d=100) == 4


def test_probe_argument_errors(lib):
    out = ctypes.c_double(0.0)
    ref = ctypes.byref(out)
    assert lib.fa_probe_mfma_bf16(100, None, None) == 1          # FA_ERR_NULL
    assert lib.fa_probe_mfma_bf16(0, None, ref) == 2             # FA_ERR_SHAPE
    assert lib.fa_probe_mfma_bf16(1 << 25, None, ref) == 2
    a, b = ctypes.c_void_p(0x100000), ctypes.c_void_p(0x900000)
    assert lib.fa_probe_copy(None, b, 256, 1, None, ref) == 1
    assert lib.fa_probe_copy(a, b, 0, 1, None, ref) == 2
    assert lib.fa_probe_copy(a, b, 256, 0, None, ref) == 2
    assert lib.fa_probe_copy(a, b, 250, 1, None, ref) == 7          # size not a multiple of 16
    assert lib.fa_probe_copy(ctypes.c_void_p(0x100008), b, 256, 1, None, ref) == 7
    assert lib.fa_probe_copy(a, ctypes.c_void_p(0x100080), 256, 1, None, ref) == 10  # overlap


def test_standard_workspace_and_errors(lib):
    n = 300
    want = (((1 * 2 * n * ((n + 3) // 4 * 4) * 4) + 255) // 256 * 256
            + ((1 * 2 * n * ((n + 7) // 8 * 8) * 2) + 255) // 256 * 256)
    assert lib.fa_fwd_standard_workspace_bytes(1, 2, n, 128, 1) == want
    assert lib.fa_fwd_standard_workspace_bytes(1, 2, n, 128, 0) == 0   # bf16 only
    assert lib.fa_fwd_standard_workspace_bytes(1, 2, 0, 128, 1) == 0
    ws = ctypes.c_void_p(0x4000000)
    def call(ws=ws, wb=1 << 40, dtype=1, d=64, N=8, q=FAKE):
        return lib.fa_fwd_standard(q, FAKE, FAKE, ctypes.c_void_p(0x200000),
                                   ctypes.c_void_p(0x900000), ws, wb, 1, 1, N, d, dtype, 0.125,
                                   0, 0, None)
    assert call(q=None) == 1
    assert call(dtype=0) == 3                 # float32 has no standard path
    assert call(d=96) == 4
    assert call(ws=None) == 8 and call(wb=16) == 8
    assert call(ws=ctypes.c_void_p(0x4000008)) == 7
    assert call(ws=ctypes.c_void_p(0x100000)) == 10   # workspace overlaps q


def test_keymajor_workspace_and_errors(lib):
    # two lanes per query row, 256-row workgroups: 512 * (d/2 + 3) floats each
    assert lib.fa_fwd_keymajor_workspace_bytes(2, 3, 300, 128, 1) == 2 * 3 * 2 * 512 * 67 * 4
    assert lib.fa_fwd_keymajor_workspace_bytes(1, 1, 256, 64, 1) == 512 * 35 * 4
    assert lib.fa_fwd_keymajor_workspace_bytes(1, 1, 256, 64, 0) == 0
    ws = ctypes.c_void_p(0x4000000)
    def call(bc=64, d=64, dtype=1, ws=ws, wb=1 << 30):
        return lib.fa_fwd_keymajor(FAKE, FAKE, FAKE, ctypes.c_void_p(0x200000),
                                   ctypes.c_void_p(0x900000), ws, wb, 1, 1, 8, d, dtype, 0.125,
                                   0, 0, bc, None)
    assert call(bc=48) == 2 and call(bc=256, d=128) == 2 and call(bc=512) == 2
    assert call(dtype=0) == 3
    assert call(ws=None) == 8 and call(wb=100) == 8
    assert call(ws=ctypes.c_void_p(0x4000004)) == 7


def test_tuned_entry_points_reject_unknown_cfg(lib):
    """fa_fwd_tuned / fa_bwd_tuned check cfg before anything else
    (FA_ERR_CONFIG = 11), and a float32 call takes only cfg 0."""
    o, lse = ctypes.c_void_p(0x200000), ctypes.c_void_p(0x900000)
    def tf(cfg, dtype=1, d=64, q=FAKE):
        return lib.fa_fwd_tuned(q, FAKE, FAKE, o, lse, 1, 1, 8, d, dtype, 0.125, 0, 0, cfg, None)
    assert tf(-1) == 11 and tf(10) == 11 and tf(1 << 20) == 11
    assert tf(3, dtype=0, d=8) == 11
    assert tf(0, q=None) == 1 and tf(5, q=None) == 1  # a known cfg goes on to validation
    p = [ctypes.c_void_p(0x100000 * (i + 1)) for i in range(10)]
    def tb(cfg, dtype=1):
        return lib.fa_bwd_tuned(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7], p[8], p[9], 1 << 20,
                                1, 1, 8, 64, dtype, 0.125, 0, 0, cfg, None)
    assert tb(1) == 11 and tb(3) == 11 and tb(2, dtype=0) == 11
    assert _native.fa_status_string(11).startswith("FA_ERR_CONFIG")


def test_window_marshalling():
    """Radii are passed as C ints without wrapping: above 2^31 - 1 they are
    passed as 2^31 - 1 (the same pairs), below -1 as -1 (still rejected)."""
    assert _native._window(0) == 0 and _native._window(128) == 128
    assert _native._window(2 ** 31 - 1) == 2 ** 31 - 1
    assert _native._window(2 ** 31) == 2 ** 31 - 1 and _native._window(2 ** 63) == 2 ** 31 - 1
    assert _native._window(-1) == -1 and _native._window(-(2 ** 32) + 5) == -1


def test_standard_backward_workspace_and_errors(lib):
    assert lib.fa_bwd_standard_workspace_bytes(1, 2, 300, 128, 1) == \
        lib.fa_fwd_standard_workspace_bytes(1, 2, 300, 128, 1)
    assert lib.fa_bwd_standard_workspace_bytes(1, 2, 300, 128, 0) == 0
    need = lib.fa_bwd_standard_workspace_bytes(1, 1, 8, 64, 1)
    f, w = ctypes.c_void_p(0x4000000), ctypes.c_void_p(0x8000000)
    outs = [ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), ctypes.c_void_p(0x400000)]
    def call(fws=f, fb=need, ws=w, wb=need, dtype=1, d=64, q=FAKE, scale=0.125):
        return lib.fa_bwd_standard(q, FAKE, FAKE, FAKE, fws, fb, *outs, ws, wb, 1, 1, 8, d, dtype,
                                   scale, None)
    assert call(q=None) == 1
    assert call(dtype=0) == 3 and call(d=96) == 4
    assert call(fws=None) == 8 and call(fb=need - 1) == 8
    assert call(ws=None) == 8 and call(wb=16) == 8
    assert call(ws=ctypes.c_void_p(0x8000008)) == 7
    assert call(ws=f) == 10                         # the two workspaces overlap
    assert call(scale=float("nan")) == 6
