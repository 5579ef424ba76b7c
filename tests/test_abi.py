"""The C ABI library: it loads, exports what the header declares, and its host-side
validation returns the documented status codes before any HIP call (CPU only)."""

import ctypes
import os
import re

import pytest

from shifted_sparse_attention_s2attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s2attn.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(s2attn_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_the_abi():
    assert header_functions() == sorted(_lib.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_status_strings(lib):
    for code in range(8):
        assert lib.s2attn_status_str(code)
    assert lib.s2attn_status_str(99) == b"unknown status"


DUMMY = ctypes.c_void_p(0x1000)   # never dereferenced: validation rejects before any HIP call
FDUMMY = ctypes.cast(DUMMY, ctypes.POINTER(ctypes.c_float))
GOOD = dict(B=1, H=4, Hkv=4, N=512, d=64, G=128, S=2, dtype=0)


def fwd_status(lib, ptrs=True, **kw):
    p = dict(GOOD)
    p.update(kw)
    ptr = DUMMY if ptrs else None
    return lib.s2attn_fwd(ptr, ptr, ptr, ptr, FDUMMY if ptrs else None,
                          p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"], p["dtype"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(G=1024), _lib.S2ATTN_ERR_SHAPE),         # G > N
    (dict(G=0), _lib.S2ATTN_ERR_SHAPE),
    (dict(S=5), _lib.S2ATTN_ERR_SHAPE),
    (dict(S=-1), _lib.S2ATTN_ERR_SHAPE),
    (dict(Hkv=3), _lib.S2ATTN_ERR_SHAPE),
    (dict(B=-1), _lib.S2ATTN_ERR_SHAPE),
    (dict(N=-128), _lib.S2ATTN_ERR_SHAPE),
    (dict(H=0, Hkv=0), _lib.S2ATTN_ERR_SHAPE),
    (dict(d=96), _lib.S2ATTN_ERR_UNSUPPORTED),
    (dict(dtype=7), _lib.S2ATTN_ERR_UNSUPPORTED),
])
def test_fwd_rejects(lib, kw, code):
    assert fwd_status(lib, **kw) == code


def test_fwd_null_pointer(lib):
    assert fwd_status(lib, ptrs=False) == _lib.S2ATTN_ERR_NULL


@pytest.mark.parametrize("kw", [dict(B=0), dict(N=0), dict(B=0, N=0)])
def test_empty_problem_is_a_no_op(lib, kw):
    """B == 0 or N == 0: every entry point validates the other sizes and returns
    OK without reading a pointer (all NULL here) or calling HIP; no workspace."""
    p = dict(GOOD)
    p.update(kw)
    dims = [p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"], p["dtype"], None]
    assert fwd_status(lib, ptrs=False, **kw) == _lib.S2ATTN_OK
    assert lib.s2attn_bwd_workspace_bytes(*dims[:-1]) == 0
    assert lib.s2attn_bwd(*([None] * 10), 0, *dims) == _lib.S2ATTN_OK
    assert lib.s2attn_bwd_prep(None, None, None, None, 0, *dims) == _lib.S2ATTN_OK
    assert lib.s2attn_bwd_dkdv(*([None] * 7), 0, *dims) == _lib.S2ATTN_OK
    assert lib.s2attn_bwd_dq(*([None] * 6), 0, *dims) == _lib.S2ATTN_OK
    assert lib.s2attn_bwd_prep_dq(*([None] * 8), 0, *dims[:7], 0, *dims[7:]) == _lib.S2ATTN_OK
    # the other sizes are still checked
    assert fwd_status(lib, ptrs=False, d=96, **kw) == _lib.S2ATTN_ERR_UNSUPPORTED
    assert fwd_status(lib, ptrs=False, S=9, **kw) == _lib.S2ATTN_ERR_SHAPE


def test_grid_size_limit(lib):
    """Grids are one-dimensional over (batch, head, 128-row tile): B and H may be
    large as long as B * H * N / 128 stays below 2^31."""
    assert lib.s2attn_bwd_workspace_bytes(70000, 1, 1, 128, 64, 128, 0, 0) == 70000 * 128 * 4 * 2
    assert fwd_status(lib, B=1 << 20, H=1 << 10, Hkv=1 << 10, S=0, N=256) == _lib.S2ATTN_ERR_UNSUPPORTED


def test_noalloc_scratch_limit(lib):
    """s2attn_bwd_noalloc keeps its row sums in a fixed device array of
    S2ATTN_NOALLOC_MAX_ROWS rows: larger problems are rejected after the size
    checks and before the pointers or any HIP call (NULL pointers here)."""
    text = open(HEADER).read()
    assert re.search(r"#define S2ATTN_NOALLOC_MAX_ROWS \(1 << 22\)", text)
    assert _lib.S2ATTN_NOALLOC_MAX_ROWS == 1 << 22
    rows = _lib.S2ATTN_NOALLOC_MAX_ROWS

    def call(B, H, N, G=128, d=64, S=0, wrap=0):
        return lib.s2attn_bwd_noalloc(*([None] * 9), B, H, H, N, d, G, S, wrap, 0, None)

    assert call(1, 32, rows // 32) == _lib.S2ATTN_ERR_NULL                 # at the limit: only pointers left
    assert call(1, 32, rows // 32 + 128) == _lib.S2ATTN_ERR_SCRATCH
    assert call(2, 64, 32768) == _lib.S2ATTN_ERR_NULL                      # B * H * N = 2^22 exactly
    assert call(2, 64, 32768 + 128) == _lib.S2ATTN_ERR_SCRATCH
    assert call(1, 4, 512, G=1024) == _lib.S2ATTN_ERR_SHAPE                # size errors come first
    assert call(1, 4, 512, wrap=5) == _lib.S2ATTN_ERR_UNSUPPORTED
    assert call(0, 4, 512) == _lib.S2ATTN_OK                               # empty problem: a no-op
    assert lib.s2attn_status_str(_lib.S2ATTN_ERR_SCRATCH).startswith(b"the problem does not fit")


def test_fused_rope_validation(lib):
    """s2attn_fwd_rope / s2attn_bwd_rope: bf16 only, rotary parameters as
    s2attn_rope, checked after the sizes and before the pointers (NULL here)."""
    p = dict(GOOD)
    dims = [p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"]]
    need = lib.s2attn_bwd_workspace_bytes(*dims, 0)

    def fwd(scale=1.0, base=1e4, dtype=0, wrap=0, dd=dims):
        return lib.s2attn_fwd_rope(*([None] * 4), None, None, *dd, wrap, scale, base, dtype, None)

    def bwd(scale=1.0, base=1e4, dtype=0, wrap=0, dd=dims):
        return lib.s2attn_bwd_rope(*([None] * 4), None, *([None] * 5), need, *dd, wrap, scale, base, dtype, None)

    for f in (fwd, bwd):
        assert f() == _lib.S2ATTN_ERR_NULL
        assert f(dtype=_lib.S2ATTN_F32) == _lib.S2ATTN_ERR_UNSUPPORTED
        assert f(scale=-1.0) == _lib.S2ATTN_ERR_UNSUPPORTED
        assert f(scale=float("nan")) == _lib.S2ATTN_ERR_UNSUPPORTED
        assert f(base=1.0) == _lib.S2ATTN_ERR_UNSUPPORTED
        assert f(wrap=9) == _lib.S2ATTN_ERR_UNSUPPORTED
        assert f(dd=[dims[0], dims[1], dims[2], 64] + dims[4:]) == _lib.S2ATTN_ERR_SHAPE   # G > N
        assert f(scale=0.0) == _lib.S2ATTN_ERR_NULL                                        # identity rotation: valid
        assert f(dd=[0] + dims[1:]) == _lib.S2ATTN_OK                                       # empty problem


def test_row_width_limit(lib):
    """A 64-row tile is addressed with 32-bit byte offsets from its first row, so
    one token row of q (H * d elements) must stay below 2^24 elements."""
    assert fwd_status(lib, ptrs=False, B=1, H=1 << 17, Hkv=1, S=0, d=128, N=256) == _lib.S2ATTN_ERR_UNSUPPORTED
    assert fwd_status(lib, ptrs=False, B=1, H=(1 << 17) - 1, Hkv=1, S=0, d=128, N=256) == _lib.S2ATTN_ERR_NULL


def test_unaligned_group_sizes_pass_validation(lib):
    """G need not divide N, nor be a multiple of 128 (EDGE instantiations): only the
    pointers are left to reject (NULL here)."""
    for kw in (dict(N=500), dict(G=129, N=129 * 4), dict(G=64, N=512), dict(G=1365, N=8192), dict(G=1, N=7),
               dict(G=512, N=512)):
        assert fwd_status(lib, ptrs=False, **kw) == _lib.S2ATTN_ERR_NULL, kw
    # workspace of a short last group: still one fp32 row sum and one lse2 per row
    assert lib.s2attn_bwd_workspace_bytes(1, 4, 4, 500, 64, 128, 2, 0) == 2 * ((4 * 500 * 4 + 255) // 256 * 256)


def test_wrap_option_validation(lib):
    """The _ex calls take wrap in {ROLL, SPLIT, SWAP}; anything else is
    unsupported, checked after the sizes and before the pointers."""
    p = dict(GOOD)
    dims = [p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"]]
    need = lib.s2attn_bwd_workspace_bytes(*dims, 0)
    for wrap, code in ((3, _lib.S2ATTN_ERR_UNSUPPORTED), (-1, _lib.S2ATTN_ERR_UNSUPPORTED),
                       (_lib.S2ATTN_WRAP_SPLIT, _lib.S2ATTN_ERR_NULL), (_lib.S2ATTN_WRAP_SWAP, _lib.S2ATTN_ERR_NULL),
                       (_lib.S2ATTN_WRAP_ROLL, _lib.S2ATTN_ERR_NULL)):
        assert lib.s2attn_fwd_ex(None, None, None, None, None, *dims, wrap, 0, None) == code
        assert lib.s2attn_bwd_ex(*([None] * 10), need, *dims, wrap, 0, None) == code
        assert lib.s2attn_bwd_dkdv_ex(*([None] * 7), need, *dims, wrap, 0, None) == code
        assert lib.s2attn_bwd_dq_ex(*([None] * 6), need, *dims, wrap, 0, None) == code
    bad = list(dims)
    bad[3] = 64                                          # shape errors come first (G > N)
    assert lib.s2attn_fwd_ex(None, None, None, None, None, *bad, 7, 0, None) == _lib.S2ATTN_ERR_SHAPE
    unaligned = list(dims)
    unaligned[3] = 500                                   # split and swap take any shape
    for wrap in (_lib.S2ATTN_WRAP_SPLIT, _lib.S2ATTN_WRAP_SWAP):
        assert lib.s2attn_fwd_ex(None, None, None, None, None, *unaligned, wrap, 0, None) == _lib.S2ATTN_ERR_NULL
        assert lib.s2attn_bwd_ex(*([None] * 10), need, *unaligned, wrap, 0, None) == _lib.S2ATTN_ERR_NULL
    assert lib.s2attn_fwd_ex(None, None, None, None, None, *unaligned, _lib.S2ATTN_WRAP_ROLL, 0, None) == \
        _lib.S2ATTN_ERR_NULL
    empty = list(dims)
    empty[0] = 0                                         # empty problem: validated, then a no-op
    assert lib.s2attn_fwd_ex(None, None, None, None, None, *empty, _lib.S2ATTN_WRAP_SPLIT, 0, None) == _lib.S2ATTN_OK
    assert lib.s2attn_fwd_ex(None, None, None, None, None, *empty, 9, 0, None) == _lib.S2ATTN_ERR_UNSUPPORTED


def test_mixed_shift_workspace(lib):
    """A key/value head read by shifted and unshifted query heads (H=6, Hkv=2,
    the last two heads shifted: key/value head 1 serves query heads 3..5, of
    which 3 is unshifted).  Where both frames cut the keys
    into the same 128-row tiles (whole groups, G a multiple of 256) one dK/dV
    pass serves; otherwise dK/dV takes two passes and the workspace also holds
    the first pass's fp32 dK and dV, 2 * B * N * Hkv * d floats."""
    up = lambda n: -(-n // 256) * 256                      # each array starts 256-byte aligned
    rows = lambda B, H, N: 2 * up(B * H * N * 4)
    assert lib.s2attn_bwd_workspace_bytes(1, 6, 2, 1024, 64, 256, 2, 0) == rows(1, 6, 1024)
    for N, G in ((1024, 128), (640, 256), (1000, 300), (512, 384)):
        assert lib.s2attn_bwd_workspace_bytes(1, 6, 2, N, 64, G, 2, 0) == rows(1, 6, N) + up(2 * N * 2 * 64 * 4), (N, G)
    # no mixed head (every pair of query heads shifted alike), or MHA: one pass
    assert lib.s2attn_bwd_workspace_bytes(1, 6, 2, 1024, 64, 128, 3, 0) == rows(1, 6, 1024)
    assert lib.s2attn_bwd_workspace_bytes(1, 6, 6, 1024, 64, 128, 1, 0) == rows(1, 6, 1024)
    assert fwd_status(lib, ptrs=False, H=6, Hkv=2, S=2, G=128, N=512) == _lib.S2ATTN_ERR_NULL   # shape accepted
    # the noalloc backward holds the first pass's sums in its scratch array where
    # they fit (32 MiB with the row sums; the sums take 2 * N * Hkv * d floats)
    call = lambda N, G, d: lib.s2attn_bwd_noalloc(*([None] * 9), 1, 6, 2, N, d, G, 2, 0, 0, None)
    assert call(1024, 256, 64) == _lib.S2ATTN_ERR_NULL and call(1024, 128, 64) == _lib.S2ATTN_ERR_NULL
    assert call(8192, 128, 128) == _lib.S2ATTN_ERR_NULL                # 16.8 MB of sums
    assert call(16384, 128, 128) == _lib.S2ATTN_ERR_SCRATCH            # 33.6 MB of sums
    assert call(32768, 256, 128) == _lib.S2ATTN_ERR_NULL              # one pass: the row sums only


def test_workspace_size(lib):
    B, H, Hkv, N, d, G, S = 1, 32, 32, 32768, 128, 8192, 16
    n = lib.s2attn_bwd_workspace_bytes(B, H, Hkv, N, d, G, S, 0)
    assert n == 2 * B * H * N * 4
    assert lib.s2attn_bwd_workspace_bytes(B, H, Hkv, N, 96, G, S, 0) == 0


def test_bwd_workspace_checks(lib):
    p = GOOD
    need = lib.s2attn_bwd_workspace_bytes(p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"], 0)
    args = [DUMMY] * 4 + [FDUMMY] + [DUMMY] * 4
    dims = [p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"], 0, None]
    assert lib.s2attn_bwd(*args, DUMMY, need - 1, *dims) == _lib.S2ATTN_ERR_WORKSPACE
    assert lib.s2attn_bwd(*args, None, need, *dims) == _lib.S2ATTN_ERR_WORKSPACE
    assert lib.s2attn_bwd(*args, ctypes.c_void_p(0x1010), need, *dims) == _lib.S2ATTN_ERR_WORKSPACE
    bad = list(args)
    bad[6] = None
    assert lib.s2attn_bwd(*bad, DUMMY, need, *dims) == _lib.S2ATTN_ERR_NULL
    dims_bad = list(dims)
    dims_bad[3] = 64                   # G > N
    assert lib.s2attn_bwd(*args, DUMMY, need, *dims_bad) == _lib.S2ATTN_ERR_SHAPE


def test_product_path_has_no_oracle_or_fallback():
    """The package never imports the oracle and has no non-HIP compute path."""
    pkg = os.path.join(ROOT, "shifted_sparse_attention_s2attn_amd")
    for name in os.listdir(pkg):
        if name.endswith(".py"):
            src = open(os.path.join(pkg, name)).read()
            assert not re.search(r"^\s*(from|import)\s+oracle|s2attn_oracle", src, flags=re.M), name
            assert "scaled_dot_product_attention" not in src, name


def test_bwd_stage_entry_points_validate(lib):
    p = GOOD
    need = lib.s2attn_bwd_workspace_bytes(p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"], 0)
    dims = [p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"], 0, None]
    bad_n = list(dims)
    bad_n[3] = 64                      # G > N
    # prep(o, lse, dO, ws, bytes, ...)
    assert lib.s2attn_bwd_prep(DUMMY, None, DUMMY, DUMMY, need, *dims) == _lib.S2ATTN_ERR_NULL
    assert lib.s2attn_bwd_prep(DUMMY, FDUMMY, DUMMY, DUMMY, need - 4, *dims) == _lib.S2ATTN_ERR_WORKSPACE
    assert lib.s2attn_bwd_prep(DUMMY, FDUMMY, DUMMY, DUMMY, need, *bad_n) == _lib.S2ATTN_ERR_SHAPE
    # dkdv(q, k, v, dO, dk, dv, ws, bytes, ...)
    assert lib.s2attn_bwd_dkdv(DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, DUMMY, need, *dims) == _lib.S2ATTN_ERR_NULL
    assert lib.s2attn_bwd_dkdv(*([DUMMY] * 7), need, *bad_n) == _lib.S2ATTN_ERR_SHAPE
    assert lib.s2attn_bwd_dkdv(*([DUMMY] * 6), None, need, *dims) == _lib.S2ATTN_ERR_WORKSPACE
    # dq(q, k, v, dO, dq, ws, bytes, ...)
    assert lib.s2attn_bwd_dq(DUMMY, DUMMY, DUMMY, DUMMY, None, DUMMY, need, *dims) == _lib.S2ATTN_ERR_NULL
    d96 = list(dims)
    d96[4] = 96
    assert lib.s2attn_bwd_dq(*([DUMMY] * 6), need, *d96) == _lib.S2ATTN_ERR_UNSUPPORTED
    # prep_dq(q, k, v, o, lse, dO, dq, ws, bytes, ..., shift_heads, wrap, dtype, stream)
    pd = [DUMMY, DUMMY, DUMMY, DUMMY, FDUMMY, DUMMY, DUMMY]
    sz = dims[:7]
    assert lib.s2attn_bwd_prep_dq(*pd[:4], None, *pd[5:], DUMMY, need, *sz, 0, 0, None) == _lib.S2ATTN_ERR_NULL
    assert lib.s2attn_bwd_prep_dq(*pd, DUMMY, need - 4, *sz, 0, 0, None) == _lib.S2ATTN_ERR_WORKSPACE
    assert lib.s2attn_bwd_prep_dq(*pd, DUMMY, need, *bad_n[:7], 0, 0, None) == _lib.S2ATTN_ERR_SHAPE
    assert lib.s2attn_bwd_prep_dq(*pd, DUMMY, need, *sz, 3, 0, None) == _lib.S2ATTN_ERR_UNSUPPORTED


def test_misaligned_pointers_rejected(lib):
    """Element tensors need 16-byte alignment (16-byte vector accesses), lse 4:
    every entry point returns S2ATTN_ERR_ALIGN before any HIP call."""
    E = _lib
    odd = ctypes.c_void_p(0x1008)
    fodd = ctypes.cast(ctypes.c_void_p(0x1002), ctypes.POINTER(ctypes.c_float))
    p = GOOD
    sz = [p["B"], p["H"], p["Hkv"], p["N"], p["d"], p["G"], p["S"]]
    dims = sz + [0, None]
    need = lib.s2attn_bwd_workspace_bytes(*sz, 0)
    assert lib.s2attn_fwd(odd, DUMMY, DUMMY, DUMMY, FDUMMY, *dims) == E.S2ATTN_ERR_ALIGN
    assert lib.s2attn_fwd(DUMMY, DUMMY, DUMMY, odd, FDUMMY, *dims) == E.S2ATTN_ERR_ALIGN
    assert lib.s2attn_fwd(DUMMY, DUMMY, DUMMY, DUMMY, fodd, *dims) == E.S2ATTN_ERR_ALIGN
    for i in range(9):      # q, k, v, o, lse, dO, dq, dk, dv in turn
        ptrs = [DUMMY, DUMMY, DUMMY, DUMMY, FDUMMY, DUMMY, DUMMY, DUMMY, DUMMY]
        ptrs[i] = fodd if i == 4 else odd
        assert lib.s2attn_bwd(*ptrs, DUMMY, need, *dims) == E.S2ATTN_ERR_ALIGN, i
    assert lib.s2attn_bwd_prep(odd, FDUMMY, DUMMY, DUMMY, need, *dims) == E.S2ATTN_ERR_ALIGN
    assert lib.s2attn_bwd_dkdv(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, odd, DUMMY, need, *dims) == E.S2ATTN_ERR_ALIGN
    assert lib.s2attn_bwd_dq(DUMMY, odd, DUMMY, DUMMY, DUMMY, DUMMY, need, *dims) == E.S2ATTN_ERR_ALIGN
    assert lib.s2attn_bwd_prep_dq(DUMMY, DUMMY, DUMMY, DUMMY, fodd, DUMMY, DUMMY, DUMMY, need, *sz, 0, 0,
                                  None) == E.S2ATTN_ERR_ALIGN
    assert lib.s2attn_rope(DUMMY, odd, 1, 64, 2, 128, 0.125, 10000.0, 0, 0, None) == E.S2ATTN_ERR_ALIGN


def test_header_is_plain_c():
    """include/s2attn.h compiles as C11 on its own (no C++ or HIP types)."""
    import subprocess
    r = subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_client_builds_and_links(lib, tmp_path):
    """tests/c_abi_client.c builds with gcc against the header and links to
    libs2attn.so; run without arguments it prints its usage and exits 1 before
    any HIP call."""
    import subprocess
    from build_client import build_client
    exe = build_client(str(tmp_path / "c_abi_client"))
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 1 and "usage" in r.stderr, (r.returncode, r.stderr)


def test_binding_validates_tensors_before_any_call():
    """The binding passes raw pointers, so it checks shapes, dtypes, devices and
    contiguity first (CPU tensors are rejected before the library is used)."""
    import torch
    from shifted_sparse_attention_s2attn_amd import s2attn_bwd, s2attn_fwd
    q = torch.zeros(1, 256, 4, 64, dtype=torch.bfloat16)
    k = torch.zeros(1, 256, 2, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        s2attn_fwd(q, k, k, 128, 2)
    with pytest.raises(ValueError, match="bad shapes"):
        s2attn_fwd(q, torch.zeros(1, 128, 2, 64, dtype=torch.bfloat16), k, 128, 2)
    with pytest.raises(TypeError):
        s2attn_fwd(q, k.float(), k, 128, 2)
    with pytest.raises(ValueError, match="GPU tensor"):
        s2attn_bwd(q, k, k, q, torch.zeros(1, 4, 256), q, 128, 2)


def test_rope_validation(lib):
    """s2attn_rope checks sizes, then options, then pointers, before any HIP call."""
    E = _lib
    args = dict(B=1, N=64, Hx=2, d=128, scale=0.125, base=10000.0, inv=0, dtype=0)

    def call(x=None, y=None, **kw):
        a = dict(args, **kw)
        return lib.s2attn_rope(x, y, a["B"], a["N"], a["Hx"], a["d"], a["scale"], a["base"], a["inv"], a["dtype"], None)

    assert call() == E.S2ATTN_ERR_NULL
    assert call(B=-1) == E.S2ATTN_ERR_SHAPE and call(Hx=0) == E.S2ATTN_ERR_SHAPE and call(d=0) == E.S2ATTN_ERR_SHAPE
    assert call(d=96) == E.S2ATTN_ERR_UNSUPPORTED and call(dtype=7) == E.S2ATTN_ERR_UNSUPPORTED
    for bad in (dict(scale=-1.0), dict(scale=float("nan")), dict(base=1.0), dict(base=float("inf")), dict(inv=2)):
        assert call(**bad) == E.S2ATTN_ERR_UNSUPPORTED, bad
    assert call(B=0) == E.S2ATTN_OK and call(N=0) == E.S2ATTN_OK    # empty: a no-op
    assert call(scale=0.0, inv=1) == E.S2ATTN_ERR_NULL                  # valid options, NULL pointers
