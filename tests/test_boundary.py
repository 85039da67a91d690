"""The C ABI of libmi_attn, checked without a GPU.

Every call here fails validation (or is the empty no-op), which the library
does before any HIP call, so nothing is launched. The pointers are stand-in
integers that are never dereferenced.
"""

import ctypes
import os
import re

import pytest

import tiled_attention_forward_02_amd as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mi_attn.h")

OK, ERR_NULL, ERR_SHAPE, ERR_HEADDIM, ERR_ALIGN, ERR_ALIAS, ERR_SCALE, ERR_LAUNCH = (
    0, -1, -2, -3, -5, -6, -7, -8)
ERR_DTYPE, ERR_SCRATCH = -9, -10

MIB = 1 << 20
# Stand-in device addresses, 1 MiB apart and 256-byte aligned.
Q, K, V, O, L = (0x7f0000000000 + i * 64 * MIB for i in range(5))


@pytest.fixture(scope="module")
def lib():
    try:
        return mi.load_library()
    except ImportError as e:  # the build step did not run
        pytest.fail(str(e))


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["attn_bwd", "attn_bwd_noalloc", "attn_fwd", "attn_fwd_cross",
                                    "attn_fwd_ex", "attn_fwd_launch_shape", "attn_strerror"]


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_no_extra_exported_c_symbols():
    """Only the header's functions carry C linkage (nm -D of the library)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", mi.lib_path()],
                         capture_output=True, text=True, check=True).stdout
    syms = {line.split()[-1] for line in out.splitlines() if " T " in line}
    c_syms = {s for s in syms if s.startswith("attn_")}
    assert c_syms == set(declared_functions())


def test_strerror_covers_every_status(lib):
    seen = set()
    for code in (OK, ERR_NULL, ERR_SHAPE, ERR_HEADDIM, ERR_ALIGN, ERR_ALIAS,
                 ERR_SCALE, ERR_LAUNCH, ERR_DTYPE, ERR_SCRATCH):
        msg = mi.attn_strerror(code)
        assert msg and msg != "unknown status"
        seen.add(msg)
    assert len(seen) == 10
    assert mi.attn_strerror(12345) == "unknown status"


def call(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, N=100, d=64, scale=0.125,
         causal=0):
    return lib.attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, None)


@pytest.mark.parametrize("which", ["q", "k", "v", "o", "lse"])
def test_null_pointer(lib, which):
    assert call(lib, **{which: None}) == ERR_NULL


@pytest.mark.parametrize("B,H,N", [(-1, 1, 1), (1, -2, 1), (1, 1, -5)])
def test_negative_sizes(lib, B, H, N):
    assert call(lib, B=B, H=H, N=N) == ERR_SHAPE


def test_size_overflow(lib):
    big = 2**31 - 1
    assert call(lib, B=big, H=big, N=big, d=128) == ERR_SHAPE


@pytest.mark.parametrize("d", [0, 1, 16, 31, 63, 65, 95, 97, 127, 129, 255, 512])
def test_unsupported_head_dim(lib, d):
    assert call(lib, d=d) == ERR_HEADDIM


@pytest.mark.parametrize("which,offset", [("q", 8), ("k", 2), ("v", 4), ("o", 12),
                                          ("lse", 2)])
def test_misaligned(lib, which, offset):
    base = {"q": Q, "k": K, "v": V, "o": O, "lse": L}[which]
    assert call(lib, **{which: base + offset}) == ERR_ALIGN


def test_lse_four_byte_alignment_is_enough(lib):
    # lse at +4 passes alignment; o aliasing q then trips the next check,
    # so nothing is launched.
    assert call(lib, lse=L + 4, o=Q) == ERR_ALIAS


@pytest.mark.parametrize("o,lse", [(Q, L), (K + 256, L), (V, L), (O, Q + 16),
                                   (O, O + 64)])
def test_aliasing(lib, o, lse):
    assert call(lib, o=o, lse=lse) == ERR_ALIAS


def test_inputs_may_alias_each_other_but_outputs_not(lib):
    # q == k == v is legal; with o == q the call is rejected before launch.
    assert call(lib, k=Q, v=Q, o=Q) == ERR_ALIAS


@pytest.mark.parametrize("scale", [float("nan"), float("inf"), float("-inf")])
def test_non_finite_scale(lib, scale):
    assert call(lib, scale=scale) == ERR_SCALE


@pytest.mark.parametrize("B,H,N", [(0, 4, 128), (2, 0, 128), (2, 4, 0)])
def test_empty_is_a_no_op(lib, B, H, N):
    # Nothing to compute: success without touching the (null) pointers.
    assert call(lib, q=None, k=None, v=None, o=None, lse=None, B=B, H=H, N=N) == OK


def test_validation_order(lib):
    # size errors come before pointer errors
    assert call(lib, q=None, d=80) == ERR_HEADDIM
    assert call(lib, q=None, N=-1) == ERR_SHAPE


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 1, 128, 64, 0), (4, 16, 1024, 64, 0), (8, 16, 2048, 64, 1),
    (16, 16, 4096, 128, 0), (1, 32, 16384, 128, 1), (2, 3, 1, 64, 0),
    (2, 3, 129, 128, 1), (2, 3, 500, 32, 0), (1, 2, 300, 256, 1), (2, 2, 700, 96, 1)])
def test_launch_shape(lib, B, H, N, d, causal):
    s = mi.attn_fwd_launch_shape(B, H, N, d, causal)
    bm = s["block_m"]
    assert s["grid"] == B * H * ((N + bm - 1) // bm)
    assert s["block"] % 64 == 0 and s["block"] <= 1024
    assert s["block_n"] in (32, 64, 128)
    assert 0 < s["lds_bytes"] <= 160 * 1024


def test_launch_shape_errors(lib):
    with pytest.raises(mi.AttnError):
        mi.attn_fwd_launch_shape(1, 1, 128, 80)
    out = [ctypes.c_int(0) for _ in range(4)]
    assert lib.attn_fwd_launch_shape(1, 1, 128, 64, 0, None,
                                     *[ctypes.byref(x) for x in out]) == ERR_NULL
    assert mi.attn_fwd_launch_shape(0, 1, 128, 64)["grid"] == 0


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):  # CPU tensors never reach the library
        mi.attn_fwd(q, q, q)
    with pytest.raises(TypeError):
        mi.attn_fwd(q.float(), q, q)
    with pytest.raises(TypeError):
        mi.attn_fwd([1], q, q)


# ------------------------------------------------------ attn_fwd_cross --

def cross(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=70, d=128, scale=0.125,
          causal=0):
    return lib.attn_fwd_cross(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, None)


@pytest.mark.parametrize("Nq,Nk", [(-1, 4), (4, -1)])
def test_cross_negative_lengths(lib, Nq, Nk):
    assert cross(lib, Nq=Nq, Nk=Nk) == ERR_SHAPE


@pytest.mark.parametrize("d", [32, 64, 96, 128, 256])
def test_longest_accepted_key_axis(lib, d):
    # One head's keys plus a 128-row tile of slack must stay below 2^31 bytes:
    # the longest such Nk passes the size checks (and then fails on the null
    # q), one more is rejected as a shape error.
    longest = (2**31 - 1 - 128 * d * 2) // (d * 2)
    assert cross(lib, q=None, Nk=longest, d=d) == ERR_NULL
    assert cross(lib, q=None, Nk=longest + 1, d=d) == ERR_SHAPE
    assert cross(lib, q=None, Nq=longest + 1, d=d) == ERR_SHAPE


def test_cross_null_and_empty(lib):
    assert cross(lib, q=None) == ERR_NULL
    assert cross(lib, k=None) == ERR_NULL
    # no keys: k and v may be NULL (every row is empty); still validated, not
    # launched here because o aliases q
    assert cross(lib, k=None, v=None, Nk=0, o=Q) == ERR_ALIAS
    # no queries: nothing to do
    assert cross(lib, q=None, k=None, v=None, o=None, lse=None, Nq=0) == OK


def test_cross_aliasing_uses_each_tensors_size(lib):
    # o (Nq rows) placed right after a k of Nk rows: no overlap -> would launch;
    # placed inside k -> rejected.
    kbytes = 2 * 3 * 70 * 128 * 2
    assert cross(lib, o=K + kbytes - 256) == ERR_ALIAS
    assert cross(lib, lse=V + 4) == ERR_ALIAS


def test_cross_headdim_and_scale(lib):
    assert cross(lib, d=80) == ERR_HEADDIM
    assert cross(lib, scale=float("nan")) == ERR_SCALE


# ---------------------------------------------------------- attn_fwd_ex --

def ex(lib, dtype=0, d=128, **kw):
    args = dict(q=Q, k=K, v=V, o=O, lse=L, B=2, H=3, Nq=100, Nk=70, scale=0.125, causal=0)
    args.update(kw)
    return lib.attn_fwd_ex(args["q"], args["k"], args["v"], args["o"], args["lse"], args["B"],
                           args["H"], args["Nq"], args["Nk"], d, dtype, args["scale"],
                           args["causal"], None)


@pytest.mark.parametrize("dtype", [-1, 2, 7])
def test_ex_rejects_unknown_dtype(lib, dtype):
    assert ex(lib, dtype=dtype) == ERR_DTYPE


@pytest.mark.parametrize("dtype", [0, 1])
def test_ex_validates_like_the_others(lib, dtype):
    assert ex(lib, dtype=dtype, d=80) == ERR_HEADDIM
    assert ex(lib, dtype=dtype, q=None) == ERR_NULL
    assert ex(lib, dtype=dtype, o=Q) == ERR_ALIAS
    assert ex(lib, dtype=dtype, Nq=0, q=None, o=None, lse=None) == OK


def test_binding_dtype_rules():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.float16)
    with pytest.raises(TypeError):  # attn_fwd is bf16 only
        mi.attn_fwd(q, q, q)
    with pytest.raises(TypeError):  # mixed dtypes
        mi.attn_fwd_ex(q, q.to(torch.bfloat16), q)


# -------------------------------------------------------------- attn_bwd --
# Fake, distinct, 16-byte aligned device addresses: validation happens before
# any HIP call, so none of these is ever dereferenced.
BQ_, BK_, BV_, BO_, BL_, BDO_, BDQ_, BDK_, BDV_, BDL_ = (0x100000 * (i + 1) for i in range(10))


def bwd(lib, d=128, dtype=0, B=2, H=3, Nq=100, Nk=70, scale=0.125, causal=0, **ptrs):
    p = dict(q=BQ_, k=BK_, v=BV_, o=BO_, lse=BL_, do=BDO_, dq=BDQ_, dk=BDK_, dv=BDV_, delta=BDL_)
    p.update(ptrs)
    return lib.attn_bwd(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"], p["dk"],
                        p["dv"], p["delta"], B, H, Nq, Nk, d, dtype, scale, causal, None)


@pytest.mark.parametrize("d", [0, 16, 48, 80, 255, 512])
def test_bwd_head_dims(lib, d):
    assert bwd(lib, d=d) == ERR_HEADDIM


def test_bwd_rejects_bad_arguments(lib):
    assert bwd(lib, dtype=2) == ERR_DTYPE
    assert bwd(lib, scale=float("nan")) == ERR_SCALE
    assert bwd(lib, Nq=-1) == ERR_SHAPE
    assert bwd(lib, Nq=1 << 30) == ERR_SHAPE
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv", "delta"):
        assert bwd(lib, **{name: None}) == ERR_NULL, name
    assert bwd(lib, dk=BDQ_) == ERR_ALIAS      # two outputs on one buffer
    assert bwd(lib, dv=BV_) == ERR_ALIAS       # output over an input
    assert bwd(lib, delta=BL_) == ERR_ALIAS
    assert bwd(lib, dq=BQ_ + 8) == ERR_ALIGN
    assert bwd(lib, delta=BDL_ + 2) == ERR_ALIGN


def test_bwd_empty_sides(lib):
    # nothing to do: no launch, OK even with every pointer NULL
    assert bwd(lib, B=0) == OK
    assert bwd(lib, Nq=0, Nk=0, **{n: None for n in ("q", "k", "v", "o", "lse", "do", "dq",
                                                      "dk", "dv", "delta")}) == OK
    # a side with no rows may pass NULL for its own tensors (validation only here)
    assert bwd(lib, Nq=0, q=None, o=None, lse=None, do=None, dq=None, delta=None,
               k=None) == ERR_NULL
    assert bwd(lib, Nk=0, k=None, v=None, dk=None, dv=None, q=None) == ERR_NULL


def bwd_noalloc(lib, d=128, dtype=0, B=2, H=3, Nq=100, Nk=70, scale=0.125, causal=0,
                **ptrs):
    p = dict(q=BQ_, k=BK_, v=BV_, o=BO_, lse=BL_, do=BDO_, dq=BDQ_, dk=BDK_, dv=BDV_)
    p.update(ptrs)
    return lib.attn_bwd_noalloc(p["q"], p["k"], p["v"], p["o"], p["lse"], p["do"], p["dq"],
                                p["dk"], p["dv"], B, H, Nq, Nk, d, dtype, scale, causal, None)


def test_bwd_noalloc_validates_like_attn_bwd(lib):
    """Every argument check of attn_bwd, without the delta argument; all of
    them come before the one-time lookup of the static buffer."""
    for d in (0, 16, 257):
        assert bwd_noalloc(lib, d=d) == ERR_HEADDIM
    assert bwd_noalloc(lib, dtype=2) == ERR_DTYPE
    assert bwd_noalloc(lib, scale=float("inf")) == ERR_SCALE
    assert bwd_noalloc(lib, Nk=-1) == ERR_SHAPE
    for name in ("q", "k", "v", "o", "lse", "do", "dq", "dk", "dv"):
        assert bwd_noalloc(lib, **{name: None}) == ERR_NULL, name
    assert bwd_noalloc(lib, dk=BDQ_) == ERR_ALIAS
    assert bwd_noalloc(lib, dq=BO_) == ERR_ALIAS
    assert bwd_noalloc(lib, dv=BDV_ + 4) == ERR_ALIGN
    assert bwd_noalloc(lib, lse=BL_ + 2) == ERR_ALIGN
    assert bwd_noalloc(lib, B=0) == OK
    assert bwd_noalloc(lib, Nq=0, Nk=0, **{n: None for n in ("q", "k", "v", "o", "lse", "do",
                                                             "dq", "dk", "dv")}) == OK


@pytest.mark.parametrize("B,H,Nq", [(1, 1, 4194305), (16, 16, 16385), (64, 64, 1025)])
def test_bwd_noalloc_rejects_more_rows_than_its_buffer(lib, B, H, Nq):
    """B*H*Nq beyond 4194304 rows (the static buffer's 16 MiB of floats) is
    refused before anything else is looked at; exactly the limit passes that
    check (and then fails on a NULL pointer here)."""
    assert bwd_noalloc(lib, B=B, H=H, Nq=Nq, d=64) == ERR_SCRATCH
    assert bwd_noalloc(lib, B=B, H=H, Nq=Nq, d=64, q=None) == ERR_SCRATCH
    assert bwd_noalloc(lib, B=1, H=1, Nq=4194304, d=64, q=None) == ERR_NULL


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """Without libmi_attn.so every entry point raises; nothing falls back."""
    import torch
    monkeypatch.setattr(mi, "_LIB_PATH", str(tmp_path / "libmi_attn.so"))
    monkeypatch.setattr(mi, "_lib", None)
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ImportError):
        mi.load_library()
    for call in (lambda: mi.attn_fwd(q, q, q), lambda: mi.attn_fwd_cross(q, q, q),
                 lambda: mi.attn_fwd_ex(q, q, q),
                 lambda: mi.attn_bwd(q, q, q, q, torch.zeros(1, 1, 8), q),
                 lambda: mi.attn_strerror(0), lambda: mi.attn_fwd_launch_shape(1, 1, 8, 64)):
        with pytest.raises(ImportError):
            call()


@pytest.mark.parametrize("B,H,N,rows", [(16, 16, 4096, 512), (1, 32, 16384, 512),
                                        (2, 16, 4096, 256), (4, 16, 1024, 128),
                                        (1, 1, 128, 128)])
def test_launch_shape_d128_follows_the_grid(lib, B, H, N, rows):
    # d = 128 takes the biggest workgroup (512, 256 or 128 query rows) whose grid
    # still gives each of the 256 CUs two workgroups' worth of rows
    s = mi.attn_fwd_launch_shape(B, H, N, 128, False)
    assert s["block_m"] == rows
    assert s["block"] == (512 if rows == 512 else 256)
    assert s["grid"] == B * H * ((N + rows - 1) // rows)


@pytest.mark.parametrize("B,H,N,rows", [(16, 16, 4096, 512), (1, 32, 16384, 512),
                                        (4, 16, 4100, 512), (2, 16, 4096, 128),
                                        (8, 16, 2048, 128), (4, 16, 1024, 128),
                                        (64, 16, 4095, 128)])
def test_launch_shape_d64_follows_the_grid_and_the_rows(lib, B, H, N, rows):
    # d = 64 takes the 512-row workgroups (eight waves, 48 KiB of LDS) only when
    # both axes have at least 4096 rows and the grid gives every CU two of them
    s = mi.attn_fwd_launch_shape(B, H, N, 64, True)
    assert s["block_m"] == rows
    assert s["block"] == (512 if rows == 512 else 256)
    assert s["block_n"] == 64
    assert s["grid"] == B * H * ((N + rows - 1) // rows)
    if rows == 512:
        assert s["lds_bytes"] == 3 * 2 * 8192


@pytest.mark.parametrize("B,H,N,rows", [(16, 16, 4096, 256), (1, 32, 16384, 256),
                                        (4, 16, 4000, 256), (2, 16, 4000, 128),
                                        (4, 16, 1024, 128)])
def test_launch_shape_d32_follows_the_grid(lib, B, H, N, rows):
    # d = 32 takes eight-wave, 256-row workgroups when the grid gives two full
    # rounds of two per CU, else four-wave, 128-row ones
    s = mi.attn_fwd_launch_shape(B, H, N, 32, True)
    assert s["block_m"] == rows
    assert s["block"] == (512 if rows == 256 else 256)
    assert s["grid"] == B * H * ((N + rows - 1) // rows)


@pytest.mark.parametrize("B,H,N,rows", [(16, 16, 4096, 512), (1, 32, 16384, 512),
                                        (4, 16, 4000, 512), (2, 16, 4000, 128),
                                        (4, 16, 1024, 128)])
def test_launch_shape_d96_follows_the_grid(lib, B, H, N, rows):
    # d = 96 takes the ping-pong kernel's 512-row workgroups (two blocks a
    # wave, eight waves, 48 KiB of LDS) when the grid gives every CU two of
    # them, else four-wave, 128-row ones
    s = mi.attn_fwd_launch_shape(B, H, N, 96, True)
    assert s["block_m"] == rows
    assert s["block"] == (512 if rows == 512 else 256)
    assert s["grid"] == B * H * ((N + rows - 1) // rows)
    if rows == 512:
        assert s["lds_bytes"] == 3 * 2 * 8192


@pytest.mark.parametrize("B,H,N,rows", [(16, 16, 4096, 256), (1, 32, 16384, 256),
                                        (2, 16, 4000, 256), (1, 16, 4000, 128)])
def test_launch_shape_d256_follows_the_grid(lib, B, H, N, rows):
    # d = 256 takes eight-wave, 256-row workgroups when the grid gives two full
    # rounds of one per CU, else four-wave, 128-row ones
    s = mi.attn_fwd_launch_shape(B, H, N, 256, False)
    assert s["block_m"] == rows
    assert s["block"] == (512 if rows == 256 else 256)
    assert s["grid"] == B * H * ((N + rows - 1) // rows)
    if rows == 256:  # the ping-pong kernel: three stages of 16 KiB of K and 16 of V
        assert s["lds_bytes"] == 3 * 2 * 16384
