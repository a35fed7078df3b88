"""CPU tests of the C ABI: the library loads, exports every declared symbol, and
rejects invalid arguments before touching a device (no compute calls here)."""

import ctypes
import math
import os
import re
import subprocess
import sys

import pytest

import dense_attention_amd as da

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(da.library_path()):
        from dense_attention_amd import build
        build.build()
    return da.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["attn_fwd", "attn_fwd_ex", "attn_get_config", "attn_variant_count",
              "attn_variant_info", "attn_strerror", "attn_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", da.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (attn_\w+)", out))
    assert set(declared_functions()) <= exported


def test_library_is_gfx950_code_object(lib):
    data = open(da.library_path(), "rb").read()
    assert b"gfx950" in data


def _call(lib, q=0x1000, k=0x2000, v=0x3000, o=0x4000, lse=None, B=1, H=1, S=16, D=64,
          scale=0.125, dtype=1, opts=None):
    if opts is None:
        return lib.attn_fwd(q, k, v, o, lse, B, H, S, D, scale, dtype, None)
    return lib.attn_fwd_ex(q, k, v, o, lse, B, H, S, D, scale, dtype, None, ctypes.byref(opts))


def test_rejects_bad_dtype(lib):
    assert _call(lib, dtype=2) == -2
    assert _call(lib, dtype=-1) == -2


def test_rejects_bad_shapes(lib):
    assert _call(lib, S=-1) == -3
    assert _call(lib, B=-2) == -3
    assert _call(lib, D=96) == -3
    assert _call(lib, D=0) == -3
    assert _call(lib, S=1 << 30, D=128) == -3          # key index beyond 2^30
    assert _call(lib, B=1 << 12, H=1 << 12, S=1 << 8) == -3


def test_rejects_non_finite_scale(lib):
    assert _call(lib, scale=float("nan")) == -5
    assert _call(lib, scale=float("inf")) == -5


def test_empty_problem_is_ok_without_pointers(lib):
    assert _call(lib, q=None, k=None, v=None, o=None, B=0) == 0
    assert _call(lib, q=None, k=None, v=None, o=None, S=0) == 0
    assert _call(lib, q=None, k=None, v=None, o=None, H=0, D=128, dtype=0) == 0


def test_rejects_null_and_misaligned(lib):
    assert _call(lib, q=None) == -1
    assert _call(lib, o=None) == -1
    assert _call(lib, k=0x2008) == -4
    assert "16-byte" in lib.attn_last_error().decode()
    assert _call(lib, lse=0x5002) == -4
    assert "4-byte" in lib.attn_last_error().decode()


def test_rejects_bad_options(lib):
    o = da.attn_fwd_options()
    o.rescale_threshold = -1.0
    o.reserved[1] = 1
    assert _call(lib, opts=o) == -8
    o = da.attn_fwd_options()
    o.rescale_threshold = 100.0
    assert _call(lib, opts=o) == -8
    o = da.attn_fwd_options()
    o.rescale_threshold = float("nan")
    assert _call(lib, opts=o) == -8
    o = da.attn_fwd_options()
    o.variant = 12345
    assert _call(lib, opts=o) == -8
    # fp16 P holds at most 65504 < 2^16: thresholds above 15 are refused for
    # fp16 only (bf16 keeps the bound of 64).
    for thr, dtype, want in [(15.0, 0, "ok"), (15.5, 0, -8), (16.0, 0, -8), (64.0, 0, -8),
                             (16.0, 1, "ok"), (64.0, 1, "ok")]:
        o = da.attn_fwd_options()
        o.rescale_threshold = thr
        if want == "ok":
            # attn_get_config validates exactly as attn_fwd_ex and never launches:
            # 0 on a gfx950 device, ATTN_ERR_DEVICE without one, never ATTN_ERR_ARG
            cfg = da.attn_config()
            st = lib.attn_get_config(1, 1, 16, 64, dtype, ctypes.byref(o), ctypes.byref(cfg))
            assert st in (0, -6), (thr, dtype, st)
        else:
            assert _call(lib, dtype=dtype, opts=o) == want, (thr, dtype)
            assert "15" in lib.attn_last_error().decode()
    o = da.attn_fwd_options()
    o.grid = -3
    assert _call(lib, opts=o) == -8


def test_variant_must_match_head_dim_and_dtype(lib):
    for var in da.attn_variants():
        other_d = 64 if var["head_dim"] == 128 else 128
        o = da.attn_fwd_options()
        o.variant = var["id"]
        o.rescale_threshold = -1.0
        assert _call(lib, D=other_d, dtype=var["dtype"], opts=o) == -8
        assert _call(lib, D=var["head_dim"], dtype=1 - var["dtype"], opts=o) == -8


def test_variant_table(lib):
    vs = da.attn_variants()
    assert len(vs) == lib.attn_variant_count() >= 4
    ids = [v["id"] for v in vs]
    assert len(set(ids)) == len(ids)
    for v in vs:
        assert v["head_dim"] in (64, 128)
        assert v["dtype"] in (0, 1)
        assert v["key_split"] in (0, 1)
        assert v["soft_exp"] >= 0
        rows_waves = v["waves"] // (2 if v["key_split"] else 1)
        assert v["block_m"] > 0 and v["block_m"] % (32 * rows_waves) == 0
        assert v["block_n"] % 64 == 0
    for d in (64, 128):
        for dt in (0, 1):
            assert any(v["head_dim"] == d and v["dtype"] == dt for v in vs)
    assert lib.attn_variant_info(len(vs), None, None, None, None, None, None, None, None, None) == -8


def test_strerror_covers_every_status(lib):
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9, 7]:
        s = lib.attn_strerror(code)
        assert s is not None and len(s) > 0


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(ImportError):
        da.load_library(str(tmp_path / "missing.so"))


def test_binding_validates_before_calling(lib):
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        da.attn_fwd(q, q, q)          # CPU tensors are rejected before any library call
    with pytest.raises(TypeError):
        da._dtype_code(torch.zeros(1, dtype=torch.float32))
    assert math.isclose(1.0 / math.sqrt(64), 0.125)


# --- strided, partial, merge and split entry points: validation without a device ----

FAKE = 1 << 20   # a 16-byte aligned non-null address; never dereferenced on these paths


def _layout(b, h, s):
    return da.attn_layout(b, h, s)


def test_strided_rejects_bad_layouts(lib):
    B, H, S, D = 1, 2, 64, 64
    ok = _layout(H * S * D, S * D, D)
    bad_mult = _layout(H * S * D, S * D, D + 4)        # not a multiple of 8 elements
    neg = _layout(-8, S * D, D)
    huge = _layout(H * S * D, S * D, 1 << 24)
    narrow_o = _layout(H * S * D, S * D, 32)            # output rows would overlap
    f = ctypes.c_float(0.125)
    for ql, ol in [(bad_mult, ok), (neg, ok), (huge, ok), (ok, narrow_o)]:
        st = lib.attn_fwd_strided(FAKE, ctypes.byref(ql), FAKE, ctypes.byref(ok), FAKE,
                                  ctypes.byref(ok), FAKE, ctypes.byref(ol), None, B, H, S, S, D,
                                  f, da.ATTN_BF16, None, None)
        assert st == -3, (ql.seq_stride, ol.seq_stride)
    # queries without keys have no softmax
    st = lib.attn_fwd_strided(FAKE, None, FAKE, None, FAKE, None, FAKE, None, None, B, H, S, 0, D,
                              f, da.ATTN_BF16, None, None)
    assert st == -3
    # no queries: empty, fine without pointers
    st = lib.attn_fwd_strided(None, None, None, None, None, None, None, None, None, B, H, 0, 5, D,
                              f, da.ATTN_BF16, None, None)
    assert st == 0


def test_partial_requires_lse(lib):
    st = lib.attn_fwd_partial(FAKE, None, FAKE, None, FAKE, None, FAKE, None, 1, 1, 64, 64, 64,
                              ctypes.c_float(0.1), da.ATTN_F16, None, None)
    assert st == -1


def test_merge_validation(lib):
    args = dict(B=1, H=1, S=8, D=64, dtype=da.ATTN_F32)

    def merge(n=2, o_parts=FAKE, lse_parts=FAKE, o=FAKE, **kw):
        a = dict(args, **kw)
        return lib.attn_merge(o_parts, lse_parts, n, o, None, None, a["B"], a["H"], a["S"],
                              a["D"], a["dtype"], None)

    assert merge(n=0) == -8
    assert merge(dtype=3) == -2
    assert merge(D=96) == -3
    assert merge(o=None) == -1
    assert merge(o_parts=FAKE + 4) == -4
    assert merge(S=0, o=None, o_parts=None, lse_parts=None) == 0


def test_split_validation_and_workspace_size(lib):
    f = ctypes.c_float(0.1)
    assert lib.attn_fwd_split(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 512, 64, f, da.ATTN_F16, None,
                              65, FAKE, 1 << 20, None) == -8
    assert lib.attn_fwd_split(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 512, 64, f, da.ATTN_F16, None,
                              -1, FAKE, 1 << 20, None) == -8
    # partial O (fp32) then partial LSE, each rounded up to 256 bytes
    n, B, H, S, D = 3, 2, 4, 1000, 128
    o_bytes = n * B * H * S * D * 4
    l_bytes = n * B * H * S * 4
    up = lambda x: (x + 255) // 256 * 256
    assert lib.attn_fwd_split_workspace_size(B, H, S, D, n) == up(o_bytes) + up(l_bytes)
    # automatic choice: sized for at most S / 1024 ranges (capped at 64, at least 1)
    assert lib.attn_fwd_split_workspace_size(1, 1, 4096, 64, 0) == up(4 * 4096 * 64 * 4) + up(4 * 4096 * 4)
    assert lib.attn_fwd_split_workspace_size(1, 1, 100, 64, 0) == up(100 * 64 * 4) + up(100 * 4)
    assert lib.attn_fwd_split_workspace_size(1, 1, 100, 96, 1) == 0


def test_causal_option_validation(lib):
    opts = da.attn_fwd_options()
    opts.rescale_threshold = -1
    opts.causal = 3
    assert _call(lib, opts=opts) == -8
    opts.causal = -1
    assert _call(lib, opts=opts) == -8
    # Python side: True -> 1, an int -> 2 with that offset, False -> 0
    assert da._options(None, 0, 0, True).causal == 1
    o = da._options(None, 0, 0, -7)
    assert (o.causal, o.causal_offset) == (2, -7)
    assert da._options(None, 0, 0, False).causal == 0


def test_library_shares_torch_hip_runtime():
    """Loading the library before torch must still leave one HIP runtime mapped.

    A second libamdhip64 next to torch's own would keep its own device state,
    so pointers and streams from torch would not be valid in the library.
    """
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import dense_attention_amd as da\n"
        "da.load_library()\n"
        "import torch\n"
        "maps = open('/proc/self/maps').read()\n"
        "print(len({l.split()[-1] for l in maps.splitlines() if 'libamdhip64' in l}))\n"
    ) % os.path.dirname(os.path.dirname(os.path.abspath(da.__file__)))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip().splitlines()[-1] == "1"


def test_noalloc_refuses_partials_beyond_the_static_scratch(lib):
    """With an explicit range count the scratch size is known before any device
    query: a problem whose partials exceed the static scratch is refused with
    ATTN_ERR_SCRATCH and nothing is launched."""
    f = ctypes.c_float(0.1)
    B, H, S, D, n = 1, 16, 4096, 128, 8          # 8 ranges: 256 MiB of fp32 partials
    need = lib.attn_fwd_split_workspace_size(B, H, S, D, n)
    assert need > da.NOALLOC_SCRATCH_BYTES
    st = lib.attn_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, None, B, H, S, D, f, da.ATTN_BF16,
                                    None, n, None)
    assert st == -9
    assert str(need) in lib.attn_last_error().decode()
    # same validation as attn_fwd_split before that
    assert lib.attn_fwd_split_noalloc(FAKE, FAKE, FAKE, FAKE, None, 1, 1, 512, 64, f, da.ATTN_F16,
                                      None, 65, None) == -8
    assert lib.attn_fwd_split_noalloc(None, None, None, None, None, 0, 1, 512, 64, f, da.ATTN_F16,
                                      None, 2, None) == 0
    # the header's size is the binding's
    text = open(HEADER).read()
    assert "#define ATTN_NOALLOC_SCRATCH_BYTES (64u * 1024u * 1024u)" in text
    assert da.NOALLOC_SCRATCH_BYTES == 64 * 1024 * 1024


def test_plain_c_caller(tmp_path):
    """The header compiles as strict C99 (and as C++) with warnings as errors,
    and a C program linked against libattn.so runs the host-only calls and
    the argument checks (tests/c_abi_check.c)."""
    import shutil
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    inc = os.path.join(os.path.dirname(here), "include")
    libdir = os.path.dirname(da.library_path())
    exe = str(tmp_path / "c_abi_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc,
                    os.path.join(here, "c_abi_check.c"), "-o", exe, "-L", libdir, "-lattn",
                    "-Wl,-rpath," + libdir], check=True, capture_output=True, text=True)
    cxx = shutil.which("g++")
    if cxx is not None:
        src = tmp_path / "hdr.cpp"
        src.write_text('#include "attn.h"\nint main() { return attn_variant_count() > 0 ? 0 : 1; }\n')
        subprocess.run([cxx, "-std=c++11", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", inc,
                        "-c", str(src), "-o", str(tmp_path / "hdr.o")], check=True,
                       capture_output=True, text=True)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and "c abi check ok" in run.stdout, run.stdout + run.stderr
