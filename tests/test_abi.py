"""The C-ABI library on the CPU: it loads, exports every symbol include/fa.h
declares, and rejects invalid arguments before making any HIP call (no
compute call is made here)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_io_aware_18_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake, never-dereferenced device addresses: validation fails before use.
BASE = 0x7F0000000000
MB = 1 << 20


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        from exact_io_aware_18_amd import build

        build.build()
    return fa.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\s*\*?\s*(fa_[a-z0-9_]+)\s*\(", text, flags=re.M)))


def test_header_declares_expected_api():
    assert declared_functions() == sorted(fa.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True)
    if out.returncode == 0:
        exported = set(re.findall(r" T (fa_[a-z0-9_]+)$", out.stdout, flags=re.M))
        assert set(declared_functions()) <= exported
        assert exported <= set(declared_functions()), exported - set(declared_functions())


def test_strerror_and_version(lib):
    assert fa.fa_version() == 10000
    for code, name in fa.STATUS_NAMES.items():
        msg = fa.fa_strerror(code)
        assert isinstance(msg, str) and msg
    assert fa.fa_strerror(12345) == "unknown status"


def test_workspace_bytes(lib):
    assert fa.fa_bwd_workspace_bytes(2, 3, 1000, 64) >= 2 * 3 * 1000 * 4
    assert fa.fa_bwd_workspace_bytes(2, 3, 1000, 64) % 256 == 0
    assert fa.fa_bwd_workspace_bytes(0, 3, 1000, 64) == 0
    assert fa.fa_bwd_workspace_bytes(1, 1, 10, 96) == 0


def test_fwd_query_rows(lib):
    q = fa.fa_fwd_query_rows
    # block mask: one 128-row workgroup per mask row
    assert q(1, 16, 65536, 64, 0, 1, 0) == 128
    # small grids: the 128-row kernel (fewer than 512 two-group workgroups)
    assert q(8, 12, 1024, 64, 1, 0, 0) == 128
    assert q(1, 16, 4096, 128, 0, 0, 0) == 128
    # exactly 512 two-group workgroups
    assert q(2, 64, 1000, 64, 1, 0, 0) == 256
    assert q(2, 64, 1000, 128, 0, 0, 0) == 256
    # three groups at d = 64 from N = 4096 with at least 512 of their workgroups
    assert q(1, 16, 16384, 64, 1, 0, 0) == 384
    assert q(2, 24, 4100, 64, 0, 0, 0) == 384
    assert q(2, 24, 4095, 64, 0, 0, 0) == 256     # N below 4096: two groups (768 workgroups)
    assert q(1, 16, 16384, 64, 1, 0, 1) == 256   # dropout: two groups
    assert q(1, 16, 16384, 128, 1, 0, 0) == 256  # d = 128: two groups
    # rejected sizes and flags
    assert q(0, 16, 4096, 64, 0, 0, 0) == 0
    assert q(1, 16, 4096, 96, 0, 0, 0) == 0
    assert q(1, 16, 4096, 64, 2, 0, 0) == 0
    assert q(1, 16, 4096, 64, 0, 0, 3) == 0


def fwd_args(B=1, H=2, N=256, d=64, esz=2, **over):
    tb = B * H * N * d * esz
    a = dict(q=BASE, k=BASE + 1 * tb + MB, v=BASE + 2 * (tb + MB), o=BASE + 3 * (tb + MB),
             lse=BASE + 4 * (tb + MB), B=B, H=H, N=N, d=d, scale=0.125, causal=0,
             blockmask=None, stream=None)
    a.update(over)
    return a


def call_fwd(f, a):
    return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"], a["scale"],
             a["causal"], a["blockmask"], a["stream"])


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("over,code", [
    (dict(q=None), -1), (dict(lse=None), -1), (dict(o=None), -1),
    (dict(B=0), -2), (dict(H=-1), -2), (dict(N=0), -2), (dict(N=1 << 25, d=128), -2),
    (dict(d=96), -3), (dict(d=32), -3),
    (dict(q=BASE + 8), -4), (dict(lse=BASE + 4 * (256 * 128 * 2 + MB) + 2), -4),
    (dict(causal=2), -7), (dict(causal=-1), -7),
    (dict(scale=float("nan")), -10), (dict(scale=float("inf")), -10),
])
def test_fwd_rejects(lib, f32, over, code):
    esz = 4 if f32 else 2
    a = fwd_args(esz=esz)
    a.update(over)
    f = fa.fa_fwd_f32 if f32 else fa.fa_fwd
    assert call_fwd(f, a) == code


@pytest.mark.parametrize("f32", [False, True])
def test_fwd_rejects_aliasing(lib, f32):
    esz = 4 if f32 else 2
    f = fa.fa_fwd_f32 if f32 else fa.fa_fwd
    a = fwd_args(esz=esz)
    assert call_fwd(f, dict(a, o=a["q"])) == -5               # O on top of Q
    assert call_fwd(f, dict(a, o=a["v"] + 64)) == -5          # O overlapping V
    assert call_fwd(f, dict(a, lse=a["o"] + 16)) == -5        # lse inside O
    assert call_fwd(f, dict(a, blockmask=a["o"] + 32)) == -5  # mask inside O


def bwd_args(B=1, H=2, N=256, d=64, esz=2, **over):
    tb = B * H * N * d * esz
    gb = B * H * N * d * 4
    step = max(tb, gb) + MB
    names = ["q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "workspace"]
    a = {n: BASE + i * step for i, n in enumerate(names)}
    a.update(B=B, H=H, N=N, d=d, scale=0.125, causal=1, blockmask=None,
             workspace_bytes=fa.fa_bwd_workspace_bytes(B, H, N, d), stream=None)
    a.update(over)
    return a


def call_bwd(f, a):
    return f(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"], a["dv"],
             a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"], a["blockmask"],
             a["workspace"], a["workspace_bytes"], a["stream"])


@pytest.mark.parametrize("f32", [False, True])
@pytest.mark.parametrize("over,code", [
    (dict(dout=None), -1), (dict(dq=None), -1), (dict(lse=None), -1),
    (dict(N=0), -2), (dict(d=80), -3),
    (dict(dk=BASE + 7 * (256 * 64 * 2 * 4 + MB) + 4), -4),
    (dict(causal=3), -7), (dict(scale=float("-inf")), -10),
    (dict(workspace=None), -6), (dict(workspace_bytes=100), -6),
])
def test_bwd_rejects(lib, f32, over, code):
    esz = 4 if f32 else 2
    a = bwd_args(esz=esz)
    a.update(over)
    f = fa.fa_bwd_f32 if f32 else fa.fa_bwd
    assert call_bwd(f, a) == code


@pytest.mark.parametrize("f32", [False, True])
def test_bwd_rejects_aliasing(lib, f32):
    esz = 4 if f32 else 2
    f = fa.fa_bwd_f32 if f32 else fa.fa_bwd
    a = bwd_args(esz=esz)
    assert call_bwd(f, dict(a, dq=a["q"])) == -5
    assert call_bwd(f, dict(a, dk=a["dq"] + 256)) == -5
    assert call_bwd(f, dict(a, workspace=a["dv"])) == -5
    assert call_bwd(f, dict(a, dv=a["lse"])) == -5


def test_stage_calls_reject(lib):
    a = bwd_args()
    ws, wn = a["workspace"], a["workspace_bytes"]
    pre = lambda **o: fa.fa_bwd_preprocess(o.get("o", a["o"]), o.get("dout", a["dout"]), 1, 2, 256,
                                           o.get("d", 64), o.get("ws", ws), o.get("wn", wn), None)
    assert pre(o=None) == -1
    assert pre(d=48) == -3
    assert pre(ws=None) == -6
    assert pre(wn=16) == -6
    assert pre(ws=a["o"]) == -5

    def dkdv(**o):
        return fa.fa_bwd_dkdv(a["q"], a["k"], a["v"], a["lse"], a["dout"], o.get("dk", a["dk"]),
                              o.get("dv", a["dv"]), 1, 2, o.get("N", 256), 64, o.get("scale", 0.1),
                              o.get("causal", 1), None, ws, o.get("wn", wn), None)
    assert dkdv(dk=None) == -1
    assert dkdv(N=-3) == -2
    assert dkdv(causal=5) == -7
    assert dkdv(scale=float("nan")) == -10
    assert dkdv(wn=0) == -6
    assert dkdv(dk=a["q"]) == -5
    assert dkdv(dv=ws) == -5
    assert dkdv(dv=a["dk"]) == -5

    def dq(**o):
        return fa.fa_bwd_dq(a["q"], a["k"], a["v"], a["lse"], a["dout"], o.get("dq", a["dq"]), 1, 2,
                            256, o.get("d", 64), 0.1, 0, None, ws, wn, None)
    assert dq(dq=None) == -1
    assert dq(d=256) == -3
    assert dq(dq=a["dout"]) == -5
    assert dq(dq=a["dq"] + 8) == -4


def test_tensor_wrapper_raises_typed_error(lib):
    with pytest.raises(fa.FAError) as e:
        fa._check(-3, "fa_fwd")
    assert e.value.status == -3 and "FA_ERR_HEADDIM" in str(e.value)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(fa, "_lib", None)
    monkeypatch.setattr(fa, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        fa.lib()


@pytest.mark.parametrize("p", [1.0, 1.5, -0.1, float("nan"), float("inf")])
def test_dropout_calls_reject_probability(lib, p):
    a = fwd_args()
    assert fa.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], 1, 2, 256, 64, 0.125, 0,
                             None, p, 7, None) == -11
    b = bwd_args()
    assert fa.fa_bwd_dropout(b["q"], b["k"], b["v"], b["o"], b["lse"], b["dout"], b["dq"], b["dk"],
                             b["dv"], 1, 2, 256, 64, 0.125, 1, None, p, 7, b["workspace"],
                             b["workspace_bytes"], None) == -11


def test_dropout_calls_check_the_common_arguments_first(lib):
    a = fwd_args()
    f = lambda **o: fa.fa_fwd_dropout(o.get("q", a["q"]), a["k"], a["v"], o.get("o", a["o"]),
                                      a["lse"], 1, 2, 256, o.get("d", 64), 0.125, o.get("causal", 0),
                                      None, o.get("p", 0.1), 7, None)
    assert f(q=None) == -1
    assert f(d=96) == -3
    assert f(causal=2) == -7
    assert f(o=a["q"]) == -5
    assert f(d=96, p=2.0) == -3  # shape errors come before the probability check
    b = bwd_args()
    g = lambda **o: fa.fa_bwd_dropout(b["q"], b["k"], b["v"], b["o"], b["lse"], b["dout"],
                                      o.get("dq", b["dq"]), b["dk"], b["dv"], 1, 2, 256, 64, 0.125,
                                      1, None, 0.1, 2**64 - 1, o.get("ws", b["workspace"]),
                                      o.get("wn", b["workspace_bytes"]), None)
    assert g(dq=None) == -1
    assert g(wn=8) == -6
    assert g(dq=b["q"]) == -5
    assert g(ws=None) == -6


def test_decode_workspace_bytes(lib):
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 1, 64) >= 4 * 65
    assert fa.fa_decode_workspace_bytes(2, 8, 4, 100000, 128) >= 2 * 8 * 4 * 129 * 4
    assert fa.fa_decode_workspace_bytes(1, 1, 0, 10, 64) == 0
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 0, 64) == 0
    assert fa.fa_decode_workspace_bytes(1, 1, 1, 10, 80) == 0


def test_decode_rejects(lib):
    B, H, Nq, Nk, d = 2, 4, 3, 5000, 64
    tq, tk = B * H * Nq * d * 2, B * H * Nk * d * 2
    ws = fa.fa_decode_workspace_bytes(B, H, Nq, Nk, d)
    a = dict(q=BASE, k=BASE + tq + MB, v=BASE + tq + tk + 2 * MB, o=BASE + tq + 2 * tk + 3 * MB,
             lse=BASE + 2 * tq + 2 * tk + 4 * MB, ws=BASE + 2 * tq + 2 * tk + 5 * MB)

    def call(**o):
        x = dict(a, **o)
        return fa.fa_fwd_decode(x["q"], x["k"], x["v"], x["o"], x["lse"], B, H, o.get("Nq", Nq),
                                o.get("Nk", Nk), o.get("d", d), o.get("scale", 0.1),
                                o.get("causal", 1), x["ws"], o.get("wn", ws), None)
    assert call(q=None) == -1
    assert call(o=None) == -1
    assert call(Nq=0) == -2
    assert call(Nk=-1) == -2
    assert call(d=96) == -3
    assert call(causal=4) == -7
    assert call(scale=float("nan")) == -10
    assert call(ws=None) == -6
    assert call(wn=ws - 1) == -6
    assert call(q=BASE + 4) == -4
    assert call(o=a["k"] + 64) == -5
    assert call(ws=a["o"]) == -5


@pytest.mark.parametrize("compiler,lang,std", [("gcc", "c", "c99"), ("g++", "c++", "c++11")])
def test_header_is_plain_c(compiler, lang, std, tmp_path):
    """include/fa.h compiles as strict C99 and as C++ (no torch or HIP types
    in the signatures), and a C translation unit can take every entry point's
    address."""
    import shutil

    if shutil.which(compiler) is None:
        pytest.skip(f"{compiler} not available")
    src = tmp_path / ("use.c" if lang == "c" else "use.cpp")
    names = declared_functions()
    body = "\n".join(f"  (void)&{n};" for n in names)
    src.write_text(f'#include "fa.h"\nint main(void) {{\n{body}\n  return 0;\n}}\n')
    out = subprocess.run([compiler, f"-std={std}", "-Wall", "-Wextra", "-Werror", "-pedantic"
                          if lang == "c" else "-Wall", "-fsyntax-only", "-I",
                          os.path.join(ROOT, "include"), str(src)], capture_output=True, text=True)
    assert out.returncode == 0, out.stderr


def call_noalloc(a):
    return fa.fa_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                             a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                             a["blockmask"], a["stream"])


def test_noalloc_limit(lib):
    assert fa.fa_bwd_noalloc_max_rows() == 1 << 22
    assert fa.fa_strerror(-12).startswith("B * H * N exceeds")


@pytest.mark.parametrize("over,code", [
    (dict(dout=None), -1), (dict(o=None), -1), (dict(lse=None), -1),
    (dict(N=0), -2), (dict(d=80), -3),
    (dict(dk=BASE + 7 * (256 * 64 * 2 * 4 + MB) + 4), -4),
    (dict(causal=3), -7), (dict(scale=float("nan")), -10),
])
def test_noalloc_rejects(lib, over, code):
    a = bwd_args()
    a.update(over)
    assert call_noalloc(a) == code


def test_noalloc_rejects_aliasing_and_size(lib):
    a = bwd_args()
    assert call_noalloc(dict(a, dq=a["q"])) == -5
    assert call_noalloc(dict(a, dv=a["dk"] + 64)) == -5
    # one row past the fixed array: rejected before any HIP call
    big = bwd_args(B=1, H=64, N=65537)
    assert call_noalloc(big) == -12
    ok = bwd_args(B=1, H=64, N=65536)  # exactly the limit passes the size check
    assert 64 * 65536 == fa.fa_bwd_noalloc_max_rows()
    assert call_noalloc(dict(ok, dq=ok["q"])) == -5  # ... and reaches the alias check
