"""The C-ABI library on the CPU: it loads, exports what include/fa.h declares,
and rejects bad arguments before touching the GPU (no compute calls here)."""
import ctypes
import os
import re
import shutil
import subprocess

import pytest

import exact_attention_26_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
FAKE = ctypes.c_void_p(0x1000)   # never dereferenced: every call below fails validation


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    assert _declared_functions() == sorted([
        "fa_fwd", "fa_bwd", "fa_bwd_workspace_size", "fa_paged_decode",
        "fa_paged_decode_workspace_size", "fa_paged_prefill", "fa_status_string",
        "fa_last_hip_error", "fa_tree_decode", "fa_rope", "fa_fwd_rope_workspace_size",
        "fa_fwd_rope", "fa_paged_decode_noalloc"])


def test_library_exports_every_declared_symbol():
    lib = fa.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", fa.library_path()],
                             capture_output=True, text=True, check=True).stdout
        exported = set(re.findall(r" T (fa_\w+)", out))
        assert set(_declared_functions()) <= exported


def test_read_probe_library_is_separate():
    """The benchmark's read probe lives in its own library: libfa.so exports
    only the attention boundary, and the probe rejects bad arguments before
    launching anything."""
    path = os.path.join(ROOT, "exact_attention_26_amd", "libfa_probe.so")
    if not os.path.exists(path):
        pytest.skip("libfa_probe.so not built")
    probe = ctypes.CDLL(path)
    probe.fa_probe_read.restype = ctypes.c_int
    probe.fa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p]
    assert not hasattr(fa.load_library(), "fa_probe_read")
    assert probe.fa_probe_read(None, 1 << 20, None, FAKE, None) != 0
    assert probe.fa_probe_read(FAKE, 8, None, FAKE, None) != 0
    assert probe.fa_probe_read(FAKE, 4096 * 33, FAKE, FAKE, None) != 0   # not whole 128 KiB


def test_status_strings_and_last_error():
    assert fa.fa_status_string(0) == "FA_OK"
    assert "INVALID" in fa.fa_status_string(1)
    assert "UNSUPPORTED" in fa.fa_status_string(2)
    assert "HIP" in fa.fa_status_string(3)
    assert "unknown" in fa.fa_status_string(42)
    assert fa.fa_last_hip_error() == 0


def _fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, H=1, N=16, d=64, causal=0,
             scale=0.125, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.load_library().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                    a["N"], a["d"], a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(B=0), 1), (dict(H=0), 1), (dict(N=0), 1), (dict(N=-3), 1), (dict(causal=3), 1),
    (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1),
    (dict(d=96), 2), (dict(d=32), 2), (dict(d=256), 2), (dict(dtype=5), 2),
])
def test_fwd_rejects_before_launch(kw, status):
    assert _fwd(**kw) == status


def test_bwd_workspace_size():
    # 256 bytes per 32 rows of every head
    assert fa.fa_bwd_workspace_size(8, 16, 2048, 128) == 8 * 16 * 64 * 256
    assert fa.fa_bwd_workspace_size(1, 2, 65, 64) == 2 * 3 * 256
    assert fa.fa_bwd_workspace_size(1, 1, 0, 64) == 0


def _bwd(**kw):
    ws = fa.fa_bwd_workspace_size(1, 1, 16, 64)
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE, B=1,
             H=1, N=16, d=64, causal=0, scale=0.125, dtype=fa.FA_BF16, ws=FAKE, wsb=ws)
    a.update(kw)
    return fa.load_library().fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                    a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["causal"],
                                    a["scale"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(k=None), 1), (dict(v=None), 1), (dict(o=None), 1),
    (dict(lse=None), 1), (dict(do=None), 1), (dict(dq=None), 1), (dict(dk=None), 1),
    (dict(dv=None), 1), (dict(B=0), 1), (dict(N=0), 1), (dict(causal=2), 1),
    (dict(scale=float("inf")), 1), (dict(ws=None), 1), (dict(wsb=255), 1),
    (dict(d=96), 2), (dict(dtype=fa.FA_F32), 2), (dict(dtype=7), 2),
])
def test_bwd_rejects_before_launch(kw, status):
    assert _bwd(**kw) == status


def test_decode_workspace_size():
    assert fa.fa_paged_decode_workspace_size(64, 32, 128, 16, 512) == 64 * 32 * 16 * 130 * 4
    assert fa.fa_paged_decode_workspace_size(3, 2, 64, 16, 33) == 3 * 2 * 2 * 66 * 4
    assert fa.fa_paged_decode_workspace_size(0, 2, 64, 16, 33) == 0


def _decode(**kw):
    ws = fa.fa_paged_decode_workspace_size(2, 2, 128, 16, 4)
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, o=FAKE, lse=None, S=2, H=2, d=128,
             P=16, mb=4, nb=10, scale=0.1, dtype=fa.FA_BF16, ws=FAKE, wsb=ws)
    a.update(kw)
    return fa.load_library().fa_paged_decode(
        a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["o"], a["lse"], a["S"], a["H"], a["d"],
        a["P"], a["mb"], a["nb"], a["scale"], a["dtype"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(vc=None), 1), (dict(bt=None), 1),
    (dict(sl=None), 1), (dict(o=None), 1), (dict(S=0), 1), (dict(H=0), 1), (dict(mb=0), 1),
    (dict(nb=0), 1), (dict(scale=float("nan")), 1), (dict(ws=None), 1), (dict(wsb=16), 1),
    (dict(d=96), 2), (dict(P=8), 2), (dict(dtype=fa.FA_F32), 2), (dict(dtype=9), 2),
])
def test_decode_rejects_before_launch(kw, status):
    assert _decode(**kw) == status


def _prefill(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, o=FAKE, lse=None, S=2, H=2,
             d=128, P=16, mb=4, nb=10, tq=30, mq=20, causal=1, scale=0.1, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.load_library().fa_paged_prefill(
        a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["cu"], a["o"], a["lse"], a["S"], a["H"],
        a["d"], a["P"], a["mb"], a["nb"], a["tq"], a["mq"], a["causal"], a["scale"], a["dtype"],
        None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(kc=None), 1), (dict(vc=None), 1), (dict(bt=None), 1),
    (dict(sl=None), 1), (dict(cu=None), 1), (dict(o=None), 1), (dict(S=0), 1), (dict(H=0), 1),
    (dict(mb=0), 1), (dict(nb=0), 1), (dict(tq=0), 1), (dict(mq=0), 1), (dict(causal=2), 1),
    (dict(scale=float("inf")), 1), (dict(S=65536, H=65536), 1),
    (dict(d=96), 2), (dict(P=8), 2), (dict(dtype=fa.FA_F32), 2), (dict(dtype=3), 2),
])
def test_prefill_rejects_before_launch(kw, status):
    assert _prefill(**kw) == status


def _tree(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, bt=FAKE, sl=FAKE, cu=FAKE, par=FAKE, o=FAKE, lse=None,
             S=2, H=2, d=128, P=16, mb=4, nb=10, tq=30, mq=20, scale=0.1, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.load_library().fa_tree_decode(
        a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["cu"], a["par"], a["o"], a["lse"], a["S"],
        a["H"], a["d"], a["P"], a["mb"], a["nb"], a["tq"], a["mq"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(par=None), 1), (dict(q=None), 1), (dict(cu=None), 1), (dict(S=0), 1), (dict(tq=0), 1),
    (dict(mq=0), 1), (dict(scale=float("nan")), 1),
    (dict(mq=65), 2), (dict(d=96), 2), (dict(P=32), 2), (dict(dtype=fa.FA_F32), 2),
])
def test_tree_rejects_before_launch(kw, status):
    assert _tree(**kw) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), 1), (dict(out=None), 1), (dict(c=None), 1), (dict(s=None), 1), (dict(N=0), 1),
    (dict(d=96), 2), (dict(dtype=fa.FA_F32), 2),
])
def test_rope_rejects_before_launch(kw, status):
    a = dict(x=FAKE, out=FAKE, c=FAKE, s=FAKE, B=1, H=2, N=16, d=64, dtype=fa.FA_BF16)
    a.update(kw)
    assert fa.load_library().fa_rope(a["x"], a["out"], a["c"], a["s"], a["B"], a["H"], a["N"],
                                     a["d"], a["dtype"], None) == status


def test_fwd_rope_workspace_and_rejections():
    lib = fa.load_library()
    assert fa.fa_fwd_rope_workspace_size(8, 16, 2048, 128) == 8 * 16 * 2048 * 128 * 2
    assert fa.fa_fwd_rope_workspace_size(0, 1, 1, 64) == 0
    ws = fa.fa_fwd_rope_workspace_size(1, 1, 16, 64)

    def call(**kw):
        a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, c=FAKE, s=FAKE, N=16, d=64, dtype=fa.FA_BF16,
                 ws=FAKE, wsb=ws)
        a.update(kw)
        return lib.fa_fwd_rope(a["q"], a["k"], a["v"], a["o"], None, a["c"], a["s"], 1, 1, a["N"],
                               a["d"], 0, 0.125, a["dtype"], a["ws"], a["wsb"], None)
    assert call(c=None) == 1 and call(s=None) == 1 and call(ws=None) == 1
    assert call(wsb=ws - 1) == 1 and call(q=None) == 1 and call(N=0) == 1
    assert call(d=96) == 2 and call(dtype=fa.FA_F32) == 2


def test_host_validation_unit_with_sanitizers(tmp_path):
    """The validation header on its own, compiled with g++ (no HIP) under ASan/UBSan."""
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    exe = tmp_path / "test_validate"
    subprocess.run([gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I" + os.path.join(ROOT, "include"),
                    "-I" + os.path.join(ROOT, "exact_attention_26_amd", "csrc"),
                    os.path.join(ROOT, "tests", "host", "test_validate.cpp"), "-o", str(exe)],
                   check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_binding_raises_when_library_missing(monkeypatch, tmp_path):
    import exact_attention_26_amd._binding as b
    monkeypatch.setattr(b, "_LIB", None)
    monkeypatch.setenv("FA_LIBRARY", str(tmp_path / "missing.so"))
    with pytest.raises(fa.FaError):
        b.load_library()


@pytest.mark.parametrize("entry", ["decode", "prefill", "tree"])
@pytest.mark.parametrize("bad", ["k", "v"])
def test_binding_rejects_cache_dtype_mismatch(entry, bad):
    """The library is told q's dtype only, so a float32 cache passed with a
    bf16 q would be read as bf16: the binding refuses it before any call."""
    import torch
    q = torch.zeros((3, 2, 64), dtype=torch.bfloat16)
    good = torch.zeros((4, 2, 16, 64), dtype=torch.bfloat16)
    wrong = torch.zeros((4, 2, 16, 64), dtype=torch.float32)
    kc, vc = (wrong, good) if bad == "k" else (good, wrong)
    table = torch.zeros((3, 4), dtype=torch.int32)
    lens = torch.ones(3, dtype=torch.int32)
    cu = torch.arange(4, dtype=torch.int32)
    o = torch.empty_like(q)
    with pytest.raises(ValueError, match="dtype"):
        if entry == "decode":
            fa.fa_paged_decode(q, kc, vc, table, lens, o, None, 0.125,
                               torch.empty(64, dtype=torch.uint8))
        elif entry == "prefill":
            fa.fa_paged_prefill(q, kc, vc, table, lens, cu, o, None, 1, True, 0.125)
        else:
            fa.fa_tree_decode(q, kc, vc, table, lens, cu, torch.full((3,), -1, dtype=torch.int32),
                              o, None, 1, 0.125)


def _decode_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, table=FAKE, lens=FAKE, o=FAKE, lse=None, S=2, H=2, d=128,
             page_size=16, max_blocks=4, num_blocks=8, scale=0.1, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.load_library().fa_paged_decode_noalloc(
        a["q"], a["kc"], a["vc"], a["table"], a["lens"], a["o"], a["lse"], a["S"], a["H"],
        a["d"], a["page_size"], a["max_blocks"], a["num_blocks"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(table=None), 1), (dict(S=0), 1), (dict(num_blocks=0), 1),
    (dict(scale=float("nan")), 1), (dict(d=96), 2), (dict(page_size=8), 2),
    (dict(dtype=fa.FA_F32), 2),
    # d = 128: 520 bytes per (sequence, head, split of 32 pages); 64 x 32 heads with
    # 32 splits need 34 MB, and one (sequence, head) with 64 528 splits 1 byte too many
    (dict(S=64, H=32, max_blocks=32 * 32), 4),
    (dict(S=1, H=1, max_blocks=32 * (((32 << 20) // 520) + 1)), 4),
])
def test_decode_noalloc_rejects_before_launch(kw, status):
    """The allocation-free decode checks what fa_paged_decode checks (less the
    workspace) and refuses, with FA_ERR_TOO_LARGE, any call whose partials do
    not fit its 32 MiB scratch array -- all before touching the GPU."""
    assert _decode_noalloc(**kw) == status


def test_decode_noalloc_limit_matches_the_workspace_size():
    """The largest call that fits needs exactly what fa_paged_decode's workspace
    for the same sizes would hold, up to FA_NOALLOC_SCRATCH_BYTES."""
    splits = (32 << 20) // 520                    # d = 128: 520 bytes per split
    assert fa.fa_paged_decode_workspace_size(1, 1, 128, 16, 32 * splits) <= \
        fa.FA_NOALLOC_SCRATCH_BYTES
    assert fa.fa_paged_decode_workspace_size(1, 1, 128, 16, 32 * (splits + 1)) > \
        fa.FA_NOALLOC_SCRATCH_BYTES
    assert "TOO_LARGE" in fa.fa_status_string(4)
