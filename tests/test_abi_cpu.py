"""The C-ABI library loads, exports every symbol include/chipmunk.h declares,
and rejects bad arguments before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from dynamic_column_sparse_amd.digest import source_digest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "chipmunk.h")
LIBSO = os.path.join(ROOT, "dynamic_column_sparse_amd", "libchipmunk.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIBSO), reason="libchipmunk.so not built")


@pytest.fixture(scope="module")
def L():
    from dynamic_column_sparse_amd import lib
    return lib


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]*?\b(chipmunk_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    decl = _declared()
    for name in ("chipmunk_dense_step", "chipmunk_identify_topk", "chipmunk_sparse_mlp_delta",
                 "chipmunk_sparse_attn_delta", "chipmunk_cache_writeback", "chipmunk_sparse_step",
                 "chipmunk_sparse_attn_reident", "chipmunk_sparse_step_reident"):
        assert name in decl


def test_every_declared_symbol_is_exported(L):
    so = ctypes.CDLL(LIBSO)
    decl = _declared()
    assert len(decl) >= 12
    for name in decl:
        assert hasattr(so, name), name
    assert set(L.EXPORTS) <= set(decl)


def test_version_names_workspace(L):
    assert L.chipmunk_abi_version() == L.ABI_VERSION == 8
    assert L.chipmunk_source_digest() == source_digest()
    names = L.kernel_names()
    assert "mlp_gemm1_sparse" in names and "attn_sparse" in names and "topk_rows" in names
    assert "attn_reident" in names
    assert L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, 4352, 3072, 12288, 3686) == 34 * 3712 * 128 * 2
    assert L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, 300, 128, 640, 0) == 0
    assert L.chipmunk_workspace_bytes(L.OP_DENSE_MLP, 300, 128, 640, 200) == 0


FAKE = 0x7f0000000000  # aligned, never dereferenced: every case below fails validation first


def _mlp(L, n=300, d=256, h=640, **kw):
    args = dict(w1t=FAKE, w2=FAKE, a_cache=FAKE, score=FAKE)
    args.update(kw)
    return L.mlp_layer(n, d, h, **args)


def _code(L, fn, *a, **kw):
    try:
        fn(*a, **kw)
    except L.ChipmunkError as e:
        assert L.chipmunk_last_error() != ""
        return e.code
    return 0


@pytest.mark.parametrize("case,code", [
    (dict(n=0), 2), (dict(d=100), 2), (dict(d=64), 2), (dict(h=0), 2), (dict(h=100), 2),
    (dict(w1t=None), 1), (dict(a_cache=None), 1), (dict(w2=FAKE + 8), 4),
    (dict(flags=8), 2),                      # unknown flag bit
    (dict(flags=4), 1),                      # fp8 second product needs w2_f8 and w2_scale
    (dict(flags=4, w2_f8=FAKE + 4, w2_scale=FAKE), 4),
    (dict(flags=1, score=None), 1),          # rescoring needs the score array
    (dict(flags=2), 1),                      # fp8 needs w1t_f8 and w1t_scale
    (dict(flags=2, w1t_f8=FAKE, w1t_scale=None), 1),
    (dict(flags=2, w1t_f8=FAKE + 8, w1t_scale=FAKE), 4),
    (dict(w1t=None), 1),                     # a bf16 layer needs w1t
])
def test_sparse_mlp_rejects_bad_layer(L, case, code):
    lay = _mlp(L, **case)
    assert _code(L, L.chipmunk_sparse_mlp_delta, lay, FAKE, FAKE, 10, FAKE, None, FAKE, stream=0, ws_bytes=1 << 40) == code


def test_sparse_mlp_argument_checks(L):
    lay = _mlp(L)
    f = L.chipmunk_sparse_mlp_delta
    big = 1 << 40
    assert _code(L, f, lay, FAKE, FAKE, 641, FAKE, None, FAKE, stream=0, ws_bytes=big) == 2   # k > h
    assert _code(L, f, lay, FAKE, FAKE, -1, FAKE, None, FAKE, stream=0, ws_bytes=big) == 2    # k < 0
    assert _code(L, f, lay, None, FAKE, 10, FAKE, None, FAKE, stream=0, ws_bytes=big) == 1    # x NULL
    assert _code(L, f, lay, FAKE + 2, FAKE, 10, FAKE, None, FAKE, stream=0, ws_bytes=big) == 4  # x misaligned
    assert _code(L, f, lay, FAKE, None, 10, FAKE, None, FAKE, stream=0, ws_bytes=big) == 1    # idx NULL
    assert _code(L, f, lay, FAKE, FAKE, 10, None, None, FAKE, stream=0, ws_bytes=big) == 1    # y NULL
    assert _code(L, f, lay, FAKE, FAKE, 10, FAKE, FAKE + 4, FAKE, stream=0, ws_bytes=big) == 4  # packed misaligned
    assert _code(L, f, lay, FAKE, FAKE, 10, FAKE, None, None, stream=0) == 5         # no workspace
    raw = L.raw()
    small = L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, 300, 256, 640, 10) - 1
    rc = raw.chipmunk_sparse_mlp_delta(ctypes.byref(lay), FAKE, FAKE, 10, FAKE, None, FAKE, small, None)
    assert rc == 5
    # k = 0 is a valid no-op: validated, nothing enqueued
    assert _code(L, f, lay, FAKE, None, 0, FAKE, None, None, stream=0) == 0


def test_dense_step_checks(L):
    lay = _mlp(L)
    f = L.chipmunk_dense_step
    big = 1 << 40
    assert _code(L, f, L.MLP, lay, FAKE, FAKE, None, FAKE, FAKE, stream=0, ws_bytes=big) == 2   # k given for an MLP
    assert _code(L, f, L.MLP, lay, FAKE, None, None, None, FAKE, stream=0, ws_bytes=big) == 1   # out NULL
    assert _code(L, f, L.MLP, _mlp(L, score=None), FAKE, None, None, FAKE, FAKE, stream=0, ws_bytes=big) == 1
    assert _code(L, f, 7, lay, FAKE, None, None, FAKE, stream=0) == 2              # unknown kind
    att = L.attn_layer(300, 2, FAKE, FAKE, FAKE, FAKE, head_dim=64)
    assert _code(L, f, L.ATTN, att, FAKE, FAKE, FAKE, FAKE, stream=0) == 3         # head_dim 64
    att = L.attn_layer(300, 2, FAKE, FAKE, FAKE, None)
    assert _code(L, f, L.ATTN, att, FAKE, FAKE, FAKE, FAKE, stream=0) == 1         # no score buffer
    att = L.attn_layer(300, 2, FAKE, FAKE, FAKE, FAKE)
    assert _code(L, f, L.ATTN, att, FAKE, None, FAKE, FAKE, stream=0) == 1         # k NULL
    rc = L.raw().chipmunk_dense_step(0, None, FAKE, None, None, FAKE, None, 0, None)
    assert rc == 1


def test_topk_and_attn_checks(L):
    t = L.chipmunk_identify_topk
    assert _code(L, t, FAKE, 4, 10, 11, FAKE, stream=0) == 2
    assert _code(L, t, FAKE, 4, 0, 0, FAKE, stream=0) == 2
    assert _code(L, t, None, 4, 10, 3, FAKE, stream=0) == 1
    assert _code(L, t, FAKE + 2, 4, 10, 3, FAKE, stream=0) == 4
    assert _code(L, t, FAKE, 0, 10, 3, FAKE, stream=0) == 0      # no rows: no-op
    assert _code(L, t, FAKE, 4, 10, 0, FAKE, stream=0) == 0      # k = 0: no-op
    att = L.attn_layer(300, 2, FAKE, FAKE, FAKE, FAKE)
    s = L.chipmunk_sparse_attn_delta
    assert _code(L, s, att, FAKE, FAKE, FAKE, FAKE, 301, L.ATTN_SPARSE, FAKE, stream=0) == 2
    assert _code(L, s, att, FAKE, FAKE, FAKE, FAKE, 10, 5, FAKE, stream=0) == 2
    assert _code(L, s, att, FAKE, FAKE, FAKE, FAKE, 10, L.ATTN_SPARSE, None, stream=0) == 1
    assert _code(L, s, att, FAKE, FAKE, FAKE, None, 10, L.ATTN_SPARSE, FAKE, stream=0) == 1
    assert _code(L, s, att, FAKE, FAKE, FAKE, None, 0, L.ATTN_REFRESH, None, stream=0) == 0
    assert _code(L, s, L.attn_layer(300, 0, FAKE, FAKE, FAKE), FAKE, FAKE, FAKE, FAKE, 1, 0, FAKE, stream=0) == 2
    # gathered K/V rows use 32-bit byte offsets within a head: n < 2^24
    assert _code(L, s, L.attn_layer(1 << 24, 1, FAKE, FAKE, FAKE), FAKE, FAKE, FAKE, FAKE, 1, 0, FAKE, stream=0) == 2
    w = L.chipmunk_cache_writeback
    assert _code(L, w, _mlp(L), FAKE, FAKE, 700, stream=0) == 2
    assert _code(L, w, _mlp(L), None, FAKE, 10, stream=0) == 1
    assert _code(L, w, _mlp(L), FAKE, FAKE, 0, stream=0) == 0


def test_index_set_check_arguments(L):
    # Rejected before anything is enqueued (a valid call launches kernels).
    c = L.chipmunk_check_index_sets
    assert _code(L, c, FAKE, -1, 3, 10, FAKE, stream=0) == 2       # rows < 0
    assert _code(L, c, FAKE, 4, 11, 10, FAKE, stream=0) == 2       # k > cols
    assert _code(L, c, FAKE, 4, -1, 10, FAKE, stream=0) == 2       # k < 0
    assert _code(L, c, FAKE, 4, 3, 0, FAKE, stream=0) == 2         # cols < 1
    assert _code(L, c, FAKE, 4, 3, 10, None, stream=0) == 1        # no result buffer
    assert _code(L, c, None, 4, 3, 10, FAKE, stream=0) == 1        # no index sets to check
    assert _code(L, c, FAKE, 4, 3, 10, FAKE + 4, stream=0) == 4    # result not 8-byte aligned
    assert _code(L, c, FAKE + 2, 4, 3, 10, FAKE, stream=0) == 4    # idx not 4-byte aligned


def test_sparse_step_checks(L):
    # Every buffer at its own 4 GiB-spaced fake address, so only the pairs a
    # case makes overlap do; each case fails validation before any launch.
    base = {name: FAKE + i * (1 << 32) for i, name in enumerate(
        ("w1t", "w2", "a_cache", "score", "x", "midx", "y", "ws", "m", "num", "den", "ascore", "q", "k", "v",
         "aidx", "o"))}

    def call(k=200, kk=100, **over):
        a = {**base, **over}
        lay = L.mlp_layer(300, 256, 640, a["w1t"], a["w2"], a["a_cache"], a["score"])
        att = L.attn_layer(300, 2, a["m"], a["num"], a["den"], a["ascore"])
        return _code(L, L.chipmunk_sparse_step, lay, a["x"], a["midx"], k, a["y"], None, a["ws"], att, a["q"],
                     a["k"], a["v"], a["aidx"], kk, a["o"], stream=0, ws_bytes=1 << 30)

    assert call(k=641) == 2                       # MLP argument checks apply
    assert call(x=None) == 1
    assert call(kk=301) == 2                      # attention argument checks apply
    assert call(o=None) == 1
    assert call(o=base["y"]) == 2                 # o is y
    assert "overlaps" in L.chipmunk_last_error()
    assert call(q=base["ws"] + 4096) == 2         # the MLP's workspace inside q
    assert call(o=base["x"] + 16) == 2            # o over the MLP's input
    assert call(num=base["a_cache"]) == 2         # the attention cache over the MLP cache


def test_reident_checks(L):
    base = {name: FAKE + i * (1 << 32) for i, name in enumerate(
        ("m", "num", "den", "score", "qp", "kp", "vp", "q", "k", "v", "idx", "o"))}

    def call(kk=100, n=300, heads=2, **over):
        a = {**base, **over}
        att = L.attn_layer(n, heads, a["m"], a["num"], a["den"], a["score"])
        return _code(L, L.chipmunk_sparse_attn_reident, att, a["qp"], a["kp"], a["vp"], a["q"], a["k"], a["v"],
                     a["idx"], kk, a["o"], stream=0)

    assert call(kk=301) == 2 and call(kk=-1) == 2
    assert call(o=None) == 1 and call(qp=None) == 1 and call(vp=None) == 1 and call(idx=None) == 1
    assert call(score=None) == 1                  # the step rescores its keys
    assert call(kp=base["kp"] + 2) == 4           # misaligned
    assert call(o=base["num"]) == 2               # written buffers must not overlap
    assert "overlaps" in L.chipmunk_last_error()
    assert call(num=base["k"] + 256) == 2         # nor overlap an input
    assert call(score=base["den"] + 4) == 2
    assert call(n=1 << 24) == 2                   # 32-bit gathered row offsets
    # the previous step's inputs may be the current ones (read-only)
    assert call(qp=base["q"], kp=base["k"], vp=base["v"], kk=-1) == 2   # still fails on kk alone


def test_fp8_checks(L):
    q = L.chipmunk_quantize_fp8
    assert _code(L, q, FAKE, 4, 12, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 2      # cols % 8
    assert _code(L, q, FAKE, 4, 0, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 2
    assert _code(L, q, FAKE, -1, 16, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 2
    assert _code(L, q, None, 4, 16, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 1
    assert _code(L, q, FAKE, 4, 16, FAKE + (1 << 32), None, stream=0) == 1
    assert _code(L, q, FAKE + 8, 4, 16, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 4
    assert _code(L, q, FAKE, 4, 16, FAKE + 64, FAKE + (2 << 32), stream=0) == 2          # dst inside src
    assert _code(L, q, FAKE, 0, 16, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 0    # no rows: no-op
    qc = L.chipmunk_quantize_fp8_cols
    assert _code(L, qc, FAKE, 4, 12, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 2
    assert _code(L, qc, FAKE, 4, 16, None, FAKE + (2 << 32), stream=0) == 1
    assert _code(L, qc, FAKE, 4, 16, FAKE + (1 << 32), FAKE + 100, stream=0) == 2       # scale inside src
    assert _code(L, qc, FAKE, 0, 16, FAKE + (1 << 32), FAKE + (2 << 32), stream=0) == 0
    # workspace sizes of an fp8 layer: the D tiles, then x's codes and scales
    base = L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, 4352, 3072, 12288, 3686)
    xq = (4352 * 3072 + 4352 + 15) // 16 * 16
    assert L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP_FP8, 4352, 3072, 12288, 3686) == base + xq
    assert L.chipmunk_workspace_bytes(L.OP_DENSE_MLP_FP8, 4352, 3072, 12288, 0) == xq
    # an fp8 layer's sparse delta wants the larger workspace; its dense step one too
    lay = _mlp(L, flags=2, w1t_f8=FAKE + (3 << 32), w1t_scale=FAKE + (4 << 32))
    small = L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, 300, 256, 640, 10)
    rc = L.raw().chipmunk_sparse_mlp_delta(ctypes.byref(lay), FAKE, FAKE, 10, FAKE, None, FAKE, small, None)
    assert rc == 5
    rc = L.raw().chipmunk_dense_step(0, ctypes.byref(lay), FAKE, None, None, FAKE, None, 0, None)
    assert rc == 5


def test_reident_step_checks(L):
    base = {name: FAKE + i * (1 << 32) for i, name in enumerate(
        ("w1t", "w2", "a_cache", "score", "x", "midx", "y", "ws", "m", "num", "den", "ascore", "qp", "kp", "vp",
         "q", "k", "v", "aidx", "o"))}

    def call(k=200, kk=100, **over):
        a = {**base, **over}
        lay = L.mlp_layer(300, 256, 640, a["w1t"], a["w2"], a["a_cache"], a["score"])
        att = L.attn_layer(300, 2, a["m"], a["num"], a["den"], a["ascore"])
        return _code(L, L.chipmunk_sparse_step_reident, lay, a["x"], a["midx"], k, a["y"], None, a["ws"], att,
                     a["qp"], a["kp"], a["vp"], a["q"], a["k"], a["v"], a["aidx"], kk, a["o"], stream=0,
                     ws_bytes=1 << 30)

    assert call(k=641) == 2 and call(kk=301) == 2
    assert call(ascore=None) == 1                 # the attention step rescores its keys
    assert call(qp=None) == 1
    assert call(num=base["y"]) == 2               # the attention cache over the MLP output
    assert "overlaps" in L.chipmunk_last_error()
    assert call(ascore=base["ws"] + 64) == 2      # the attention scores inside the MLP workspace
    assert call(o=base["num"]) == 2               # two attention outputs on one buffer
    assert call(qp=base["a_cache"]) == 2          # the MLP writes what the attention reads


def test_timer_api_without_launches(L):
    L.chipmunk_timing_enable(True)
    for kid in range(len(L.kernel_names())):
        assert L.chipmunk_timing_read(kid) == (0.0, 0)
    L.chipmunk_timing_enable(False)
    assert _code(L, L.chipmunk_timing_read, 99) == 2


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "dynamic_column_sparse_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", text, re.M), f
                assert "chipmunk_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert not re.search(r"^\s*(from|import)\s+(dynamic_column_sparse_amd|synthetic)\b", text, re.M), f


def test_binding_refuses_a_library_built_from_other_sources(L, monkeypatch):
    # The loaded library carries the digest of the sources it was built from;
    # the binding compares it with the sources in the tree and refuses a stale
    # build instead of running it.
    assert L.chipmunk_source_digest() == source_digest()
    monkeypatch.setattr(L, "source_digest", lambda: "0123456789abcdef")
    with pytest.raises(ImportError, match="does not match the sources"):
        L._load()


def test_noalloc_entry_checks_before_any_hip_call(L):
    # The allocation-free form of the sparse MLP delta validates every argument,
    # and its scratch size against the library's 64 MiB array, before touching
    # the GPU (these calls run without one).
    f = L.chipmunk_sparse_mlp_delta_noalloc
    assert L.NOALLOC_SCRATCH_BYTES == 64 << 20
    # the HunyuanVideo shape needs 929 * 896 * 256 bytes of D tiles: refused
    big = _mlp(L, n=118800, d=3072, h=12288)
    assert L.chipmunk_workspace_bytes(L.OP_SPARSE_MLP, 118800, 3072, 12288, 860) > L.NOALLOC_SCRATCH_BYTES
    assert _code(L, f, big, FAKE, FAKE, 860, FAKE, None, stream=0) == 5
    assert "allocation-free" in L.chipmunk_last_error()
    lay = _mlp(L)
    assert _code(L, f, lay, FAKE, FAKE, 641, FAKE, None, stream=0) == 2       # k > h
    assert _code(L, f, lay, None, FAKE, 10, FAKE, None, stream=0) == 1        # x NULL
    assert _code(L, f, lay, FAKE, FAKE, 10, FAKE + 4, None, stream=0) == 4    # y misaligned
    assert _code(L, f, _mlp(L, a_cache=None), FAKE, FAKE, 10, FAKE, None, stream=0) == 1
    assert _code(L, f, lay, FAKE, None, 0, FAKE, None, stream=0) == 0         # k = 0: no-op, nothing enqueued


def test_plain_c_caller_compiles_links_and_runs(tmp_path):
    """The header is valid C99 (warnings are errors) and a C program links the
    library and gets the documented results from the calls that need no GPU
    (tests/c/abi_client.c)."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    exe = str(tmp_path / "abi_client")
    libdir = os.path.dirname(LIBSO)
    r = subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I", os.path.join(ROOT, "include"),
                        os.path.join(ROOT, "tests", "c", "abi_client.c"), "-o", exe, "-L", libdir, "-lchipmunk",
                        f"-Wl,-rpath,{libdir}"], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    r = subprocess.run([exe, source_digest()], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.stdout, r.stderr[-3000:])
