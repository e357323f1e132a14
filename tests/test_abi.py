"""The C-ABI library loads, exports every declared symbol and rejects bad
arguments on the host, before any launch (no GPU needed: no call here reaches
a kernel)."""
import ctypes
import os
import re

import pytest

import decoder_shared_kv_amd as dk
from decoder_shared_kv_amd import xattn as X

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    inc = os.path.join(ROOT, "include")
    for f in sorted(os.listdir(inc)):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(yoco_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    return dk.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(X.EXPORTS) <= set(names), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for s in range(5):
        assert lib.yoco_status_string(s)
    assert lib.yoco_status_string(99) == b"unknown status"


FAKE = 1 << 20  # a 16-byte aligned fake device address; never dereferenced on the host


def _cache(**kw):
    d = dict(k=FAKE, v=FAKE, pool_rows=100, seq_start=FAKE, seq_len=FAKE, seq_cap=FAKE)
    d.update(kw)
    return X.KvCache(**d)


def _dims(**kw):
    d = dict(batch=1, num_q_heads=4, num_kv_heads=2, head_dim=128, dtype=1, scale=0.1)
    d.update(kw)
    return X.Dims(**d)


@pytest.mark.parametrize("bad,code", [
    (dict(batch=0), 1), (dict(num_q_heads=3, num_kv_heads=2), 1), (dict(num_kv_heads=0), 1),
    (dict(head_dim=96), 2), (dict(dtype=7), 2), (dict(scale=float("inf")), 1), (dict(scale=float("nan")), 1),
    (dict(scale=0.0), 1), (dict(scale=-0.5), 1),
])
def test_dims_rejected_everywhere(lib, bad, code):
    dims, cache = _dims(**bad), _cache()
    ws = ctypes.c_size_t(0)
    assert lib.yoco_xattn_workspace_size(ctypes.byref(dims), 10, 1, ctypes.byref(ws)) == code
    assert lib.yoco_xattn_workspace_size(ctypes.byref(dims), 10, 0, ctypes.byref(ws)) == code
    assert lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, 10, 10, FAKE, None, None, 0,
                                  None) == code
    assert lib.yoco_xattn_decode(ctypes.byref(dims), ctypes.byref(cache), FAKE, 10, 0, FAKE, None, FAKE, 1 << 30,
                                 None) == code
    assert lib.yoco_kv_append(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, None, None) == code


@pytest.mark.parametrize("bad", [dict(k=None), dict(v=None), dict(k=FAKE + 2), dict(seq_start=None),
                                 dict(seq_len=None), dict(seq_cap=None), dict(pool_rows=-1), dict(seq_start=FAKE + 4)])
def test_cache_rejected(lib, bad):
    dims, cache = _dims(), _cache(**bad)
    assert lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, 10, 10, FAKE, None, None, 0,
                                  None) == 1
    assert lib.yoco_kv_append(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, None, None) == 1
    assert lib.yoco_xattn_decode(ctypes.byref(dims), ctypes.byref(cache), FAKE, 10, 0, FAKE, None, FAKE, 1 << 30,
                                 None) == 1


def test_null_structs(lib):
    cache, dims = _cache(), _dims()
    assert lib.yoco_xattn_prefill(None, ctypes.byref(cache), FAKE, FAKE, 1, 1, FAKE, None, None, 0, None) == 1
    assert lib.yoco_xattn_prefill(ctypes.byref(dims), None, FAKE, FAKE, 1, 1, FAKE, None, None, 0, None) == 1
    assert lib.yoco_xattn_workspace_size(ctypes.byref(dims), 5, 1, None) == 1


def test_prefill_argument_checks(lib):
    dims, cache = _dims(), _cache()
    P = lambda *a: lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(cache), *a[:-1], None, 0, a[-1])  # noqa: E731
    assert P(None, FAKE, 10, 10, FAKE, None, None) == 1          # q
    assert P(FAKE, None, 10, 10, FAKE, None, None) == 1          # cu_seqlens
    assert P(FAKE, FAKE, 10, 10, None, None, None) == 1          # out
    assert P(FAKE + 8, FAKE, 10, 10, FAKE, None, None) == 1      # misaligned q
    assert P(FAKE, FAKE, 10, 10, FAKE + 8, None, None) == 1      # misaligned out
    assert P(FAKE, FAKE, 10, 10, FAKE, FAKE + 2, None) == 1      # misaligned lse
    assert P(FAKE, FAKE, -1, 10, FAKE, None, None) == 1          # max_q_len
    assert P(FAKE, FAKE, 10, -5, FAKE, None, None) == 1          # total_q
    assert P(FAKE, FAKE, 10, 0, FAKE, None, None) == 0           # nothing to do, nothing launched
    # the work-queue workspace: 2 KB for bf16 (0 for fp32), 16-byte aligned
    need = ctypes.c_size_t(0)
    assert lib.yoco_xattn_workspace_size(ctypes.byref(dims), 1 << 20, 0, ctypes.byref(need)) == 0 and need.value == 2048
    assert lib.yoco_xattn_workspace_size(ctypes.byref(_dims(dtype=0)), 10, 0, ctypes.byref(need)) == 0
    assert need.value == 0
    Q = lambda *a: lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, 10, 10, FAKE, None,
                                          *a, None)  # noqa: E731
    assert Q(FAKE, 2047) == 3                                     # too small
    assert Q(FAKE + 8, 2048) == 3                                 # misaligned
    assert lib.yoco_xattn_prefill(ctypes.byref(dims), ctypes.byref(cache), FAKE, FAKE, 10, 0, FAKE, None, FAKE, 2048,
                                  None) == 0                     # nothing to do, nothing launched


def test_decode_workspace_checks(lib):
    dims, cache = _dims(batch=2), _cache()
    need = ctypes.c_size_t(0)
    assert lib.yoco_xattn_workspace_size(ctypes.byref(dims), 5000, 1, ctypes.byref(need)) == 0
    assert need.value > 0
    D = lambda *a: lib.yoco_xattn_decode(ctypes.byref(dims), ctypes.byref(cache), *a)  # noqa: E731
    assert D(FAKE, 5000, 0, FAKE, None, None, need.value, None) == 3
    assert D(FAKE, 5000, 0, FAKE, None, FAKE, need.value - 1, None) == 3
    assert D(FAKE, 5000, 0, FAKE, None, FAKE + 4, need.value, None) == 3
    assert D(FAKE, -1, 0, FAKE, None, FAKE, need.value, None) == 1
    assert D(FAKE, 5000, -3, FAKE, None, FAKE, need.value, None) == 1
    assert D(None, 5000, 0, FAKE, None, FAKE, need.value, None) == 1
    assert D(FAKE, 5000, 0, FAKE + 8, None, FAKE, need.value, None) == 1


def test_append_argument_checks(lib):
    dims, cache = _dims(), _cache()
    A = lambda *a: lib.yoco_kv_append(ctypes.byref(dims), ctypes.byref(cache), *a)  # noqa: E731
    assert A(None, FAKE, None, None) == 1
    assert A(FAKE, None, None, None) == 1
    assert A(FAKE + 2, FAKE, None, None) == 1
    assert A(FAKE, FAKE, FAKE + 1, None) == 1


def test_window_argument_checks(lib):
    dims, cache = _dims(batch=2), _cache()
    need = ctypes.c_size_t(0)
    assert lib.yoco_xattn_workspace_size(ctypes.byref(dims), 5000, 1, ctypes.byref(need)) == 0
    PW = lambda *a: lib.yoco_xattn_prefill_window(ctypes.byref(dims), ctypes.byref(cache), *a[:-1], None, 0,
                                                  a[-1])  # noqa: E731
    DW = lambda *a: lib.yoco_xattn_decode_window(ctypes.byref(dims), ctypes.byref(cache), *a)  # noqa: E731
    for w in (0, -1, -1024):
        assert PW(FAKE, FAKE, 10, 10, w, FAKE, None, None) == 1
        assert DW(FAKE, 5000, 0, w, FAKE, None, FAKE, need.value, None) == 1
    # the other checks are the unwindowed calls'
    assert PW(None, FAKE, 10, 10, 64, FAKE, None, None) == 1
    assert PW(FAKE, FAKE, 10, 0, 64, FAKE, None, None) == 0       # nothing to do, nothing launched
    assert DW(FAKE, 5000, 0, 64, FAKE, None, FAKE + 4, need.value, None) == 3
    assert DW(FAKE, 5000, 0, 64, FAKE, None, None, need.value, None) == 3
    assert lib.yoco_xattn_prefill_window(ctypes.byref(_dims(head_dim=96)), ctypes.byref(cache), FAKE, FAKE, 10,
                                         10, 64, FAKE, None, None, 0, None) == 2
    A = lambda *a: lib.yoco_kv_append_ring(ctypes.byref(dims), ctypes.byref(cache), *a)  # noqa: E731
    assert A(None, FAKE, None, None) == 1
    assert A(FAKE, FAKE + 2, None, None) == 1
    assert A(FAKE, FAKE, FAKE + 1, None) == 1


def test_producer_argument_checks(lib):
    dims, cache = _dims(batch=2), _cache()
    res = X.Residual(None, FAKE, 35.0, (ctypes.c_float * 2)(0.0, 1 / 35), (ctypes.c_float * 2)(0.0, 1 / 35))
    PA = lambda d, *a: lib.yoco_kv_project_append(ctypes.byref(d), ctypes.byref(cache), *a)  # noqa: E731
    assert PA(_dims(dtype=0), FAKE, FAKE, 10, 256, FAKE, 1e-6, None, None, None) == 2   # fp32: not built
    assert PA(dims, FAKE, FAKE, 10, 100, FAKE, 1e-6, None, None, None) == 2             # d_model % 64
    assert PA(dims, FAKE, FAKE, 10, 0, FAKE, 1e-6, None, None, None) == 2
    assert PA(dims, None, FAKE, 10, 256, FAKE, 1e-6, None, None, None) == 1
    assert PA(dims, FAKE, None, 10, 256, FAKE, 1e-6, None, None, None) == 1
    assert PA(dims, FAKE, FAKE, 10, 256, None, 1e-6, None, None, None) == 1
    assert PA(dims, FAKE + 8, FAKE, 10, 256, FAKE, 1e-6, None, None, None) == 1
    assert PA(dims, FAKE, FAKE, -1, 256, FAKE, 1e-6, None, None, None) == 1
    assert PA(dims, FAKE, FAKE, 10, 256, FAKE, -1.0, None, None, None) == 1
    assert PA(dims, FAKE, FAKE, 10, 256, FAKE, float("nan"), None, None, None) == 1
    assert PA(dims, FAKE, FAKE, 10, 256, FAKE, 1e-6, ctypes.byref(res), None, None) == 1   # k1 missing
    PK = lambda d, *a: lib.yoco_kv_project_pack(ctypes.byref(d), *a)  # noqa: E731
    assert PK(_dims(dtype=0), 256, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert PK(dims, 96, FAKE, FAKE, FAKE, FAKE, None) == 2
    assert PK(dims, 256, None, FAKE, FAKE, FAKE, None) == 1
    assert PK(dims, 256, FAKE, FAKE, FAKE, FAKE + 2, None) == 1


def test_gret_argument_checks(lib):
    gd = X.GretDims(2, 4, 128, 1)
    n = ctypes.c_size_t(0)
    assert lib.yoco_gret_workspace_size(ctypes.byref(gd), 1000, ctypes.byref(n)) == 0 and n.value > 0
    assert lib.yoco_gret_workspace_size(ctypes.byref(X.GretDims(2, 4, 96, 1)), 1000, ctypes.byref(n)) == 2
    assert lib.yoco_gret_workspace_size(ctypes.byref(X.GretDims(2, 4, 128, 0)), 1000, ctypes.byref(n)) == 2
    assert lib.yoco_gret_workspace_size(ctypes.byref(X.GretDims(0, 4, 128, 1)), 1000, ctypes.byref(n)) == 1
    assert lib.yoco_gret_workspace_size(ctypes.byref(gd), -1, ctypes.byref(n)) == 1
    need = ctypes.c_size_t(0)
    lib.yoco_gret_workspace_size(ctypes.byref(gd), 1000, ctypes.byref(need))
    G = lambda *a: lib.yoco_gret_prefill(ctypes.byref(gd), *a)  # noqa: E731
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, 1000, None, None, FAKE, FAKE, need.value, None]
    for i in (0, 1, 2, 3, 4, 8):                        # q, k, v, gamma, cu_seqlens, out
        args = list(ok)
        args[i] = None
        assert G(*args) == 1, i
    args = list(ok); args[0] = FAKE + 8; assert G(*args) == 1          # misaligned q
    args = list(ok); args[6] = FAKE + 4; assert G(*args) == 1          # misaligned state_in
    args = list(ok); args[5] = -1; assert G(*args) == 1                # total_rows
    args = list(ok); args[9] = None; assert G(*args) == 3              # workspace
    args = list(ok); args[10] = need.value - 1; assert G(*args) == 3
    args = list(ok); args[5] = 2000; assert G(*args) == 3              # more rows than the workspace was sized for
    args = list(ok); args[5] = 0; assert G(*args) == 0                 # nothing to do, no state: no launch
    D = lambda *a: lib.yoco_gret_decode(ctypes.byref(gd), *a)  # noqa: E731
    assert D(FAKE, FAKE, FAKE, FAKE, None, FAKE, None) == 1
    assert D(FAKE, FAKE, FAKE, FAKE, FAKE + 4, FAKE, None) == 1
    assert lib.yoco_gret_decode(ctypes.byref(X.GretDims(2, 4, 128, 0)), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                None) == 2
    # more rows never need less workspace; the slots bound the chunks of any split of the rows
    sizes = []
    for m in (1, 255, 256, 257, 10000):
        lib.yoco_gret_workspace_size(ctypes.byref(gd), m, ctypes.byref(n))
        sizes.append(n.value)
    assert sizes == sorted(sizes)
    rows, batch = 1000, 2
    slots = (rows + 255) // 256 + batch
    for split in [(0, 1000), (1, 999), (255, 745), (257, 743), (500, 500), (1000, 0)]:
        assert sum((x + 255) // 256 for x in split) <= slots, split


def test_split_plan():
    # bf16: 512 workgroups over one or two (KV head, head chunk) columns, 1024
    # over more; each share is one equal part of all sequences' 128-row blocks
    s, r = dk.decode_splits(8, 16, 2, 128, X.torch.bfloat16, 131072)
    assert s == 256 and r == 4096
    s, r = dk.decode_splits(1, 16, 2, 128, X.torch.bfloat16, 1048640, 1048640)
    assert s == 256 and s * r >= 1048640 and r % 128 == 0
    s, r = dk.decode_splits(4, 32, 4, 128, X.torch.bfloat16, 131072)
    assert s == 256 and r == 2048
    # few blocks: one share per block, never a planned-empty share
    s, r = dk.decode_splits(1, 4, 1, 64, X.torch.float32, 1)
    assert s == 1 and r == 128
    s, r = dk.decode_splits(3, 32, 1, 128, X.torch.bfloat16, 0)
    assert s == 1
    s, r = dk.decode_splits(2, 16, 2, 128, X.torch.bfloat16, 1000, 1300)
    assert s == 11 and r == 128
    # a total hint above B x max_kv_len counts as B x max_kv_len
    assert dk.decode_splits(2, 16, 2, 128, X.torch.bfloat16, 1000, 10 ** 9) == (16, 128)
    # g = 32: two head chunks per KV head
    s, r = dk.decode_splits(1, 32, 1, 128, X.torch.bfloat16, 1 << 20)
    assert s == 256


def test_workspace_is_monotone_and_bounds_every_plan():
    import torch
    prev = 0
    for n in [0, 1, 127, 128, 129, 1000, 4096, 65535, 131071, 131072, 131085, 131200, 1 << 20, (1 << 20) + 64]:
        ws = dk.workspace_size(8, 16, 2, 128, torch.bfloat16, n)
        assert ws >= prev, (n, ws)
        prev = ws
        for total in [0, n, 2 * n + 5, 8 * n, 3 * n // 2, 100 * n + 7]:
            for m in {n, n // 2, max(n - 1, 0)}:
                s, r = dk.decode_splits(8, 16, 2, 128, torch.bfloat16, m, total)
                # partials [Hq, shares + B, d + 2] fp32 and [B, 2] int32
                assert s * r >= max(m, 1) and ws >= 16 * (s + 8) * (128 + 2) * 4 + 8 * 8, (n, m, total, s, r, ws)


def test_split_plan_counts_all_rows():
    import torch
    # 16 ragged sequences: the shares follow the total rows; every workgroup of a
    # column gets the same number of blocks, so the ~1024 workgroups are balanced
    lens = [13257, 14478, 45818, 11785, 13140, 8156, 31001, 13071, 23276, 22166, 17936, 22454, 5776, 11113, 5199, 18047]
    s, r = dk.decode_splits(16, 32, 8, 128, torch.bfloat16, max(lens), sum(lens))
    blocks = -(-sum(lens) // 128)
    assert s * 8 == 1024 and r == -(-blocks // s) * 128, (s, r)
    s0, r0 = dk.decode_splits(16, 32, 8, 128, torch.bfloat16, max(lens), 0)
    assert s0 == s and r0 > r


def test_missing_library_fails_loudly():
    """Without the built library the binding raises; there is no other path to fall back on."""
    import subprocess
    import sys
    code = ("import decoder_shared_kv_amd.xattn as x\n"
            "try:\n"
            "    x.load_library('/nonexistent/libyoco_xattn.so')\n"
            "except OSError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    print('loaded')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "is not built" in r.stdout


def test_noalloc_decode_argument_checks(lib):
    """The no-allocation decode rejects bad arguments and plans whose partials
    exceed its scratch on the host, before it looks for a device."""
    dims, cache = _dims(batch=2), _cache()
    N = lambda d, *a: lib.yoco_xattn_decode_noalloc(ctypes.byref(d), ctypes.byref(cache), *a)  # noqa: E731
    assert N(dims, None, 5000, 0, FAKE, None, None) == 1          # q
    assert N(dims, FAKE, 5000, 0, None, None, None) == 1          # out
    assert N(dims, FAKE, -1, 0, FAKE, None, None) == 1            # max_kv_len
    assert N(_dims(batch=0), FAKE, 5000, 0, FAKE, None, None) == 1
    # a plan needing more than the scratch: thousands of sequences of 128 query heads
    big = _dims(batch=4096, num_q_heads=128, num_kv_heads=8)
    need = ctypes.c_size_t(0)
    assert lib.yoco_xattn_workspace_size(ctypes.byref(big), 100000, 1, ctypes.byref(need)) == 0
    assert need.value > X.NOALLOC_SCRATCH_BYTES
    assert N(big, FAKE, 100000, 0, FAKE, None, None) == 3
    # the header's constant and the binding's agree
    text = open(os.path.join(ROOT, "include", "yoco_xattn.h")).read()
    m = re.search(r"#define YOCO_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == X.NOALLOC_SCRATCH_BYTES


def test_binding_rejects_bad_tensors():
    """The binding checks dtype, shape, device and contiguity before any ABI
    call (all cases here fail before the library is reached)."""
    import torch
    k = torch.zeros(16, 2, 64, dtype=torch.bfloat16)
    meta = dict(seq_start=torch.zeros(1, dtype=torch.int64), seq_len=torch.ones(1, dtype=torch.int32),
                seq_cap=torch.full((1,), 16, dtype=torch.int32))
    good = dk.SharedKV(k, k.clone(), **meta)
    cases = [
        dk.SharedKV(k, k.clone().to(torch.float32), **meta),                       # v dtype
        dk.SharedKV(k, k.clone()[:8], **meta),                                      # v shape
        dk.SharedKV(k, k.clone().transpose(0, 1).contiguous().transpose(0, 1), **meta),  # v strided
        dk.SharedKV(k, k.clone(), **{**meta, "seq_start": torch.zeros(1, dtype=torch.int32)}),
        dk.SharedKV(k, k.clone(), **{**meta, "seq_len": torch.ones(1, dtype=torch.int64)}),
        dk.SharedKV(k, k.clone(), **{**meta, "seq_cap": torch.ones(2, dtype=torch.int32)}),
    ]
    for c in cases:
        with pytest.raises(dk.YocoError):
            c.validate()
    q = torch.zeros(4, 4, 64, dtype=torch.bfloat16)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(dk.YocoError):      # q in another dtype than the cache
        dk.xattn_prefill(good, q.float(), cu, 4, 0.1)
    with pytest.raises(dk.YocoError):      # q not contiguous
        dk.xattn_prefill(good, torch.zeros(4, 64, 4, dtype=torch.bfloat16).transpose(1, 2), cu, 4, 0.1)
    with pytest.raises(dk.YocoError):      # int64 cu_seqlens
        dk.xattn_prefill(good, q, cu.long(), 4, 0.1)
    with pytest.raises(dk.YocoError):      # lse of the wrong shape
        dk.xattn_prefill(good, q, cu, 4, 0.1, lse=torch.zeros(4, 5))
    with pytest.raises(dk.YocoError):      # decode: one query row per sequence
        dk.xattn_decode(good, q, 4, 0.1, torch.zeros(64, dtype=torch.uint8))
    with pytest.raises(dk.YocoError):      # decode workspace of the wrong dtype
        dk.xattn_decode(good, q[:1], 4, 0.1, torch.zeros(64, dtype=torch.float32))
    with pytest.raises(dk.YocoError):      # the no-allocation decode needs out
        dk.xattn_decode_noalloc(good, q[:1], 4, 0.1, None)
    with pytest.raises(dk.YocoError):      # appended rows of the wrong shape
        dk.kv_append(good, torch.zeros(1, 2, 32, dtype=torch.bfloat16), torch.zeros(1, 2, 32, dtype=torch.bfloat16))
    with pytest.raises(dk.YocoError):      # gRet gates in bf16
        dk.gret_decode(q[:1], q[:1], q[:1], torch.zeros(1, 4, dtype=torch.bfloat16),
                       torch.zeros(1, 4, 64, 64))


def test_gret_workspace_never_shrinks(lib):
    """The gRet prefill groups chunks into longer segments as the rows grow, so a
    call with fewer rows can need more segment slots; the reported size covers
    every smaller row count, so a workspace sized once for the longest input
    serves every shorter one."""
    n = ctypes.c_size_t(0)
    for heads, batch, dim in ((1, 1, 128), (16, 1, 128), (16, 5, 64), (64, 3, 128)):
        gd = X.GretDims(batch, heads, dim, 1)
        rows = set(range(0, 20000, 97))
        for seg in (1, 2, 4, 8, 16, 32, 64):          # around the row counts where segments double
            edge = 512 * seg * 256 // heads
            rows.update(r for r in range(edge - 600, edge + 600, 37) if r >= 0)
        rows.update(range(0, 3_000_000, 65_537))
        last = 0
        for r in sorted(rows):
            assert lib.yoco_gret_workspace_size(ctypes.byref(gd), r, ctypes.byref(n)) == 0
            assert n.value >= last, (heads, batch, r, n.value, last)
            last = n.value
