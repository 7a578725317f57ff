"""The C-ABI library loads, exports what the header declares, and rejects bad
arguments on the host.  CPU only: nothing here launches a kernel."""

import ctypes
import os
import re

import numpy as np
import pytest

from sparse_attention_indexer_row_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "topk_select.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b(topk_\w+)\s*\(", text, flags=re.M)
    return names


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_declares_what_the_binding_declares():
    assert tuple(declared_functions()) == _lib.EXPORTS


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_constants_match_header():
    text = open(HEADER).read()
    for cname in ("TOPK_OK", "TOPK_EINVAL", "TOPK_EK_RANGE", "TOPK_EWORKSPACE", "TOPK_ESPLIT",
                  "TOPK_ELAUNCH", "TOPK_EDEVICE", "TOPK_EALLOC", "TOPK_MAX_K", "TOPK_MAX_SPLIT",
                  "TOPK_MAX_POOL_SLOTS", "TOPK_MAX_K_RADIX", "TOPK_MAX_K_STREAM",
                  "TOPK_MAX_K_POOLED", "TOPK_PATH_STREAM", "TOPK_PATH_RADIX"):
        m = re.search(rf"#define {cname} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == getattr(_lib, cname), cname


def test_options_and_plan_struct_sizes():
    assert ctypes.sizeof(_lib.TopkOptions) == 32
    assert ctypes.sizeof(_lib.TopkPlan) == 40


FAKE = 0x10000  # a non-null, 256-aligned address that is never dereferenced


@pytest.mark.parametrize("args,status", [
    ((FAKE, None, -1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # rows < 0
    ((FAKE, None, 1, 0, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),        # n < 1
    ((FAKE, None, 1, 16, 0, FAKE, FAKE, None), _lib.TOPK_EK_RANGE),     # k < 1
    ((FAKE, None, 1, 16, 4097, FAKE, FAKE, None), _lib.TOPK_EK_RANGE),  # k > max
    ((None, None, 1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),       # null scores
    ((FAKE, None, 1, 16, 4, None, FAKE, None), _lib.TOPK_EINVAL),       # null out_vals
    ((FAKE, None, 1, 16, 4, FAKE, None, None), _lib.TOPK_EINVAL),       # null out_idx
    ((FAKE + 2, None, 1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),   # misaligned scores
    ((FAKE, FAKE + 1, 1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),   # misaligned lengths
    ((None, None, 0, 16, 4, None, None, None), _lib.TOPK_OK),           # rows == 0: no-op
])
def test_select_argument_errors(lib, args, status):
    assert lib.topk_select(*args) == status


def test_split_and_ex_argument_errors(lib):
    a = (FAKE, None, 4, 4096, 8, FAKE, FAKE)
    assert lib.topk_select_split(*a, -1, FAKE, 1 << 20, None) == _lib.TOPK_ESPLIT
    assert lib.topk_select_split(*a, 1025, FAKE, 1 << 20, None) == _lib.TOPK_ESPLIT
    assert lib.topk_select_split(*a, 2, FAKE + 8, 1 << 20, None) == _lib.TOPK_EWORKSPACE
    o = _lib.TopkOptions()
    o.waves = 1
    assert lib.topk_select_ex(*a, ctypes.byref(o), None, 0, None) == _lib.TOPK_EINVAL
    o.waves = 9
    assert lib.topk_select_ex(*a, ctypes.byref(o), None, 0, None) == _lib.TOPK_EINVAL
    o.waves = 5   # k = 2048 lists run at most four waves
    big = (FAKE, None, 4, 4096, 2048, FAKE, FAKE)
    assert lib.topk_select_ex(*big, ctypes.byref(o), None, 0, None) == _lib.TOPK_EINVAL
    o.waves, o.watermark = 4, -3
    assert lib.topk_select_ex(*a, ctypes.byref(o), None, 0, None) == _lib.TOPK_EINVAL
    o.watermark, o.split = 0, 2000
    assert lib.topk_select_ex(*a, ctypes.byref(o), None, 0, None) == _lib.TOPK_ESPLIT
    o.split, o.flags = 0, 4
    assert lib.topk_select_ex(*a, ctypes.byref(o), None, 0, None) == _lib.TOPK_EINVAL


@pytest.mark.parametrize("args,status", [
    # scores, lengths, rows, n, group, keep, pinned, out_vals, out_idx, stream
    ((FAKE, None, -1, 64, 8, 16, 2, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # rows < 0
    ((FAKE, None, 1, 0, 8, 16, 2, FAKE, FAKE, None), _lib.TOPK_EINVAL),        # n < 1
    ((FAKE, None, 1, 64, 0, 16, 2, FAKE, FAKE, None), _lib.TOPK_EINVAL),       # group < 1
    ((FAKE, None, 1, 64, 8, 0, 0, FAKE, FAKE, None), _lib.TOPK_EINVAL),        # keep < 1
    ((FAKE, None, 1, 64, 8, 16, -1, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # pinned < 0
    ((FAKE, None, 1, 64, 8, 16, 17, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # pinned > keep
    ((FAKE, None, 1, 64, 8, 4200, 51, FAKE, FAKE, None), _lib.TOPK_EK_RANGE),  # keep - pinned > max
    ((None, None, 1, 64, 8, 16, 2, FAKE, FAKE, None), _lib.TOPK_EINVAL),       # null scores
    ((FAKE, None, 1, 64, 8, 16, 2, None, FAKE, None), _lib.TOPK_EINVAL),       # null out_vals
    ((FAKE, None, 1, 64, 8, 16, 2, FAKE, None, None), _lib.TOPK_EINVAL),       # null out_idx
    ((FAKE, FAKE + 2, 1, 64, 8, 16, 2, FAKE, FAKE, None), _lib.TOPK_EINVAL),   # misaligned lengths
    ((FAKE, None, 0, 64, 8, 16, 2, None, None, None), _lib.TOPK_OK),           # no rows
])
def test_block_pool_argument_errors(lib, args, status):
    assert lib.topk_block_pool(*args) == status


@pytest.mark.parametrize("args,status", [
    # pool_scores, pool_idx, lengths, rows, n, group, keep, k, out_vals, out_idx, stream
    ((FAKE, FAKE, None, -1, 64, 8, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),     # rows < 0
    ((FAKE, FAKE, None, 1, 0, 8, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),       # n < 1
    ((FAKE, FAKE, None, 1, 64, 0, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # group < 1
    ((FAKE, FAKE, None, 1, 64, 8, 0, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),       # keep < 1
    ((FAKE, FAKE, None, 1, 64, 8, 8193, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),    # keep > max
    ((FAKE, FAKE, None, 1, 64, 1 << 20, 4096, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),  # too long
    ((FAKE, FAKE, None, 1, 64, 8, 16, 0, FAKE, FAKE, None), _lib.TOPK_EK_RANGE),    # k < 1
    ((FAKE, FAKE, None, 1, 64, 8, 16, 2049, FAKE, FAKE, None), _lib.TOPK_EK_RANGE), # k > pooled max
    ((None, FAKE, None, 1, 64, 8, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # null scores
    ((FAKE, None, None, 1, 64, 8, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # null pool
    ((FAKE, FAKE, None, 1, 64, 8, 16, 4, None, FAKE, None), _lib.TOPK_EINVAL),      # null out
    ((FAKE, FAKE + 1, None, 1, 64, 8, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),  # misaligned
    ((FAKE, FAKE, None, 0, 64, 8, 16, 4, None, None, None), _lib.TOPK_OK),          # no rows
])
def test_pooled_select_argument_errors(lib, args, status):
    assert lib.topk_pooled_select(*args) == status


@pytest.mark.parametrize("args,status", [
    ((FAKE, None, -1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),      # rows < 0
    ((FAKE, None, 1, 0, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),        # n < 1
    ((FAKE, None, 1, 16, 0, FAKE, FAKE, None), _lib.TOPK_EK_RANGE),     # k < 1
    ((FAKE, None, 1, 16, 8193, FAKE, FAKE, None), _lib.TOPK_EK_RANGE),  # k > 8192
    ((None, None, 1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),       # null scores
    ((FAKE, None, 1, 16, 4, None, FAKE, None), _lib.TOPK_EINVAL),       # null out_vals
    ((FAKE + 2, None, 1, 16, 4, FAKE, FAKE, None), _lib.TOPK_EINVAL),   # misaligned scores
    ((FAKE, None, 0, 16, 8192, None, None, None), _lib.TOPK_OK),        # no rows
])
def test_radix_argument_errors(lib, args, status):
    assert lib.topk_select_radix(*args) == status


def test_sparse_decode_argument_errors(lib):
    import ctypes as C
    f = lib.topk_sparse_decode
    ok = dict(q=FAKE, kv=FAKE, idx=FAKE, rows=2, heads=16, n=100, k=8, dqk=64, dv=64, scale=0.5,
              out=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["kv"], a["idx"], a["rows"], a["heads"], a["n"], a["k"], a["dqk"],
                 a["dv"], C.c_float(a["scale"]), a["out"], None)

    assert call(rows=-1) == _lib.TOPK_EINVAL
    assert call(heads=8) == _lib.TOPK_EINVAL           # not a multiple of 16
    assert call(n=0) == _lib.TOPK_EINVAL
    assert call(dqk=72) == _lib.TOPK_EINVAL            # not a multiple of 16
    assert call(dqk=2048, dv=64) == _lib.TOPK_EINVAL   # dqk above 1024
    assert call(dv=96) == _lib.TOPK_EINVAL             # not a multiple of 64
    assert call(dqk=64, dv=128) == _lib.TOPK_EINVAL    # dv above dqk
    assert call(scale=float("nan")) == _lib.TOPK_EINVAL
    assert call(scale=float("inf")) == _lib.TOPK_EINVAL
    assert call(scale=float("-inf")) == _lib.TOPK_EINVAL
    assert call(k=0) == _lib.TOPK_EK_RANGE
    assert call(k=8193) == _lib.TOPK_EK_RANGE
    assert call(q=None) == _lib.TOPK_EINVAL
    assert call(kv=FAKE + 8) == _lib.TOPK_EINVAL       # not 16-byte aligned
    assert call(rows=0, q=None, kv=None, idx=None, out=None) == _lib.TOPK_OK


def test_workspace_init_and_probe_argument_errors(lib):
    assert lib.topk_workspace_init(None, 256, None) == _lib.TOPK_EWORKSPACE
    assert lib.topk_workspace_init(FAKE + 16, 256, None) == _lib.TOPK_EWORKSPACE
    assert lib.topk_workspace_init(FAKE, 100, None) == _lib.TOPK_EWORKSPACE
    assert lib.topk_workspace_init(FAKE, 0, None) == _lib.TOPK_OK
    assert lib.topk_probe_read(FAKE, 100, FAKE, None) == _lib.TOPK_EINVAL
    cfg = lib.topk_probe_read_cfg
    assert cfg(FAKE, 1 << 20, 4, 128, 4, 1, 0, FAKE, None) == _lib.TOPK_EINVAL    # threads
    assert cfg(FAKE, 1 << 20, 4, 256, 3, 1, 0, FAKE, None) == _lib.TOPK_EINVAL    # loads
    assert cfg(FAKE, 1000, 4, 256, 4, 1, 0, FAKE, None) == _lib.TOPK_EINVAL       # share size
    assert cfg(FAKE, 1 << 20, 4, 256, 4, 1, 200 << 10, FAKE, None) == _lib.TOPK_EINVAL  # LDS
    assert cfg(FAKE + 8, 1 << 20, 4, 256, 4, 1, 0, FAKE, None) == _lib.TOPK_EINVAL  # alignment
    assert cfg(FAKE, 1 << 20, 0, 256, 4, 1, 0, FAKE, None) == _lib.TOPK_OK        # nothing
    assert lib.topk_probe_copy(FAKE, None, 256, None) == _lib.TOPK_EINVAL
    assert lib.topk_probe_copy(FAKE, FAKE, 0, None) == _lib.TOPK_OK


def test_strerror(lib):
    assert lib.topk_strerror(0) == b"ok"
    assert lib.topk_strerror(_lib.TOPK_EK_RANGE) == b"k out of range"
    assert lib.topk_strerror(12345) == b"unknown status"


def _plan(lib, rows, n, k, split=0, waves=0, watermark=0):
    o = _lib.TopkOptions()
    o.split, o.waves, o.watermark = split, waves, watermark
    p = _lib.TopkPlan()
    assert lib.topk_plan(rows, n, k, ctypes.byref(o), ctypes.byref(p)) == 0
    return p


def test_plan_list_sizes_and_lds(lib):
    for k, words in [(1, 64), (64, 64), (65, 128), (512, 512), (513, 1024), (1000, 1024),
                     (2048, 2048)]:
        p = _plan(lib, 4, 1 << 16, k)
        assert p.list_words == words
        assert p.lds_bytes == (8 * (2 * (p.waves - 1) * p.tray_words + 2 * words + 1024 + 64)
                               + 4 * 3 * 256)
        assert p.lds_bytes <= 160 * 1024
        assert p.tray_words == p.watermark + 1024


def test_plan_rejects_what_does_not_fit(lib):
    # eight waves fit for k <= 1024; k = 2048 lists run at most four waves
    assert _plan(lib, 4, 1 << 16, 512, waves=8).waves == 8
    o = _lib.TopkOptions()
    o.waves = 8
    p = _lib.TopkPlan()
    assert lib.topk_plan(4, 1 << 16, 2048, ctypes.byref(o), ctypes.byref(p)) == _lib.TOPK_EINVAL
    o.waves, o.watermark = 8, 4096   # trays of 4096 + 1024 words per streamer exceed LDS
    assert lib.topk_plan(4, 1 << 16, 512, ctypes.byref(o), ctypes.byref(p)) == _lib.TOPK_EINVAL


def test_plan_split_policy(lib):
    cus = _plan(lib, 1, 1024, 1).compute_units
    big = _plan(lib, 128, 1 << 20, 512)
    assert big.split * 128 >= cus            # enough workgroups to cover the chip
    one = _plan(lib, 1, 1 << 20, 512)
    assert one.split > 1 and one.workspace_bytes > 0
    small = _plan(lib, 4, 16384, 512)       # 16 blocks per row: no room to split
    assert small.split == 1 and small.workspace_bytes == 0
    forced = _plan(lib, 4, 16384, 512, split=3)
    assert forced.split == 3
    assert lib.topk_split_workspace_bytes(4, 16384, 512, 3) == forced.workspace_bytes
    assert forced.workspace_bytes >= 4 * 3 * 512 * 8
    assert lib.topk_split_workspace_bytes(4, 16384, 0, 3) == 0


@pytest.mark.parametrize("nb", [1, 2, 3, 5, 16, 100, 128, 255, 256, 257, 1000, 1024, 4097])
def test_visit_order_is_a_permutation(nb):
    out = np.empty(nb, dtype=np.int32)
    lib = _lib.load()
    for seed, row in [(0, 0), (1, 0), (0, 7), (123456789, 3)]:
        assert lib.topk_visit_order(seed, row, nb, out.ctypes.data) == 0
        assert np.array_equal(np.sort(out), np.arange(nb))


def test_visit_order_depends_on_seed_and_row_only():
    lib = _lib.load()
    a = np.empty(1024, dtype=np.int32)
    b = np.empty(1024, dtype=np.int32)
    lib.topk_visit_order(5, 9, 1024, a.ctypes.data)
    lib.topk_visit_order(5, 9, 1024, b.ctypes.data)
    assert np.array_equal(a, b)
    lib.topk_visit_order(6, 9, 1024, b.ctypes.data)
    assert not np.array_equal(a, b)
    lib.topk_visit_order(5, 10, 1024, b.ctypes.data)
    assert not np.array_equal(a, b)


def test_visit_order_looks_shuffled():
    # a sequential or strided walk would make ascending rows expensive; check
    # that the first block visited is spread over the range and that the walk
    # has few ascending runs' worth of records
    lib = _lib.load()
    nb = 1024
    out = np.empty(nb, dtype=np.int32)
    firsts = []
    records = []
    for row in range(400):
        lib.topk_visit_order(0, row, nb, out.ctypes.data)
        firsts.append(out[0])
        records.append(int(np.sum(out == np.maximum.accumulate(out))))
    hist = np.bincount(np.array(firsts) * 8 // nb, minlength=8)
    assert hist.min() > 20                  # about 50 per eighth if uniform
    # records of a uniform random order average H(1024) ~ 7.5
    assert 5.0 < np.mean(records) < 10.5


def test_main_calls_take_k_up_to_4096(lib):
    # The page's own kernel stops near k = 4,000 ("The Secret GPU Kernel
    # Behind DeepSeek V4.1 Flash", transcript 5:45): the main calls accept
    # 1 <= k <= 4096 and reject 4097 before any HIP call (rows = 0 launches
    # nothing, after the k check).
    assert _lib.TOPK_MAX_K == 4096
    for k, want in [(4096, _lib.TOPK_OK), (2049, _lib.TOPK_OK), (4097, _lib.TOPK_EK_RANGE)]:
        assert lib.topk_select(FAKE, None, 0, 1 << 20, k, FAKE, FAKE, None) == want
        assert lib.topk_select_split(FAKE, None, 0, 1 << 20, k, FAKE, FAKE, 2, None, 0,
                                     None) == want
        o = _lib.TopkOptions()
        assert lib.topk_select_ex(FAKE, None, 0, 1 << 20, k, FAKE, FAKE, ctypes.byref(o), None,
                                  0, None) == want
    # options are range-checked for every k
    o = _lib.TopkOptions()
    o.waves = 9
    assert lib.topk_select_ex(FAKE, None, 0, 1 << 20, 3000, FAKE, FAKE, ctypes.byref(o), None, 0,
                              None) == _lib.TOPK_EINVAL
    o.waves, o.split = 0, 2000
    assert lib.topk_select_ex(FAKE, None, 0, 1 << 20, 3000, FAKE, FAKE, ctypes.byref(o), None, 0,
                              None) == _lib.TOPK_ESPLIT


def _select_plan(lib, rows, n, k):
    p = _lib.TopkPlan()
    assert lib.topk_plan(rows, n, k, None, ctypes.byref(p)) == 0
    return p


def test_plan_paths(lib):
    # lists wider than the streaming filter's run the radix selection, with
    # options or without, and need no workspace
    for k in (2049, 3000, 4096):
        p = _plan(lib, 4, 1 << 20, k, split=4)
        assert p.path == _lib.TOPK_PATH_RADIX and p.split == 1 and p.workspace_bytes == 0
        assert p.list_words >= k and p.list_words & (p.list_words - 1) == 0
        assert p.lds_bytes <= 160 * 1024
        assert _select_plan(lib, 1, 1 << 20, k).path == _lib.TOPK_PATH_RADIX
        assert lib.topk_split_workspace_bytes(4, 1 << 20, k, 4) == 0
    assert _plan(lib, 4, 1 << 20, 2048).path == _lib.TOPK_PATH_STREAM
    # topk_select's own routing (no options): wide lists over many short rows
    # go to the radix selection, million-score rows at k <= 2048 stream
    assert _select_plan(lib, 256, 262144, 2048).path == _lib.TOPK_PATH_RADIX
    assert _select_plan(lib, 128, 1 << 20, 2048).path == _lib.TOPK_PATH_STREAM
    assert _select_plan(lib, 128, 1 << 20, 512).path == _lib.TOPK_PATH_STREAM
    # short rows: the radix selection from k = 129 up (longer rows and more
    # of them raise the bar, a few rows of 128K go to the split stream), the
    # streaming filter below
    cus = _select_plan(lib, 1, 1 << 20, 512).compute_units
    for rows, n, k, radix in ((4, 16384, 512, True), (64, 131072, 512, True),
                              (64, 262144, 512, False), (cus, 262144, 512, True),
                              (1, 16384, 1024, True), (1, 262144, 1000, True),
                              (16, 65536, 256, True), (16, 131072, 256, False),
                              (cus, 131072, 256, True), (cus, 262144, 256, False),
                              (1, 16384, 128, False), (cus, 65536, 64, False),
                              (1, 131072, 512, False), (16, 131072, 384, False),
                              (4, 65536, 512, True), (1, 65536, 256, False)):
        want = _lib.TOPK_PATH_RADIX if radix else _lib.TOPK_PATH_STREAM
        assert _select_plan(lib, rows, n, k).path == want, (rows, n, k)
    # with options the streaming path is kept up to its widest list
    assert _plan(lib, 256, 262144, 2048).path == _lib.TOPK_PATH_STREAM


def test_noalloc_entry_point_rejects_sizes_beyond_its_array(lib):
    assert _lib.TOPK_NOALLOC_SCRATCH_BYTES == 8 << 20
    assert "#define TOPK_NOALLOC_SCRATCH_BYTES (8u << 20)" in open(HEADER).read()
    # 2,000 rows x 8 segments x 2,048-word lists: 262 MB of lists, refused
    # before any HIP call
    need = lib.topk_split_workspace_bytes(2000, 1 << 20, 2048, 8)
    assert need > _lib.TOPK_NOALLOC_SCRATCH_BYTES
    assert lib.topk_select_split_noalloc(FAKE, None, 2000, 1 << 20, 2048, FAKE, FAKE, 8,
                                         None) == _lib.TOPK_EWORKSPACE
    assert lib.topk_select_split_noalloc(FAKE, None, 4, 1 << 20, 512, FAKE, FAKE, -1,
                                         None) == _lib.TOPK_ESPLIT
    assert lib.topk_select_split_noalloc(FAKE, None, 4, 1 << 20, 4097, FAKE, FAKE, 2,
                                         None) == _lib.TOPK_EK_RANGE
    assert lib.topk_select_split_noalloc(None, None, 0, 16, 8, None, None, 2, None) == _lib.TOPK_OK
