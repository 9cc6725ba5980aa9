"""The C ABI without a GPU: exports, argument validation and the split planner.

Nothing here launches a kernel. fd_plan_splits with an explicit compute-unit
count is pure host code; the error paths of the launching calls return before
any HIP call.
"""

import ctypes
import math
import os
import re

import pytest

import split_kv_flash_decoding_amd as fd
from split_kv_flash_decoding_amd import _capi
from tests.split_cuts import SHARE_COST, plan_cuts

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
INCLUDE = os.path.join(ROOT, "include")


def declared_functions():
    names = set()
    for h in sorted(os.listdir(INCLUDE)):
        if h.endswith(".h"):
            text = open(os.path.join(INCLUDE, h)).read()
            names |= set(re.findall(r"^\s*(?:fd_status|const char\*)\s+(fd_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_library_exports_every_declared_function():
    lib = fd.load_library()
    names = declared_functions()
    assert set(names) == set(fd.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_calls_validate_before_launching():
    lib = fd.load_library()
    fake = ctypes.c_void_p(0x10000)
    assert lib.fd_probe_read(None, 16, fake, None) == fd.FD_ERR_INVALID_ARGUMENT
    assert lib.fd_probe_read(fake, 24, fake, None) == fd.FD_ERR_INVALID_ARGUMENT
    assert lib.fd_probe_copy(fake, ctypes.c_void_p(0x10010), 64, None) == fd.FD_ERR_INVALID_ARGUMENT  # overlap
    assert lib.fd_probe_copy(fake, ctypes.c_void_p(0x10008), 16, None) == fd.FD_ERR_INVALID_ARGUMENT  # misaligned
    # row probe: 1 KB blocks with the waves along the rows, 8 KB blocks with the waves across
    rp = lib.fd_probe_read_rows
    assert rp(fake, fake, 16, 8192, 4096, 64, 0, fake, None) == fd.FD_ERR_INVALID_ARGUMENT   # block size
    assert rp(fake, fake, 16, 8192, 1024, 64, 1, fake, None) == fd.FD_ERR_INVALID_ARGUMENT   # block size
    assert rp(fake, fake, 16, 1536, 1024, 64, 0, fake, None) == fd.FD_ERR_INVALID_ARGUMENT   # row not whole KB
    assert rp(fake, fake, 16, 4096, 8192, 64, 1, fake, None) == fd.FD_ERR_INVALID_ARGUMENT   # block wider than row
    assert rp(fake, fake, 0, 8192, 1024, 64, 0, fake, None) == fd.FD_ERR_INVALID_ARGUMENT    # no rows
    assert rp(fake, ctypes.c_void_p(0x10008), 16, 8192, 1024, 64, 0, fake, None) == fd.FD_ERR_INVALID_ARGUMENT
    # mode 2 (rotated head rows) takes 1 KB blocks; modes past 2 are refused
    assert rp(fake, fake, 16, 8192, 8192, 64, 2, fake, None) == fd.FD_ERR_INVALID_ARGUMENT   # block size
    assert rp(fake, fake, 16, 8192, 1024, 64, 3, fake, None) == fd.FD_ERR_INVALID_ARGUMENT   # unknown mode
    assert rp(fake, fake, 16, 8192, 1024, 64, -1, fake, None) == fd.FD_ERR_INVALID_ARGUMENT  # unknown mode


def test_status_strings():
    assert fd.status_string(fd.FD_OK) == "FD_OK"
    assert fd.status_string(fd.FD_ERR_WORKSPACE_TOO_SMALL) == "FD_ERR_WORKSPACE_TOO_SMALL"
    assert fd.status_string(99) == "FD_ERR_UNKNOWN"


def prob(**kw):
    import torch
    base = dict(batch=1, num_q_heads=32, num_kv_heads=32, head_dim=128, kv_dtype=torch.float16)
    base.update(kw)
    return fd.make_problem(**base)


def ceil_div(a, b):
    return -(-a // b)


def mfma_kernel(hq, hkv, q_len=1):
    """The matrix-core form the planner picks: each wave owning a (KV head,
    column tile) (kernel 4) when the column tiles divide the four waves of a
    work-group and the heads fill them, else kernel 1."""
    nt = ceil_div(q_len * (hq // hkv), 16)
    return 4 if nt in (1, 2, 4) and hkv % (4 // nt) == 0 else 1


def mfma_work_groups(hq, hkv, q_len, kernel):
    """Work-groups per split (or balanced work item) of a matrix-core kernel."""
    nt = ceil_div(q_len * (hq // hkv), 16)
    return hkv * nt // 4 if kernel == 4 else hkv * nt


def workspace_bytes(B, rows, hkv, S, d=128):
    """O and (m, l) per (sequence, query row, split), then a 16-byte aligned
    uint32 arrival counter per (sequence, KV head)."""
    part = B * rows * S * (d + 2) * 4
    return ceil_div(part, 16) * 16 + ceil_div(B * hkv * 4, 16) * 16


@pytest.mark.parametrize("hq,hkv,lens", [
    (32, 32, [32768]),
    (32, 32, [131072]),
    (32, 8, [1024, 16384, 5000, 7777] * 4),
    (64, 8, [512, 32768, 900, 20000] * 16),
    (8, 8, [1024]),
    (8, 2, [1, 2, 3, 300]),
])
def test_planner_properties(hq, hkv, lens, monkeypatch):
    monkeypatch.setenv("FD_SPLIT_MODE", "0")  # the balanced mode has its own test below
    p = prob(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv)
    plan = fd.fd_plan_splits(p, lens, num_cus=256)
    assert plan.split_mode == 0
    C = plan.chunk_tokens
    assert C % 64 == 0 and C >= 256 or C == max(lens)
    splits = [ceil_div(L, C) for L in lens]
    assert plan.max_splits == max(splits) and plan.total_splits == sum(splits)
    assert plan.total_tokens == sum(lens) and plan.num_cus == 256 and plan.partial_kernel in (0, 1, 2, 4)
    # every split non-empty, splits tile [0, L)
    for L, S in zip(lens, splits):
        assert (S - 1) * C < L <= S * C
    assert plan.workspace_bytes == workspace_bytes(len(lens), hq, hkv, plan.max_splits)
    # enough work-groups to cover the chip when there are enough tokens
    if sum(lens) * hkv >= 256 * 4 * 256:
        assert plan.total_splits * hkv >= 256


@pytest.mark.parametrize("hq,hkv,lens,page", [
    (32, 8, [2915, 4487, 5931, 8309, 8336, 8684, 8905, 10375, 10902, 12067, 12486, 12967, 15191, 15198, 15709,
             15847], 0),
    (64, 8, [512, 32768, 900, 20000, 574, 604, 7006, 31712] * 8, 16),
    (64, 8, [1, 2, 15, 16, 17, 3000, 1, 40000], 16),
    (16, 4, [7, 100000, 3, 5], 0),
])
def test_balanced_plan(hq, hkv, lens, page):
    """Ragged batches on the matrix-core kernel get the balanced tile list:
    every work item but the last holds P tiles, the items cover every tile
    once, each sequence's splits cut [0, L_b) into consecutive non-empty
    ranges, and S_max bounds every sequence's split count."""
    p = prob(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, page_size=page,
             max_pages_per_seq=ceil_div(max(lens), 16) if page else 0)
    plan = fd.fd_plan_splits(p, lens, num_cus=256)
    assert plan.partial_kernel == mfma_kernel(hq, hkv) and plan.split_mode == 1
    wg = mfma_work_groups(hq, hkv, 1, plan.partial_kernel)
    C = plan.chunk_tokens
    assert C % 16 == 0 and C >= 256
    P = C // 16
    tiles = [ceil_div(L, 16) for L in lens]
    positions = sum(tiles) + SHARE_COST * len(lens)
    assert plan.total_splits == ceil_div(positions, P)
    assert plan.max_splits == ceil_div(max(tiles), P) + 1
    cuts = plan_cuts(lens, plan)
    for L, rs in zip(lens, cuts):
        assert rs[0][0] == 0 and rs[-1][1] == L and len(rs) <= plan.max_splits
        assert all(lo < hi for lo, hi in rs) and all(rs[i][1] == rs[i + 1][0] for i in range(len(rs) - 1))
        assert all(lo % 16 == 0 for lo, _ in rs)  # splits start on a page / tile
    # work per item, in list positions (a share's cost, then its tiles): P for
    # every item but the last (the list is dealt out evenly)
    per_item = [0] * plan.total_splits
    U = 0
    for n in tiles:
        for t in range(U, U + SHARE_COST + n):
            per_item[t // P] += 1
        U += SHARE_COST + n
    assert all(c == P for c in per_item[:-1]) and 0 < per_item[-1] <= P
    # one round of work-groups: one per compute unit on the kernel whose waves
    # own heads (a single column tile, 16-bit cache), two on the other:
    # P = ceil(positions * wg / (256 k)) tiles, so the items fall short of
    # 256 k / wg by at most the fraction 1 / P that the ceiling adds, plus one item
    k = 1 if plan.partial_kernel == 4 else 2
    if positions * wg >= 256 * k * 16:
        assert 256 * k * (P - 1) / P - wg <= plan.total_splits * wg <= 256 * k + wg
    assert plan.workspace_bytes == workspace_bytes(len(lens), hq, hkv, plan.max_splits)


@pytest.mark.parametrize("hq,hkv,q_len,fp8,per_cu", [
    (32, 8, 1, True, 2),    # FP8 on the kernel whose waves own heads: two per compute unit
    (16, 2, 1, True, 3),    # FP8 on the kernel whose waves share a head (two KV heads): three
    (64, 8, 8, False, 4),   # four column tiles: four
    (32, 8, 8, False, 2),   # two column tiles, 16-bit: two
    (32, 8, 4, False, 1),   # one column tile, 16-bit: one
    (32, 8, 1, False, 1),
])
def test_balanced_plan_work_groups_per_cu(hq, hkv, q_len, fp8, per_cu):
    """The balanced list's items are sized for the work-groups per compute unit
    each matrix-core form runs best with."""
    import torch
    lens = [2915, 4487, 5931, 8309, 8336, 8684, 8905, 10375] * 2
    kw = dict(kv_dtype=torch.float8_e4m3fn if fp8 else torch.bfloat16)
    p = prob(batch=len(lens), num_q_heads=hq, num_kv_heads=hkv, q_dtype=torch.bfloat16, q_len=q_len, **kw)
    plan = fd.fd_plan_splits(p, lens, num_cus=256)
    kern = mfma_kernel(hq, hkv, q_len)
    assert plan.split_mode == 1 and plan.partial_kernel == kern
    wg = mfma_work_groups(hq, hkv, q_len, kern)
    P = plan.chunk_tokens // 16
    assert 256 * per_cu * (P - 1) / P - wg <= plan.total_splits * wg <= 256 * per_cu + wg


def test_balanced_plan_choice(monkeypatch):
    """Only ragged matrix-core batches without forced splits get split_mode 1;
    FD_SPLIT_MODE overrides where the mode applies."""
    ragged = [1000, 5000, 300, 9000]
    gqa = prob(batch=4, num_q_heads=32, num_kv_heads=8)
    assert fd.fd_plan_splits(gqa, ragged, num_cus=256).split_mode == 1
    assert fd.fd_plan_splits(gqa, [5000] * 4, num_cus=256).split_mode == 0          # equal lengths
    assert fd.fd_plan_splits(gqa, ragged, num_cus=256, force_num_splits=3).split_mode == 0
    assert fd.fd_plan_splits(prob(batch=4), ragged, num_cus=256).split_mode == 0    # MHA: vector kernels
    for ql in (2, 4, 16):                                                           # 8, 16 and 64 query rows
        plan = fd.fd_plan_splits(prob(batch=4, num_q_heads=32, num_kv_heads=8, q_len=ql), ragged, num_cus=256)
        assert plan.split_mode == 1 and plan.partial_kernel == mfma_kernel(32, 8, ql)
    # past the batch bound (the combine walks the lengths before its sequence) the chunks stay per sequence
    assert fd.fd_plan_splits(prob(batch=4096, num_q_heads=32, num_kv_heads=8), [1, 2] * 2048,
                             num_cus=256).split_mode == 1
    assert fd.fd_plan_splits(prob(batch=4097, num_q_heads=32, num_kv_heads=8), [1, 2] * 2048 + [3],
                             num_cus=256).split_mode == 0
    monkeypatch.setenv("FD_SPLIT_MODE", "0")
    assert fd.fd_plan_splits(gqa, ragged, num_cus=256).split_mode == 0
    monkeypatch.setenv("FD_SPLIT_MODE", "1")
    assert fd.fd_plan_splits(gqa, [5000] * 4, num_cus=256).split_mode == 1
    assert fd.fd_plan_splits(prob(batch=4), ragged, num_cus=256).split_mode == 0    # not applicable


def test_balanced_plan_is_checked():
    """A balanced plan is refused for the vector kernels and for chunks that are
    not a multiple of 16."""
    lib = fd.load_library()
    fake = ctypes.c_void_p(0x10000)
    gqa = prob(batch=2, num_q_heads=32, num_kv_heads=8)
    plan = fd.fd_plan_splits(gqa, [1000, 3000], num_cus=256)
    assert plan.split_mode == 1
    need = plan.workspace_bytes
    for field, value in (("chunk_tokens", plan.chunk_tokens + 8), ("partial_kernel", 0), ("split_mode", 2)):
        bad = fd.FdPlan.from_buffer_copy(plan)
        setattr(bad, field, value)
        st = lib.fd_decode_partial(ctypes.byref(gqa), ctypes.byref(bad), fake, fake, fake, None, fake, fake,
                                   need, None)
        assert st == fd.FD_ERR_INVALID_ARGUMENT, field
        st = lib.fd_combine(ctypes.byref(gqa), ctypes.byref(bad), fake, fake, need, fake, None, None)
        assert st == fd.FD_ERR_INVALID_ARGUMENT, field
    mha = prob(batch=2)
    bad = fd.fd_plan_splits(mha, [1000, 3000], num_cus=256)
    assert bad.partial_kernel != 1
    bad.split_mode = 1
    bad.chunk_tokens = 1024
    st = lib.fd_decode_partial(ctypes.byref(mha), ctypes.byref(bad), fake, fake, fake, None, fake, fake,
                               bad.workspace_bytes, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT


def test_planner_sizes_long_contexts_to_fill_the_chip(monkeypatch):
    monkeypatch.delenv("FD_PARTIAL_KERNEL", raising=False)
    # head-rows kernel: a work-group covers 4 of the 32 heads
    plan = fd.fd_plan_splits(prob(), [131072], num_cus=256)
    assert plan.partial_kernel == 2
    assert plan.chunk_tokens == 2048 and plan.max_splits == 64  # 8 head groups x 64 splits = 2 WGs per CU
    plan = fd.fd_plan_splits(prob(), [32768], num_cus=256)
    assert plan.chunk_tokens == 1024 and plan.max_splits == 32  # the head-rows floor
    # one KV head per work-group
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "0")
    plan = fd.fd_plan_splits(prob(), [131072], num_cus=256)
    assert plan.chunk_tokens == 8192 and plan.max_splits == 16  # 32 heads x 16 splits


def test_forced_split_counts():
    p = prob(batch=1, num_q_heads=8, num_kv_heads=8, head_dim=64)
    for S in (1, 2, 3, 4, 7, 16, 64):
        plan = fd.fd_plan_splits(p, [1024], num_cus=256, force_num_splits=S)
        assert plan.chunk_tokens == ceil_div(1024, S) and plan.max_splits == ceil_div(1024, plan.chunk_tokens)
    # the worked example: L = 4 cut in two splits of 2
    plan = fd.fd_plan_splits(p, [4], num_cus=256, force_num_splits=2)
    assert (plan.chunk_tokens, plan.max_splits) == (2, 2)
    # more splits than tokens: one token per split
    plan = fd.fd_plan_splits(p, [5], num_cus=256, force_num_splits=64)
    assert (plan.chunk_tokens, plan.max_splits) == (1, 5)


def test_env_overrides(monkeypatch):
    monkeypatch.setenv("FD_NUM_SPLITS", "3")
    plan = fd.fd_plan_splits(prob(), [3000], num_cus=256)
    assert plan.chunk_tokens == 1000
    monkeypatch.delenv("FD_NUM_SPLITS")
    monkeypatch.setenv("FD_MIN_CHUNK", "2048")
    plan = fd.fd_plan_splits(prob(), [32768], num_cus=256)
    assert plan.chunk_tokens == 2048


@pytest.mark.parametrize("kw,lens,status", [
    (dict(num_q_heads=12, num_kv_heads=8), [10], fd.FD_ERR_INVALID_ARGUMENT),
    (dict(num_q_heads=24, num_kv_heads=8), [10], fd.FD_ERR_UNSUPPORTED),
    (dict(head_dim=96), [10], fd.FD_ERR_UNSUPPORTED),
    (dict(page_size=8, max_pages_per_seq=4), [10], fd.FD_ERR_UNSUPPORTED),
    (dict(page_size=16, max_pages_per_seq=0), [10], fd.FD_ERR_INVALID_ARGUMENT),
    (dict(page_size=16, max_pages_per_seq=2), [33], fd.FD_ERR_INVALID_ARGUMENT),
    (dict(), [0], fd.FD_ERR_INVALID_ARGUMENT),
    (dict(), [-5], fd.FD_ERR_INVALID_ARGUMENT),
    (dict(batch=0), [], fd.FD_ERR_INVALID_ARGUMENT),
])
def test_planner_rejects(kw, lens, status):
    p = prob(batch=kw.pop("batch", max(1, len(lens))), **kw)
    with pytest.raises(fd.FdError) as ei:
        fd.fd_plan_splits(p, lens or [1], num_cus=256)
    assert ei.value.status == status
    assert _capi.load_library().fd_last_error_message().decode()


def test_fp32_kv_is_unsupported_and_null_args_rejected():
    lib = fd.load_library()
    p = prob()
    p.kv_dtype = fd.FD_F32
    plan = fd.FdPlan()
    lens = (ctypes.c_int32 * 1)(16)
    assert lib.fd_plan_splits(ctypes.byref(p), lens, 256, 0, ctypes.byref(plan)) == fd.FD_ERR_UNSUPPORTED
    p = prob()
    assert lib.fd_plan_splits(None, lens, 256, 0, ctypes.byref(plan)) == fd.FD_ERR_INVALID_ARGUMENT
    assert lib.fd_plan_splits(ctypes.byref(p), None, 256, 0, ctypes.byref(plan)) == fd.FD_ERR_INVALID_ARGUMENT
    assert lib.fd_plan_splits(ctypes.byref(p), lens, 256, 0, None) == fd.FD_ERR_INVALID_ARGUMENT
    assert lib.fd_plan_splits(ctypes.byref(p), lens, -1, 0, ctypes.byref(plan)) == fd.FD_ERR_INVALID_ARGUMENT


def test_launch_calls_validate_before_launching():
    """Bad arguments return an error before any HIP call (safe without a GPU)."""
    lib = fd.load_library()
    p = prob()
    plan = fd.fd_plan_splits(p, [4096], num_cus=256)
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    need = plan.workspace_bytes
    # null q
    st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(plan), None, fake, fake, None, fake, fake, need, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    # workspace too small
    st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, fake, fake, need - 4, None)
    assert st == fd.FD_ERR_WORKSPACE_TOO_SMALL
    # misaligned k
    st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(plan), fake, ctypes.c_void_p(0x10002), fake, None,
                               fake, fake, need, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    # paged without a table
    pp = prob(page_size=16, max_pages_per_seq=256)
    pplan = fd.fd_plan_splits(pp, [4096], num_cus=256)
    st = lib.fd_decode_partial(ctypes.byref(pp), ctypes.byref(pplan), fake, fake, fake, None, fake, fake,
                               pplan.workspace_bytes, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    # a plan that does not fit the problem
    bad = fd.FdPlan()
    bad.chunk_tokens, bad.max_splits, bad.workspace_bytes = 0, 1, need
    st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(bad), fake, fake, fake, None, fake, fake, need, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    # combine: null out, small workspace
    st = lib.fd_combine(ctypes.byref(p), ctypes.byref(plan), fake, fake, need, None, None, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    st = lib.fd_combine(ctypes.byref(p), ctypes.byref(plan), fake, fake, need - 1, fake, None, None)
    assert st == fd.FD_ERR_WORKSPACE_TOO_SMALL


def test_one_shot_without_gpu_reports_hip_error():
    """num_cus = 0 asks the HIP runtime; with no device that is FD_ERR_HIP, not a crash."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    lib = fd.load_library()
    p = prob()
    lens = (ctypes.c_int32 * 1)(4096)
    plan = fd.FdPlan()
    assert lib.fd_plan_splits(ctypes.byref(p), lens, 0, 0, ctypes.byref(plan)) == fd.FD_ERR_HIP


@pytest.mark.parametrize("hq,hkv,d,expect", [
    (32, 32, 128, 2), (32, 8, 128, 4), (64, 8, 128, 4), (16, 2, 128, 1), (16, 8, 128, 2), (32, 8, 64, 0),
    (8, 8, 64, 2), (4, 4, 64, 0), (6, 6, 128, 0), (4, 2, 128, 0)])
def test_planner_picks_the_partial_kernel(hq, hkv, d, expect, monkeypatch):
    monkeypatch.delenv("FD_PARTIAL_KERNEL", raising=False)
    mk = lambda: fd.fd_plan_splits(prob(num_q_heads=hq, num_kv_heads=hkv, head_dim=d), [500000], num_cus=256)
    assert mk().partial_kernel == expect
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "0")
    assert mk().partial_kernel == 0
    G = hq // hkv
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "1")
    assert mk().partial_kernel == (1 if d == 128 and G in (2, 4, 8) else expect)
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "2")
    rows = 64 // (d // 8)
    assert mk().partial_kernel == (2 if G <= 2 and hkv % rows == 0 else expect)


def test_head_rows_fall_back_when_work_groups_are_few(monkeypatch):
    """Multi-head work-groups that would leave most compute units idle (short
    context, or a forced small split count) give way to one KV head each."""
    monkeypatch.delenv("FD_PARTIAL_KERNEL", raising=False)
    p = prob(num_q_heads=8, num_kv_heads=8, head_dim=64)
    assert fd.fd_plan_splits(p, [1024], num_cus=256, force_num_splits=4).partial_kernel == 0
    assert fd.fd_plan_splits(p, [3000], num_cus=256).partial_kernel == 0
    assert fd.fd_plan_splits(p, [2_000_000], num_cus=256).partial_kernel == 2
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "2")  # an explicit request is kept
    assert fd.fd_plan_splits(p, [1024], num_cus=256, force_num_splits=4).partial_kernel == 2


def test_multi_query_problems():
    """q_len > 1 runs on the matrix-core kernel: d = 128 and q_len * G <= 64
    (one work-group per 16 query rows of a KV head, so fewer splits fill the
    chip as the rows grow)."""
    plan = fd.fd_plan_splits(prob(num_q_heads=32, num_kv_heads=32, q_len=4), [131072], num_cus=256)
    assert plan.partial_kernel == 4
    assert plan.workspace_bytes == workspace_bytes(1, 4 * 32, 32, plan.max_splits)
    assert fd.fd_plan_splits(prob(num_q_heads=64, num_kv_heads=8, q_len=2), [1000], num_cus=256).partial_kernel == 4
    splits = {}
    for ql in (2, 4, 8):  # 16, 32 and 64 query rows per KV head
        plan = fd.fd_plan_splits(prob(num_q_heads=64, num_kv_heads=8, q_len=ql), [131072], num_cus=256)
        assert plan.partial_kernel == 4
        splits[ql] = plan.max_splits
    assert splits[2] >= splits[4] >= splits[8]
    assert fd.fd_plan_splits(prob(num_q_heads=32, num_kv_heads=32, q_len=64), [1000],
                             num_cus=256).partial_kernel == 4
    # 40 query rows (three column tiles) keep the kernel with one work-group per column tile
    assert fd.fd_plan_splits(prob(num_q_heads=16, num_kv_heads=16, q_len=40), [1000],
                             num_cus=256).partial_kernel == 1
    for kw, lens, status in [
        (dict(head_dim=64, q_len=2), [100], fd.FD_ERR_UNSUPPORTED),
        (dict(num_q_heads=64, num_kv_heads=8, q_len=9), [100], fd.FD_ERR_UNSUPPORTED),  # 72 rows
        (dict(num_q_heads=32, num_kv_heads=32, q_len=65), [100], fd.FD_ERR_UNSUPPORTED),
        (dict(q_len=-1), [100], fd.FD_ERR_INVALID_ARGUMENT),
        (dict(q_len=4), [3], fd.FD_ERR_INVALID_ARGUMENT),  # shorter than its query tokens
    ]:
        with pytest.raises(fd.FdError) as ei:
            fd.fd_plan_splits(prob(**kw), lens, num_cus=256)
        assert ei.value.status == status, kw


def test_fp8_problems(monkeypatch):
    """An FP8 (E4M3) cache: 16 codes per 16-byte load, so a head-rows load
    covers 8 heads at d = 128 and 16 at d = 64; q is fp16 or bf16; the
    unscaled calls refuse it (its scales are part of the data)."""
    import torch
    f8 = torch.float8_e4m3fn
    p = prob(kv_dtype=f8, q_dtype=torch.bfloat16)
    assert p.kv_dtype == fd.FD_FP8_E4M3 and p.q_dtype == fd.FD_BF16
    assert prob(kv_dtype=f8).q_dtype == fd.FD_F16
    plan = fd.fd_plan_splits(p, [131072], num_cus=256)
    assert plan.partial_kernel == 2
    assert fd.fd_plan_splits(prob(kv_dtype=f8, num_kv_heads=8, num_q_heads=32), [500000],
                             num_cus=256).partial_kernel == 4
    # d = 64: 16 heads per load; 8 KV heads cannot fill a head-rows wave
    assert fd.fd_plan_splits(prob(kv_dtype=f8, num_q_heads=8, num_kv_heads=8, head_dim=64), [500000],
                             num_cus=256).partial_kernel == 0
    assert fd.fd_plan_splits(prob(kv_dtype=f8, num_q_heads=16, num_kv_heads=16, head_dim=64), [2_000_000],
                             num_cus=256).partial_kernel == 2
    # FP8 head-rows splits hold at least 2048 tokens (the bytes of 1024 16-bit tokens)
    assert plan.chunk_tokens == 2048 and fd.fd_plan_splits(prob(), [131072], num_cus=256).chunk_tokens == 2048
    # Shorter contexts: head-row splits are halved (not below 256 tokens) until every CU has a
    # work-group (32 heads at 8 per FP8 load, 4 per 16-bit load), before token rows take over.
    for kv, L, want in ((f8, 65536, (2, 1024)), (f8, 32768, (2, 512)), (f8, 16384, (2, 256)),
                        (None, 16384, (2, 512)), (None, 8192, (2, 256)), (None, 32768, (2, 1024))):
        pl = fd.fd_plan_splits(prob() if kv is None else prob(kv_dtype=kv), [L], num_cus=256)
        assert (pl.partial_kernel, pl.chunk_tokens) == want, (kv, L)
        groups = 4 if kv is f8 else 8
        assert -(-L // pl.chunk_tokens) * groups >= 256
    # too short for head rows even at 256 tokens: FP8 token rows, twice the work-groups a 16-bit
    # cache would get (8K tokens: 32 heads x 32 splits)
    p2 = fd.fd_plan_splits(prob(kv_dtype=f8), [8192], num_cus=256)
    assert (p2.partial_kernel, p2.chunk_tokens) == (0, 256)
    # FD_MIN_CHUNK bounds the halving too
    monkeypatch.setenv("FD_MIN_CHUNK", "1024")
    assert fd.fd_plan_splits(prob(kv_dtype=f8), [32768], num_cus=256).partial_kernel == 0
    monkeypatch.delenv("FD_MIN_CHUNK")
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "0")
    assert fd.fd_plan_splits(prob(), [32768], num_cus=256).chunk_tokens == 2048
    # the workspace does not depend on the cache type
    assert plan.workspace_bytes == fd.fd_plan_splits(prob(), [131072], num_cus=256,
                                                     force_num_splits=plan.max_splits).workspace_bytes
    bad = prob(kv_dtype=f8)
    bad.q_dtype = fd.FD_F32
    with pytest.raises(fd.FdError) as ei:
        fd.fd_plan_splits(bad, [100], num_cus=256)
    assert ei.value.status == fd.FD_ERR_INVALID_ARGUMENT
    lib = fd.load_library()
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: every call below fails validation
    need = plan.workspace_bytes
    st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, fake, fake, need, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT and b"scaled" in lib.fd_last_error_message()
    lens = (ctypes.c_int32 * 1)(131072)
    st = lib.fd_decode_attention(ctypes.byref(p), fake, fake, fake, None, lens, fake, fake, None, fake, need, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    # misaligned scales, too-small workspace
    st = lib.fd_decode_partial_scaled(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, ctypes.c_void_p(0x10002),
                                      None, None, fake, fake, need, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT
    st = lib.fd_decode_partial_scaled(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, None, None, fake,
                                      fake, need - 4, None)
    assert st == fd.FD_ERR_WORKSPACE_TOO_SMALL


def test_append_validates_before_launching():
    """fd_append_kv: paged caches only, a known RoPE style, a positive base,
    non-NULL buffers, a page count, aligned pointers; errors launch nothing."""
    import torch
    lib = fd.load_library()
    fake = ctypes.c_void_p(0x10000)
    p = prob(page_size=16, max_pages_per_seq=64, num_q_heads=8, num_kv_heads=2)

    def call(pp, style=1, base=10000.0, knew=fake, q=None, kc=fake, pages=10, ks=None):
        return lib.fd_append_kv(ctypes.byref(pp), style, base, knew, fake, q, ks, None, kc, fake, pages, fake,
                                fake, None)
    assert call(prob(num_q_heads=8, num_kv_heads=2)) == fd.FD_ERR_UNSUPPORTED   # contiguous
    assert call(p, style=3) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, base=0.0) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, base=float("inf")) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, knew=None) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, pages=0) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, knew=ctypes.c_void_p(0x10001)) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, kc=ctypes.c_void_p(0x10001)) == fd.FD_ERR_INVALID_ARGUMENT   # 2-byte cache elements
    # rows move in 16-byte pieces: 16-byte alignment (8 for an FP8 cache)
    assert call(p, knew=ctypes.c_void_p(0x10008)) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, kc=ctypes.c_void_p(0x10008)) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(p, ks=ctypes.c_void_p(0x10002)) == fd.FD_ERR_INVALID_ARGUMENT
    f8 = prob(page_size=16, max_pages_per_seq=64, num_q_heads=8, num_kv_heads=2, kv_dtype=torch.float8_e4m3fn)
    bad = prob(page_size=16, max_pages_per_seq=64, num_q_heads=8, num_kv_heads=2, kv_dtype=torch.float8_e4m3fn)
    bad.q_dtype = fd.FD_F32
    assert call(bad) == fd.FD_ERR_INVALID_ARGUMENT
    assert f8.q_dtype == fd.FD_F16
    assert call(f8, kc=ctypes.c_void_p(0x10004)) == fd.FD_ERR_INVALID_ARGUMENT


def test_prefill_validates_before_launching():
    """fd_prefill_attention: d = 128 and a 16-bit cache; any q_len; bad
    arguments launch nothing."""
    import torch
    lib = fd.load_library()
    fake = ctypes.c_void_p(0x10000)

    def call(pp, q=fake, out=fake, table=None):
        return lib.fd_prefill_attention(ctypes.byref(pp), q, fake, fake, table, fake, out, None, None)
    assert call(prob(head_dim=64, q_len=100)) == fd.FD_ERR_UNSUPPORTED
    assert call(prob(kv_dtype=torch.float8_e4m3fn, q_len=100)) == fd.FD_ERR_UNSUPPORTED
    assert call(prob(q_len=100), q=None) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(prob(q_len=100), out=None) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(prob(q_len=100), q=ctypes.c_void_p(0x10008)) == fd.FD_ERR_INVALID_ARGUMENT
    assert call(prob(q_len=100, page_size=16, max_pages_per_seq=8)) == fd.FD_ERR_INVALID_ARGUMENT  # no table
    assert call(prob(q_len=-2)) == fd.FD_ERR_INVALID_ARGUMENT


def test_fused_calls_validate_before_launching():
    lib = fd.load_library()
    p = prob()
    plan = fd.fd_plan_splits(p, [4096], num_cus=256)
    fake = ctypes.c_void_p(0x10000)
    need = plan.workspace_bytes
    st = lib.fd_decode_fused(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, None, None, fake, fake,
                             need, None, None, None)
    assert st == fd.FD_ERR_INVALID_ARGUMENT  # no out
    st = lib.fd_decode_fused(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, None, None, fake, fake,
                             need - 16, fake, None, None)
    assert st == fd.FD_ERR_WORKSPACE_TOO_SMALL
    assert lib.fd_workspace_init(ctypes.byref(p), ctypes.byref(plan), None, need, None) == fd.FD_ERR_INVALID_ARGUMENT
    assert lib.fd_workspace_init(ctypes.byref(p), ctypes.byref(plan), fake, need - 16, None) == \
        fd.FD_ERR_WORKSPACE_TOO_SMALL


@pytest.mark.parametrize("hq,hkv,d,f8,k3,k4", [
    # (Hq, Hkv, d, FP8 cache, head columns applies, matrix cores with waves owning heads applies)
    (32, 32, 128, False, True, False),   # 4 heads per wave x 8 waves = 32
    (16, 16, 128, False, False, False),  # 16 heads: not a multiple of 32
    (64, 64, 64, False, True, False),    # d = 64: 8 heads per wave x 8 waves = 64
    (32, 32, 128, True, True, False),    # FP8: 8 heads per wave x 4 waves = 32
    (32, 8, 128, False, False, True),    # G = 4: four heads per work-group
    (64, 8, 128, False, False, True),    # G = 8
    (8, 2, 128, False, False, False),    # two KV heads cannot fill four waves
    (32, 8, 64, False, False, False),    # no matrix-core form at d = 64
])
def test_head_columns_and_mfma_heads_applicability(hq, hkv, d, f8, k3, k4, monkeypatch):
    """Kernels 3 (head columns) and 4 (matrix cores, each wave owning a head)
    are chosen when forced and they cover the problem; otherwise the planner
    keeps its own choice."""
    import torch
    kw = dict(num_q_heads=hq, num_kv_heads=hkv, head_dim=d)
    if f8:
        kw.update(kv_dtype=torch.float8_e4m3fn, q_dtype=torch.bfloat16)
    monkeypatch.delenv("FD_PARTIAL_KERNEL", raising=False)
    base = fd.fd_plan_splits(prob(**kw), [300000], num_cus=256).partial_kernel
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "3")
    assert fd.fd_plan_splits(prob(**kw), [300000], num_cus=256).partial_kernel == (3 if k3 else base)
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "4")
    assert fd.fd_plan_splits(prob(**kw), [300000], num_cus=256).partial_kernel == (4 if k4 else base)


def test_mfma_heads_work_items_and_column_tiles(monkeypatch):
    """Kernel 4 puts 4 / NT KV heads in a work-group (NT column tiles of 16
    query rows each), so a split of Hkv heads takes Hkv * NT / 4 work-groups,
    and the balanced list sizes its items for that count."""
    monkeypatch.setenv("FD_PARTIAL_KERNEL", "4")
    lens = [3000, 700, 12000, 64]
    for ql, nt in ((1, 1), (2, 1), (4, 2), (8, 4)):
        p = prob(batch=4, num_q_heads=64, num_kv_heads=8, q_len=ql)
        plan = fd.fd_plan_splits(p, lens, num_cus=256)
        assert plan.partial_kernel == 4 and plan.split_mode == 1
        per_split = 8 // (4 // nt)
        positions = sum(-(-L // 16) + 4 for L in lens)
        P = plan.chunk_tokens // 16
        assert P == max(16, -(-positions * per_split // 512))
        assert plan.total_splits == -(-positions // P)
    # three column tiles (40 query rows) do not divide four waves: kernel 1 stays
    p = prob(batch=1, num_q_heads=16, num_kv_heads=16, q_len=40)
    assert fd.fd_plan_splits(p, [5000], num_cus=256).partial_kernel == 1


def test_plans_naming_kernels_that_do_not_apply_are_refused():
    """A plan that names kernel 3 or 4 for a problem they do not cover is an
    argument error, before anything is launched."""
    lib = fd.load_library()
    fake = ctypes.c_void_p(0x10000)
    for kw, kernel in ((dict(num_q_heads=16, num_kv_heads=16), 3), (dict(num_q_heads=8, num_kv_heads=2), 4),
                       (dict(num_q_heads=32, num_kv_heads=32), 4), (dict(num_q_heads=32, num_kv_heads=8), 3)):
        p = prob(**kw)
        plan = fd.fd_plan_splits(p, [4096], num_cus=256)
        plan.partial_kernel = kernel
        plan.split_mode = 0
        st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, fake, fake,
                                   plan.workspace_bytes, None)
        assert st == fd.FD_ERR_INVALID_ARGUMENT, (kw, kernel)
        plan.partial_kernel = 5
        st = lib.fd_decode_partial(ctypes.byref(p), ctypes.byref(plan), fake, fake, fake, None, fake, fake,
                                   plan.workspace_bytes, None)
        assert st == fd.FD_ERR_INVALID_ARGUMENT
