"""CPU tests of libsgmv's host side: the library loads and exports every function that
include/sgmv.h declares, the C++ segment builder equals the oracle's stable sort bit for
bit, and argument validation rejects bad calls before any HIP call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from adapter_gemv_amd import _lib, sgmv
from workloads import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgmv.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sgmv_[a-z_]+)\s*\(", src)))


def test_header_declares_the_abi():
    assert header_functions() == sorted(_lib.SIGNATURES)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in header_functions():
        assert hasattr(L, name), name
        assert ctypes.cast(getattr(L, name), ctypes.c_void_p).value


def test_abi_version_and_status_strings():
    assert sgmv.sgmv_abi_version() == 1
    for code in range(9):
        assert sgmv.sgmv_status_string(code) and sgmv.sgmv_status_string(code) != "unknown status"
    assert sgmv.sgmv_status_string(99) == "unknown status"


# --------------------------------------------------------------------------------------
# segment builder vs the oracle
# --------------------------------------------------------------------------------------
def _ids_cases():
    rng = np.random.default_rng(42)
    cases = [
        ("empty", np.zeros(0, np.int32), 3),
        ("one", np.array([2], np.int32), 3),
        ("same", np.full(33, 5, np.int32), 8),
        ("distinct", rng.permutation(32).astype(np.int32), 32),
        ("sorted", np.repeat(np.arange(4), 512).astype(np.int32), 4),
        ("empty_adapters", rng.choice([0, 7, 63], 100).astype(np.int32), 64),
        # an adapter's rows in several runs of caller rows, runs of other adapters between
        ("runs_recurring", np.array([3] * 5 + [1] * 7 + [3] * 4 + [0] * 9 + [1] * 2 + [3],
                                    np.int32), 4),
        # a pool far larger than the batch: ids spread over 2^20 entries, in runs
        ("large_pool", np.repeat(rng.integers(0, 1 << 20, 40), rng.integers(1, 20, 40)).astype(np.int32),
         1 << 20),
    ]
    for k in range(20):
        P = int(rng.integers(1, 70))
        n = int(rng.integers(1, 3000))
        cases.append((f"random{k}", rng.integers(0, P, n).astype(np.int32), P))
    return cases


@pytest.mark.parametrize("name,ids,P", _ids_cases(), ids=[c[0] for c in _ids_cases()])
def test_build_segments_matches_oracle(name, ids, P):
    tab = sgmv.sgmv_build_segments(ids, P)
    perm, starts, seg_ad = oracle.segments(ids, P)
    assert np.array_equal(tab.perm, perm)
    assert np.array_equal(tab.seg_starts, starts)
    assert np.array_equal(tab.seg_adapter, seg_ad)
    assert tab.n_segments == len(seg_ad)
    lens = np.diff(starts)
    assert tab.min_seg_len == (int(lens.min()) if lens.size else 0)
    assert tab.max_seg_len == (int(lens.max()) if lens.size else 0)


def test_build_segments_rejects_bad_ids():
    for bad in ([0, 3], [-1, 0]):
        with pytest.raises(sgmv.SgmvError) as e:
            sgmv.sgmv_build_segments(np.array(bad, np.int32), 3)
        assert e.value.status == _lib.ERR_ADAPTER_ID
    L = _lib.lib()
    assert L.sgmv_build_segments(None, 4, 3, None, None, None, None, None, None) == _lib.ERR_NULL
    out = np.zeros(4, np.int32)
    assert L.sgmv_build_segments(None, -1, 3, None, out.ctypes.data, None, out.ctypes.data,
                                 None, None) == _lib.ERR_SHAPE


def test_build_ptr_table():
    base = np.array([4096, 8192, 12288, 16384], np.uint64)
    seg_ad = np.array([0, 2, 3], np.int32)
    assert np.array_equal(sgmv.sgmv_build_ptr_table(base, seg_ad), oracle.ptr_table(base, seg_ad))
    with pytest.raises(sgmv.SgmvError) as e:
        sgmv.sgmv_build_ptr_table(base, np.array([4], np.int32))
    assert e.value.status == _lib.ERR_ADAPTER_ID
    with pytest.raises(sgmv.SgmvError) as e:
        sgmv.sgmv_build_ptr_table(np.array([4100], np.uint64), np.array([0], np.int32))
    assert e.value.status == _lib.ERR_ALIGNMENT


def test_workspace_bytes():
    assert sgmv.sgmv_workspace_bytes(32, 4096, 16) >= 8 * 32 * 16 * 4
    assert sgmv.sgmv_workspace_bytes(32, 4096, 7) == 0
    assert sgmv.sgmv_workspace_bytes(-1, 4096, 16) == 0
    a = sgmv.sgmv_workspace_bytes(2112, 28672, 64)
    assert a >= 2112 * 64 * 4 and a < 80 * 2 ** 20


def test_workspace_bytes_monotone():
    """One workspace serves every call no larger than the shape it was sized for: the
    size never shrinks when n, h_in or r grows."""
    ns, hs, rs = [1, 17, 64, 65, 600, 2112], [8, 520, 4096, 5120, 13824, 28672], [16, 32, 64]
    size = {(n, h, r): sgmv.sgmv_workspace_bytes(n, h, r) for n in ns for h in hs for r in rs}
    for (n, h, r), b in size.items():
        for (n2, h2, r2), b2 in size.items():
            if n <= n2 and h <= h2 and r <= r2:
                assert b <= b2, ((n, h, r), (n2, h2, r2))


def test_workspace_layout_sharing_rule(tmp_path):
    """The layout code itself (sgmv_checks.h, built for the host by tests/ws_layout_check.cpp):
    in a buffer sized for the largest shape, no smaller call's scratch reaches the counters
    or tagged partials of any other smaller call."""
    import shutil
    import subprocess
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "ws_layout_check")
    subprocess.run([cxx, "-O1", "-std=c++17", "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(ROOT, "tests", "ws_layout_check.cpp"), "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout


def test_host_code_under_sanitizers(tmp_path):
    """The host code that needs no GPU (segment builders, pointer table, argument checks,
    workspace layout) built with AddressSanitizer and UndefinedBehaviorSanitizer and run
    over random and edge-case inputs, every rejection included."""
    import shutil
    import subprocess
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("g++ not found")
    exe = str(tmp_path / "host_sanitize_check")
    subprocess.run([cxx, "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Werror",
                    "-I/opt/rocm/include", "-D__HIP_PLATFORM_AMD__",
                    os.path.join(ROOT, "tests", "host_sanitize_check.cpp"),
                    os.path.join(ROOT, "adapter_gemv_amd", "csrc", "sgmv_segments.cpp"),
                    os.path.join(ROOT, "adapter_gemv_amd", "csrc", "sgmv_cache.cpp"),
                    "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    env.pop("LD_PRELOAD", None)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert out.returncode == 0 and out.stdout.startswith("ok"), out.stdout + out.stderr


# --------------------------------------------------------------------------------------
# validation: every one of these returns before any HIP call
# --------------------------------------------------------------------------------------
# Fake, 256-aligned "device" addresses: never dereferenced because every call below is
# rejected by the host-side checks.
X, Y, V, WS, TAB = 1 << 40, 2 << 40, 3 << 40, 4 << 40, 5 << 40


def _lora(**kw):
    a = dict(stream=None, dtype=0, y=Y, ld_y=4096, x=X, ld_x=4096, A_ptrs=TAB, B_ptrs=TAB + 256,
             seg_starts=TAB + 512, perm=None, n=32, n_segments=32, min_seg_len=1, max_seg_len=1,
             h_in=4096, h_out=4096, r=16, scale=2.0, workspace=WS, workspace_bytes=1 << 30)
    a.update(kw)
    return sgmv.sgmv_lora_add(**a)


REJECTS = [
    ("dtype", dict(dtype=2), _lib.ERR_UNSUPPORTED),
    ("rank", dict(r=8), _lib.ERR_UNSUPPORTED),
    ("rank128", dict(r=128), _lib.ERR_UNSUPPORTED),
    ("n<0", dict(n=-1), _lib.ERR_SHAPE),
    ("S>n", dict(n_segments=33), _lib.ERR_SHAPE),
    ("S=0", dict(n_segments=0), _lib.ERR_SHAPE),
    ("min>max", dict(min_seg_len=2, max_seg_len=1), _lib.ERR_SHAPE),
    ("max<ceil(n/S)", dict(n_segments=16, max_seg_len=1), _lib.ERR_SHAPE),
    ("min>n/S", dict(n_segments=16, min_seg_len=3, max_seg_len=3), _lib.ERR_SHAPE),
    ("max>n", dict(max_seg_len=33), _lib.ERR_SHAPE),
    ("h_in%8", dict(h_in=4092, ld_x=4092), _lib.ERR_ALIGNMENT),
    ("ld_x<h_in", dict(ld_x=4088), _lib.ERR_SHAPE),
    ("ld_y%8", dict(ld_y=4100), _lib.ERR_ALIGNMENT),
    ("h_out tiny", dict(h_out=0), _lib.ERR_SHAPE),
    ("x null", dict(x=None), _lib.ERR_NULL),
    ("A null", dict(A_ptrs=None), _lib.ERR_NULL),
    ("seg null", dict(seg_starts=None), _lib.ERR_NULL),
    ("x misaligned", dict(x=X + 8), _lib.ERR_ALIGNMENT),
    ("y misaligned", dict(y=Y + 2), _lib.ERR_ALIGNMENT),
    ("alias", dict(y=X + 4096 * 2), _lib.ERR_ALIAS),
    ("ws null", dict(workspace=None), _lib.ERR_WORKSPACE),
    ("ws small", dict(workspace_bytes=100), _lib.ERR_WORKSPACE),
    ("ws misaligned", dict(workspace=WS + 16), _lib.ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", REJECTS, ids=[r[0] for r in REJECTS])
def test_lora_add_rejects(name, kw, code):
    assert _lora(**kw) == code


def test_n_zero_is_ok_without_launch():
    assert _lora(n=0, n_segments=0, min_seg_len=0, max_seg_len=0, x=None, y=None) == _lib.OK


def test_shrink_and_expand_reject():
    L = _lib.lib()
    ok = dict(n=32, S=32, lo=1, hi=1)
    # shrink: v overlapping x
    assert L.sgmv_shrink(None, 0, X + 64, X, 4096, TAB, TAB + 512, None, 32, 32, 1, 1, 4096,
                         16, WS, 1 << 30) == _lib.ERR_ALIAS
    assert L.sgmv_shrink(None, 0, V, X, 4096, TAB, TAB + 512, None, 32, 32, 1, 1, 4096,
                         12, WS, 1 << 30) == _lib.ERR_UNSUPPORTED
    assert L.sgmv_shrink(None, 0, V, X, 4096, TAB, TAB + 512, None, 32, 32, 1, 1, 4096,
                         16, WS, 16) == _lib.ERR_WORKSPACE
    # expand: y overlapping v, null B
    assert L.sgmv_expand(None, 1, Y, 4096, Y + 256, TAB, TAB + 512, None, 32, 32, 1, 1, 16,
                         4096, 1.0) == _lib.ERR_ALIAS
    assert L.sgmv_expand(None, 1, Y, 4096, V, None, TAB + 512, None, 32, 32, 1, 1, 16,
                         4096, 1.0) == _lib.ERR_NULL
    assert ok


def _no_gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() == 0
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu_visible(), reason="needs a machine without a GPU: the fake "
                    "addresses would reach a kernel")
def test_valid_call_without_device_is_hip_error():
    assert _lora() == _lib.ERR_HIP


def _pool(**kw):
    a = dict(stream=None, dtype=0, y=Y, ld_y=4096, x=X, ld_x=4096, adapter_ids=TAB, n=32,
             A_pool=V, A_stride=16 * 4096, B_pool=V + (1 << 30), B_stride=16 * 4096,
             n_adapters=4096, h_in=4096, h_out=4096, r=16, scale=2.0, workspace=WS,
             workspace_bytes=1 << 30)
    a.update(kw)
    return sgmv.sgmv_lora_add_pool(**a)


POOL_REJECTS = [
    ("n>4096", dict(n=4097), _lib.ERR_SHAPE),
    ("rank", dict(r=8), _lib.ERR_UNSUPPORTED),
    ("dtype", dict(dtype=7), _lib.ERR_UNSUPPORTED),
    ("A_stride small", dict(A_stride=16 * 4096 - 8), _lib.ERR_SHAPE),
    ("B_stride odd", dict(B_stride=16 * 4096 + 4), _lib.ERR_ALIGNMENT),
    ("ids null", dict(adapter_ids=None), _lib.ERR_NULL),
    ("pool misaligned", dict(A_pool=V + 8), _lib.ERR_ALIGNMENT),
    ("no adapters", dict(n_adapters=0), _lib.ERR_SHAPE),
    ("ws small", dict(workspace_bytes=1024), _lib.ERR_WORKSPACE),
    ("alias", dict(y=X + 64), _lib.ERR_ALIAS),
]


@pytest.mark.parametrize("name,kw,code", POOL_REJECTS, ids=[r[0] for r in POOL_REJECTS])
def test_lora_add_pool_rejects(name, kw, code):
    assert _pool(**kw) == code


HOST_IDS = np.arange(64, dtype=np.int32)


def _host_ids(**kw):
    a = dict(stream=None, dtype=0, y=Y, ld_y=4096, x=X, ld_x=4096,
             adapter_ids=HOST_IDS.ctypes.data, n=32, A_pool=V, A_stride=16 * 4096,
             B_pool=V + (1 << 30), B_stride=16 * 4096, n_adapters=4096, h_in=4096, h_out=4096,
             r=16, scale=2.0, workspace=WS, workspace_bytes=1 << 30)
    a.update(kw)
    return sgmv.sgmv_lora_add_host_ids(**a)


BAD_IDS = np.array([0, 1, 4096, 2], dtype=np.int32)
NEG_IDS = np.array([0, -1], dtype=np.int32)
HOST_ID_REJECTS = [
    ("n>64", dict(n=65), _lib.ERR_SHAPE),
    ("n<0", dict(n=-1), _lib.ERR_SHAPE),
    ("rank", dict(r=8), _lib.ERR_UNSUPPORTED),
    ("dtype", dict(dtype=7), _lib.ERR_UNSUPPORTED),
    ("A_stride small", dict(A_stride=16 * 4096 - 8), _lib.ERR_SHAPE),
    ("ids null", dict(adapter_ids=None), _lib.ERR_NULL),
    ("pool misaligned", dict(B_pool=V + 8), _lib.ERR_ALIGNMENT),
    ("ws small", dict(workspace_bytes=1024), _lib.ERR_WORKSPACE),
    ("alias", dict(y=X + 64), _lib.ERR_ALIAS),
    ("id too large", dict(adapter_ids=BAD_IDS.ctypes.data, n=4), _lib.ERR_ADAPTER_ID),
    ("id negative", dict(adapter_ids=NEG_IDS.ctypes.data, n=2), _lib.ERR_ADAPTER_ID),
]


@pytest.mark.parametrize("name,kw,code", HOST_ID_REJECTS, ids=[r[0] for r in HOST_ID_REJECTS])
def test_lora_add_host_ids_rejects(name, kw, code):
    assert _host_ids(**kw) == code


def _noalloc(**kw):
    a = dict(stream=None, dtype=0, y=Y, ld_y=4096, x=X, ld_x=4096,
             adapter_ids=HOST_IDS.ctypes.data, n=32, A_pool=V, A_stride=16 * 4096,
             B_pool=V + (1 << 30), B_stride=16 * 4096, n_adapters=4096, h_in=4096, h_out=4096,
             r=16, scale=2.0)
    a.update(kw)
    return sgmv.sgmv_lora_add_host_ids_noalloc(**a)


NOALLOC_REJECTS = [
    ("n>64", dict(n=65), _lib.ERR_SHAPE),
    ("rank", dict(r=8), _lib.ERR_UNSUPPORTED),
    ("ids null", dict(adapter_ids=None), _lib.ERR_NULL),
    ("alias", dict(y=X + 64), _lib.ERR_ALIAS),
    ("id too large", dict(adapter_ids=BAD_IDS.ctypes.data, n=4), _lib.ERR_ADAPTER_ID),
    # partial sums of h_in = 32776 at r = 64 (8.4 MB) pass the static scratch's 8 MiB
    ("beyond scratch r64", dict(r=64, h_in=32776, ld_x=32776, A_stride=64 * 32776,
                                B_stride=64 * 4096), _lib.ERR_WORKSPACE),
    ("beyond scratch r16", dict(h_in=524296, ld_x=524296, A_stride=16 * 524296),
     _lib.ERR_WORKSPACE),
]


@pytest.mark.parametrize("name,kw,code", NOALLOC_REJECTS, ids=[r[0] for r in NOALLOC_REJECTS])
def test_lora_add_host_ids_noalloc_rejects(name, kw, code):
    assert _noalloc(**kw) == code


@pytest.mark.skipif(not _no_gpu_visible(), reason="needs a machine without a GPU: the fake "
                    "addresses would reach a kernel")
def test_lora_add_host_ids_noalloc_largest_shapes_pass_the_checks():
    """The largest shapes the static scratch holds pass every host check (and fail only for
    want of a device here)."""
    assert _noalloc(r=64, h_in=32768, ld_x=32768, A_stride=64 * 32768,
                    B_stride=64 * 4096) == _lib.ERR_HIP
    assert _noalloc(h_in=524288, ld_x=524288, A_stride=16 * 524288) == _lib.ERR_HIP
    assert _noalloc(n=0) == _lib.OK


def test_lora_add_host_ids_n_zero_is_ok():
    assert _host_ids(n=0) == _lib.OK


@pytest.mark.skipif(not _no_gpu_visible(), reason="needs a machine without a GPU: the fake "
                    "addresses would reach a kernel")
def test_lora_add_host_ids_valid_call_without_device_is_hip_error():
    assert _host_ids() == _lib.ERR_HIP


def test_check_workspace_rejects():
    L = _lib.lib()
    assert L.sgmv_check_workspace(None, None, None, 0) == _lib.ERR_NULL
    assert L.sgmv_check_workspace(None, WS + 16, None, 0) == _lib.ERR_WORKSPACE


@pytest.mark.skipif(not _no_gpu_visible(), reason="needs a machine without a GPU: the fake "
                    "address would be read")
def test_check_workspace_without_device_is_hip_error():
    assert _lib.lib().sgmv_check_workspace(None, WS, None, 0) == _lib.ERR_HIP


def test_status_strings_cover_every_code():
    for code in range(0, 10):
        assert sgmv.sgmv_status_string(code) != "unknown status", code
    assert sgmv.sgmv_status_string(10) == "unknown status"


def test_build_segments_device_rejects():
    L = _lib.lib()
    assert L.sgmv_build_segments_device(None, TAB, 4097, 4, V, V, V, V) == _lib.ERR_SHAPE
    assert L.sgmv_build_segments_device(None, None, 3, 4, V, V, V, V) == _lib.ERR_NULL


# --------------------------------------------------------------------------------------
# mixed ranks
# --------------------------------------------------------------------------------------
RANKED_CASES = [
    ("random", np.random.default_rng(21).integers(0, 7, 300), [64, 16, 32, 16, 64, 16, 32]),
    ("one_rank", np.random.default_rng(22).integers(0, 5, 50), [32] * 5),
    ("mixed70b", synth.mixed70b_ids(np.random.default_rng(23)), [16, 64] * 25),
    ("n1", np.array([2]), [16, 16, 64]),
    ("n0", np.zeros(0), [16]),
]


@pytest.mark.parametrize("name,ids,rank", RANKED_CASES, ids=[c[0] for c in RANKED_CASES])
def test_build_segments_ranked_matches_oracle(name, ids, rank):
    ids = np.asarray(ids, np.int32)
    tab = sgmv.sgmv_build_segments_ranked(ids, rank)
    perm, groups = oracle.segments_ranked(ids, np.array(rank, np.int32))
    assert np.array_equal(tab.perm, perm)
    assert len(tab.groups) == len(groups)
    for g, (r, row0, n, starts, seg_ad) in zip(tab.groups, groups):
        assert (g.r, g.row0, g.n, g.n_segments) == (r, row0, n, len(seg_ad))
        assert np.array_equal(tab.seg_starts[g.starts0: g.starts0 + g.n_segments + 1], starts)
        assert np.array_equal(tab.seg_adapter[g.seg0: g.seg0 + g.n_segments], seg_ad)
        lens = np.diff(starts)
        assert (g.min_seg_len, g.max_seg_len) == (int(lens.min()), int(lens.max()))
        assert g.scale == 1.0


def test_build_segments_ranked_rejects():
    with pytest.raises(sgmv.SgmvError) as e:
        sgmv.sgmv_build_segments_ranked(np.array([0, 3], np.int32), [16, 16, 16])
    assert e.value.status == _lib.ERR_ADAPTER_ID
    with pytest.raises(sgmv.SgmvError) as e:
        sgmv.sgmv_build_segments_ranked(np.array([0, 1], np.int32), [16, 24])
    assert e.value.status == _lib.ERR_UNSUPPORTED


def _groups(*gs):
    arr = (_lib.RankGroup * max(len(gs), 1))()
    for i, g in enumerate(gs):
        arr[i] = _lib.RankGroup(*g)
    return arr


def _ranked(groups, n_groups=None, **kw):
    a = dict(stream=None, dtype=1, y=Y, ld_y=4096, x=X, ld_x=4096, A_ptrs=TAB, B_ptrs=TAB + 256,
             seg_starts=TAB + 512, perm=TAB + 1024, n=64, h_in=4096, h_out=4096, workspace=WS,
             workspace_bytes=1 << 30)
    a.update(kw)
    arr = _groups(*groups)
    return sgmv.sgmv_lora_add_ranked(groups=ctypes.addressof(arr),
                                     n_groups=len(groups) if n_groups is None else n_groups, **a)


G16 = (16, 0, 32, 0, 0, 32, 1, 1, 2.0)      # r, row0, n, seg0, starts0, S, min, max, scale
G64 = (64, 32, 32, 32, 33, 2, 16, 16, 0.5)
RANKED_REJECTS = [
    ("rank", [G16, (24,) + G64[1:]], {}, _lib.ERR_UNSUPPORTED),
    ("rows past n", [G16, G64[:1] + (40,) + G64[2:]], {}, _lib.ERR_SHAPE),
    ("segment bounds", [G16, G64[:5] + (2, 20, 20, 0.5)], {}, _lib.ERR_SHAPE),
    ("negative seg0", [G16, G64[:3] + (-1,) + G64[4:]], {}, _lib.ERR_SHAPE),
    ("n_groups<0", [G16], dict(n_groups=-1), _lib.ERR_SHAPE),
    ("perm null", [G16, G64], dict(perm=None), _lib.ERR_NULL),
    ("dtype", [G16], dict(dtype=5), _lib.ERR_UNSUPPORTED),
    ("ws for r=16 only", [G16, G64], dict(workspace_bytes=sgmv.sgmv_workspace_bytes(64, 4096, 16)),
     _lib.ERR_WORKSPACE),
    # room for the largest group alone is not the buffer the header asks for (all rows at
    # the largest rank): side-by-side scratch could reach the decode path's partial sums
    ("ws per group only", [G16, G64],
     dict(workspace_bytes=sgmv.sgmv_workspace_bytes(32, 4096, 64)), _lib.ERR_WORKSPACE),
    ("alias", [G16, G64], dict(y=X + 64), _lib.ERR_ALIAS),
    ("h_in%8", [G16], dict(h_in=4092, ld_x=4092), _lib.ERR_ALIGNMENT),
]


@pytest.mark.parametrize("name,gs,kw,code", RANKED_REJECTS, ids=[r[0] for r in RANKED_REJECTS])
def test_lora_add_ranked_rejects(name, gs, kw, code):
    assert _ranked(gs, **kw) == code


def test_lora_add_ranked_empty_is_ok():
    assert _ranked([], n_groups=0, x=None, y=None) == _lib.OK
    assert _ranked([G16[:2] + (0, 0, 0, 0, 0, 0, 1.0)], n=0) == _lib.OK


def test_binding_rejects_mismatched_adapters():
    """The binding checks adapter shapes against x and y before anything reaches the GPU
    (the kernels read A and B with strides taken from h_in and h_out)."""
    import torch
    x = torch.zeros((4, 64), dtype=torch.bfloat16)
    y = torch.zeros((4, 32), dtype=torch.bfloat16)
    ids = torch.zeros(4, dtype=torch.int32)
    A = torch.zeros((3, 16, 64), dtype=torch.bfloat16)
    B = torch.zeros((3, 32, 16), dtype=torch.bfloat16)
    with pytest.raises(ValueError):   # h_in of A differs from x
        sgmv.lora_add_pool(y, x, ids, torch.zeros((3, 16, 72), dtype=torch.bfloat16), B, 1.0)
    with pytest.raises(ValueError):   # h_out of B differs from y
        sgmv.lora_add_pool(y, x, ids, A, torch.zeros((3, 40, 16), dtype=torch.bfloat16), 1.0)
    with pytest.raises(ValueError):   # rank of B differs from A
        sgmv.lora_add_pool(y, x, ids, A, torch.zeros((3, 32, 32), dtype=torch.bfloat16), 1.0)
    with pytest.raises(ValueError):   # A not dense
        sgmv.lora_add_pool(y, x, ids, torch.zeros((3, 64, 16), dtype=torch.bfloat16).transpose(1, 2), B, 1.0)
    with pytest.raises(ValueError):   # pools of different sizes
        sgmv.lora_add_pool(y, x, ids, A, B[:2], 1.0)
    with pytest.raises(ValueError):   # ids of the wrong type
        sgmv.lora_add_pool(y, x, ids.long(), A, B, 1.0)
