"""The C-ABI library loads on a CPU-only host, exports every declared entry point,
and rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

import cache_aware_query_amd as caq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            text = open(os.path.join(inc, f)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(wa_[a-z0-9_]+)\s*\(", text))
    return names


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(caq.LIB_PATH):
        pytest.fail("libwavealign.so is not built; run __graft_entry__.build()")
    return caq.load_library()


def test_every_declared_symbol_is_exported(lib):
    declared = _declared()
    assert declared, "no declarations found"
    assert declared == set(caq.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version(lib):
    assert lib.wa_abi_version() == 4


def test_default_schedule_follows_the_head_size(lib):
    # All heads at once while one head's K and V (MB * block * head_dim * 4 bytes) take
    # at most 12 MiB; XCD-sliced in the original order beyond (a host-only call).
    hi, xcd = caq.WA_SCHED_HEADS_INTERLEAVED, caq.WA_SCHED_XCD_SLICED
    assert caq.default_schedule(192 * 128, 128, 128) == hi        # 192 blocks: exactly 12 MiB
    assert caq.default_schedule(192 * 128 + 1, 128, 128) == xcd   # 193 blocks
    assert caq.default_schedule(57 * 128, 128, 128) == hi
    assert caq.default_schedule(75600, 128, 128) == xcd
    assert caq.default_schedule(768 * 64, 64, 64) == hi           # 768 blocks of 64 x 64
    assert caq.default_schedule(768 * 64 + 1, 64, 64) == xcd
    out = ctypes.c_int32()
    assert lib.wa_default_schedule(0, 128, 128, ctypes.byref(out)) == -1
    assert lib.wa_default_schedule(100, 96, 128, ctypes.byref(out)) == -2
    assert lib.wa_default_schedule(100, 128, 128, None) == -1


def test_host_validation_rejects_bad_arguments(lib):
    # Null pointers and bad sizes are refused on the host; nothing reaches HIP.
    assert lib.wa_build_block_index(None, 1, 1, 1, None, None, 0, None, None, None, 0, None) == -1
    assert b"null" in lib.wa_last_error()
    n = ctypes.c_size_t()
    assert lib.wa_sparse_attn_workspace_size(2, 1000, 96, 128, ctypes.byref(n)) == -2
    assert lib.wa_sparse_attn_workspace_size(2, 1000, 128, 128, ctypes.byref(n)) == 0
    assert n.value == 256  # the WA_SCHED_AUTO choice; K and V are read in place
    assert lib.wa_last_error() == b""
    fake = ctypes.c_void_p(16)
    assert lib.wa_topp_select(fake, fake, fake, 4, 1, 1, 1, 1.5, fake, None) == -1
    assert lib.wa_topp_select(fake, fake, fake, 4, 1, 1, 5000, 0.5, fake, None) == -2
    assert lib.wa_topp_select(fake, fake, fake, -1, 1, 1, 1, 0.5, fake, None) == -1
    assert lib.wa_mask_recall(None, fake, fake, 4, 1, 1, 1, fake, fake, None) == -1
    assert lib.wa_mask_recall(fake, fake, fake, 4, 1, 1, 5000, fake, fake, None) == -2
    assert lib.wa_mask_recall(fake, fake, fake, -1, 1, 1, 1, fake, fake, None) == -1
    p = caq.ReorderParams(wave=0)._c()
    assert lib.wa_reorder_rows(fake, fake, fake, fake, 16, fake, 1, 4, 4, 128, 128,
                               ctypes.byref(p), fake, fake, fake, None, None, None) == -1
    p = caq.ReorderParams()._c()
    assert lib.wa_reorder_rows(fake, fake, fake, fake, 16, fake, 1, 5000, 4, 128, 128,
                               ctypes.byref(p), fake, fake, fake, None, None, None) == -2
    # the transposed lists are required once the mask no longer fits LDS as bitmasks
    assert lib.wa_reorder_rows(fake, fake, None, None, 16, fake, 1, 1000, 1000, 128, 128,
                               ctypes.byref(p), fake, fake, fake, None, None, None) == -1
    assert b"csc" in lib.wa_last_error()
    # MinHash order: coefficient ranges, hash count, geometry and sizes are checked first
    ga = (ctypes.c_uint32 * 2)(5, 7)
    gb = (ctypes.c_uint32 * 2)(1, 2)
    zero = (ctypes.c_uint32 * 2)(0, 7)
    big = (ctypes.c_uint32 * 2)(5, 0x7fffffff)
    assert lib.wa_minhash_order(fake, fake, 16, 1, 4, 4, zero, gb, 2, 4, 1, 1, fake, fake,
                                None) == -1
    assert lib.wa_minhash_order(fake, fake, 16, 1, 4, 4, ga, big, 2, 4, 1, 1, fake, fake,
                                None) == -1
    assert lib.wa_minhash_order(fake, fake, 16, 1, 4, 4, ga, gb, 3, 4, 1, 1, fake, fake,
                                None) == -1
    assert lib.wa_minhash_order(fake, fake, 16, 1, 4, 4, ga, gb, 2, 0, 1, 1, fake, fake,
                                None) == -1
    assert lib.wa_minhash_order(fake, fake, 16, 1, 5000, 4, ga, gb, 2, 4, 1, 1, fake, fake,
                                None) == -2
    assert lib.wa_minhash_order(None, fake, 16, 1, 4, 4, ga, gb, 2, 4, 1, 1, fake, fake,
                                None) == -1
    # negative capacity, bad schedule and non-positive scale are refused on the host
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, -1, None, 0, 1,
                                  0.1, fake, fake, None, None, 0, None) == -1
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1, None, 0, 7,
                                  0.1, fake, fake, None, None, 0, None) == -1
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1, None, 0, 5,
                                  0.1, fake, fake, None, None, 0, None) == -1
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1, None, 0, 1,
                                  -0.1, fake, fake, None, None, 0, None) == -1
    # the workspace is required (it carries the WA_SCHED_AUTO choice)
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1, None, 0, 3,
                                  0.1, fake, fake, None, None, 0, None) == -3
    assert lib.wa_attn_schedule_select(fake, 4, fake, 16, None) == -3
    assert lib.wa_attn_schedule_select(None, 4, fake, 256, None) == -1
    assert lib.wa_attn_schedule_select(fake, 0, fake, 256, None) == -1
    # the slice count of a permutation is checked against the range before the device
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1, fake, -1, 1,
                                  0.1, fake, fake, None, fake, 256, None) == -1
    assert lib.wa_sparse_attn_fwd(fake, fake, fake, 1, 128, 128, 128, fake, fake, 1, fake, 65, 1,
                                  0.1, fake, fake, None, fake, 256, None) == -1
    assert b"perm_slices" in lib.wa_last_error()
    # the XCD placement probe checks its arguments on the host
    assert lib.wa_xcd_placement(0, 128, fake, None) == -1
    assert lib.wa_xcd_placement(4, 128, None, None) == -1
    assert lib.wa_xcd_placement(4, 96, fake, None) == -2
    # unaligned pointer
    odd = ctypes.c_void_p(18)
    assert lib.wa_sparse_attn_fwd(odd, fake, fake, 1, 128, 128, 128, fake, fake, 1, None, 0, 1,
                                  0.1, fake, fake, None, None, 0, None) == -1
    # overlapping gather
    assert lib.wa_gather_blocks(fake, fake, fake, 1, 2, 64, None) == -1


def test_reorder_needs_csc_threshold(lib):
    assert lib.wa_reorder_needs_csc(591, 591) == 0
    assert lib.wa_reorder_needs_csc(16, 16) == 0
    assert lib.wa_reorder_needs_csc(929, 929) == 0
    assert lib.wa_reorder_needs_csc(972, 972) == 0
    assert lib.wa_reorder_needs_csc(973, 973) == 1
    assert lib.wa_reorder_needs_csc(1000, 1000) == 1
    assert lib.wa_reorder_needs_csc(0, 5) < 0
