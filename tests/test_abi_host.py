"""CPU-side checks of the C ABI: the library loads, exports every symbol the
header declares, and its host-only logic (status codes, validation before
allocation, the batch precondition check and split-K item counts) behaves as
"Forward Cuda Gemma", decodeBatch / allocSlotKv / slotKvOffsetBytes and
"Forward Cuda", slot reset, state.  No call here touches a GPU."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sequence_slot_kv_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "slot_kv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(slot_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = header_functions()
    assert len(names) >= 13
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/slot_kv.h but not exported"
    assert sorted(b.EXPORTS) == names


def test_strerror_names_every_status():
    seen = set()
    for code in (0, -1, -2, -3, -4, -5, -6, -7):
        s = b.slot_kv_strerror(code)
        assert s and s != "unknown status"
        seen.add(s)
    assert len(seen) == 8
    assert b.slot_kv_strerror(-99) == "unknown status"


def test_unallocated_handle_paths():
    h = b.slot_kv_create()
    try:
        assert b.slot_kv_offset_bytes(h, 0, 0, 0)[0] == b.SLOT_KV_ENOTALLOC
        assert b.slot_kv_layer_ptrs(h, 0)[0] == b.SLOT_KV_ENOTALLOC
        # "Forward Cuda", reset on admit: a no-op when slot state is unallocated
        assert b._lib.slot_reset(h, 12345, None) == b.SLOT_KV_OK
        many = np.array([7, 9999], np.uint32)
        assert b._lib.slot_reset_batch(h, many.ctypes.data_as(b._u32p), 2, None) == b.SLOT_KV_OK
        assert b.slot_conv_offset_bytes(h, 0, 0)[0] == b.SLOT_KV_ENOTALLOC
        assert b.slot_ssm_offset_bytes(h, 0, 0)[0] == b.SLOT_KV_ENOTALLOC
        assert b.slot_state_ptrs(h, 0)[0] == b.SLOT_KV_ENOTALLOC
        ones = np.ones(64, np.float32)
        assert b.slot_kv_set_layer(h, 0, 4, 2, 64, ones, ones, ones[:32]) == b.SLOT_KV_ENOTALLOC
        assert b._lib.slot_decode_attn(h, 0, None, None, None, None, None, 0, None,
                                       None) == b.SLOT_KV_ENOTALLOC
        assert b._lib.slot_kv_alloc(h, 0, 128, None, 0) == b.SLOT_KV_EINVAL
        dims = np.array([128], np.uint32)
        assert b._lib.slot_kv_alloc(h, 4, 0, dims.ctypes.data_as(b._u32p), 1) == b.SLOT_KV_EINVAL
        zero = np.array([0], np.uint32)
        assert b._lib.slot_kv_alloc(h, 4, 128, zero.ctypes.data_as(b._u32p), 1) == b.SLOT_KV_EINVAL
        # slot_state_alloc: argument checks that precede any device call
        u = lambda a: np.asarray(a, np.uint32).ctypes.data_as(b._u32p)
        lens = np.array([8, 16], np.uint32)
        p8 = lens.ctypes.data_as(b._u32p)
        assert b._lib.slot_state_alloc(h, 4, 16, None, 0, None, None, 0) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 0, 16, None, 0, p8, p8, 1) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 4, 16, None, 1, p8, p8, 1) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 4, 16, None, 0, None, p8, 1) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 4, 16, None, 0, p8, None, 1) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 4, 16, None, 0, zero.ctypes.data_as(b._u32p), p8,
                                       1) == b.SLOT_KV_EINVAL
        big = np.array([0xFFFFFFFF] * 1100, np.uint32)  # one slot: 2^31 tiles and more
        assert b._lib.slot_state_alloc(h, 4, 16, None, 0, big.ctypes.data_as(b._u32p),
                                       big.ctypes.data_as(b._u32p), 1100) == b.SLOT_KV_EINVAL
    finally:
        b.slot_kv_destroy(h)
    b.slot_kv_destroy(None)  # NULL accepted
    assert b._lib.slot_kv_create(None) == b.SLOT_KV_EINVAL


def test_alloc_size_overflow_is_einval_before_any_device_call():
    # "Forward Cuda Gemma", allocSlotKv; "Forward Cuda", slot state: a K/V
    # buffer holds n_slots * slot_ctx * kv_dim floats, a state buffer
    # n_slots * len.  A byte size past 2^64 - 1 would wrap to a small
    # allocation that the 64-bit offsets then overrun, so it is rejected
    # with EINVAL before any HIP call (here, with no GPU, any device call
    # would return EDEVICE instead).
    u = lambda a: np.asarray(a, np.uint32)  # noqa: E731
    p = lambda a: a.ctypes.data_as(b._u32p)  # noqa: E731
    h = b.slot_kv_create()
    try:
        dims = u([2**30])
        # 2^16 * 2^16 * 2^30 * 4 = 2^64: wraps to 0 in 64-bit arithmetic
        assert b._lib.slot_kv_alloc(h, 65536, 65536, p(dims), 1) == b.SLOT_KV_EINVAL
        two = u([128, 2**30])  # the second layer overflows: nothing is allocated
        assert b._lib.slot_kv_alloc(h, 65536, 65536, p(two), 2) == b.SLOT_KV_EINVAL
        assert b._lib.slot_kv_alloc(h, 2**32 - 1, 2**32 - 1, p(u([2**31])), 1) == b.SLOT_KV_EINVAL
        # the state analogues: n_slots * len * 4 past 2^64 - 1
        ok, big = u([8]), u([2**31])
        assert b._lib.slot_state_alloc(h, 2**32 - 1, 1, None, 0, p(big), p(ok),
                                       1) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 2**32 - 1, 1, None, 0, p(ok), p(big),
                                       1) == b.SLOT_KV_EINVAL
        assert b._lib.slot_state_alloc(h, 2**32 - 1, 2, p(dims), 1, p(ok), p(ok),
                                       1) == b.SLOT_KV_EINVAL  # attention part overflows
        assert b.slot_kv_offset_bytes(h, 0, 0, 0)[0] == b.SLOT_KV_ENOTALLOC  # nothing kept
        # one float short of the wrap passes the size check and reaches the
        # device (which this host does not have, or which cannot hold it)
        rc = b._lib.slot_kv_alloc(h, 65535, 65536, p(dims), 1)
        assert rc in (b.SLOT_KV_EDEVICE, b.SLOT_KV_ENOMEM)
    finally:
        b.slot_kv_destroy(h)


@pytest.mark.parametrize("seed", range(20))
def test_check_batch_agrees_with_oracle(seed):
    # Host validation of the library against the oracle's preconditions on
    # random batches, including out-of-range and repeated slots.
    rng = np.random.default_rng(seed)
    n_slots, slot_ctx = int(rng.integers(1, 40)), int(rng.integers(1, 600))
    B = int(rng.integers(0, 12))
    slots = rng.integers(0, n_slots + (seed % 3 == 0), size=B)
    if seed % 4 == 1 and B > 1:
        slots[-1] = slots[0]
    positions = rng.integers(0, slot_ctx + (seed % 5 == 0), size=B)
    rc, items, split = b.slot_kv_check_batch(n_slots, slot_ctx, positions, slots, chunk_keys=64)
    assert rc == oracle.check_batch(n_slots, slot_ctx, positions, slots)
    if rc == 0:
        assert items == sum(-(-(int(p) + 1) // 64) for p in positions)
        assert split == sum(int(p) + 1 > 64 for p in positions)


def test_check_batch_error_codes():
    assert b.slot_kv_check_batch(4, 128, [0, 127], [0, 3])[0] == b.SLOT_KV_OK
    assert b.slot_kv_check_batch(4, 128, [128], [0])[0] == b.SLOT_KV_ERANGE
    assert b.slot_kv_check_batch(4, 128, [0], [4])[0] == b.SLOT_KV_ERANGE
    assert b.slot_kv_check_batch(4, 128, [1, 2], [2, 2])[0] == b.SLOT_KV_EDUP
    assert b.slot_kv_check_batch(4, 128, [], [])[0] == b.SLOT_KV_OK
    assert b.slot_kv_check_batch(4, 128, [1], [1], chunk_keys=0)[0] == b.SLOT_KV_EINVAL
    # range errors win over duplicates only by scan order; both are errors
    assert b.slot_kv_check_batch(2**20, 2**20, [2**20 - 1], [2**20 - 1])[0] == b.SLOT_KV_OK


def test_chunk_keys_is_a_multiple_of_the_wave():
    C = b.slot_kv_chunk_keys()
    assert C >= 64 and C % 64 == 0
