"""Pins of the oracle's per-slot SSM state ("Forward Cuda": allocation of the
per-sequence slot state, the conv-ring and recurrent-state byte offsets, the
reset of a reused slot on admit, and the sub-step 4a smoke that distinct
slots map to non-overlapping regions).

The offsets are pinned to closed forms and to a brute-force tiling of each
buffer; the reset to a byte-level scan of every buffer, comparing against
what the page fixes: the listed slots' conv ring and recurrent state are zero
in every ssm layer, and every other byte is unchanged.
"""
import numpy as np
import pytest

import oracle


def test_offsets_closed_form_and_64_bit():
    assert oracle.slot_state_offset_bytes(0, 123) == 0
    assert oracle.slot_state_offset_bytes(5, 24576) == 5 * 24576 * 4
    # 1000 slots of a 2^20-float recurrent state end past 2^32 bytes
    assert oracle.slot_state_offset_bytes(1023, 1 << 20) == 1023 * (1 << 22)
    assert oracle.slot_state_offset_bytes(2**32 - 1, 2**32 - 1) == (2**32 - 1) ** 2 * 4 % 2**64


@pytest.mark.parametrize("n_slots,state_len", [(2, 1), (3, 7), (8, 24), (5, 1001)])
def test_slots_tile_the_buffer(n_slots, state_len):
    # "Forward Cuda", sub-step 4a smoke: distinct slots map to non-overlapping
    # regions; together they cover the [n_slots][state_len] buffer exactly.
    owner = np.full(n_slots * state_len * 4, -1)
    for s in range(n_slots):
        off = oracle.slot_state_offset_bytes(s, state_len)
        assert np.all(owner[off:off + state_len * 4] == -1)
        owner[off:off + state_len * 4] = s
    assert np.all(owner >= 0)
    # slot 0 and the last slot differ (the smoke requires n_slots >= 2)
    assert oracle.slot_state_offset_bytes(n_slots - 1, state_len) >= state_len * 4


def _state(rng, n_slots, conv_lens, ssm_lens):
    conv = [rng.standard_normal((n_slots, c)).astype(np.float32) for c in conv_lens]
    ssm = [rng.standard_normal((n_slots, s)).astype(np.float32) for s in ssm_lens]
    return conv, ssm


def _check_reset(before_conv, before_ssm, conv, ssm, slots):
    reset = set(int(s) for s in slots)
    for b, a in zip(before_conv + before_ssm, conv + ssm):
        for s in range(a.shape[0]):
            if s in reset:
                assert a[s].tobytes() == bytes(a[s].nbytes)  # +0.0 in every float
            else:
                assert a[s].tobytes() == b[s].tobytes()


@pytest.mark.parametrize("slots", [[2], [0, 4], [4, 1, 3], [1, 1], []])
def test_reset_zeroes_exactly_the_listed_slots(slots):
    rng = np.random.default_rng(70 + len(slots))
    conv_lens, ssm_lens = [3, 12, 5], [16, 7, 33]  # per-layer sizes differ
    conv, ssm = _state(rng, 5, conv_lens, ssm_lens)
    c0, s0 = [a.copy() for a in conv], [a.copy() for a in ssm]
    assert oracle.slot_reset(conv, ssm, slots) == 0
    _check_reset(c0, s0, conv, ssm, slots)


def test_reset_validates_before_writing():
    rng = np.random.default_rng(80)
    conv, ssm = _state(rng, 4, [4, 6], [8, 10])
    c0, s0 = [a.copy() for a in conv], [a.copy() for a in ssm]
    assert oracle.slot_reset(conv, ssm, [1, 4]) == oracle.ERANGE  # the second slot is past the end
    _check_reset(c0, s0, conv, ssm, [])                         # nothing written
    assert oracle.slot_reset(conv, ssm, [3]) == 0                  # the last slot is in range
    _check_reset(c0, s0, conv, ssm, [3])


def test_reset_without_state():
    # no state allocated: a no-op that succeeds, whatever the slot
    assert oracle.slot_reset([], [], [7], n_slots=0) == 0
    # slots allocated but no ssm layer: validation only
    assert oracle.slot_reset([], [], [3], n_slots=4) == 0
    assert oracle.slot_reset([], [], [4], n_slots=4) == oracle.ERANGE


def test_reset_then_accumulate_matches_fresh_state():
    # The page's reason for the reset: state that accumulates over a sequence
    # (here a running sum per slot, the simplest accumulation) must start a new
    # request from the same state as a freshly allocated slot.
    rng = np.random.default_rng(81)
    n_slots, L = 3, 9
    conv, ssm = [np.zeros((n_slots, L), np.float32)], [np.zeros((n_slots, 2 * L), np.float32)]
    fresh = [np.zeros((n_slots, L), np.float32)], [np.zeros((n_slots, 2 * L), np.float32)]
    for _ in range(4):  # an earlier request on slot 1
        conv[0][1] += rng.standard_normal(L).astype(np.float32)
        ssm[0][1] += rng.standard_normal(2 * L).astype(np.float32)
    assert oracle.slot_reset(conv, ssm, [1]) == 0
    x = rng.standard_normal(L).astype(np.float32)
    conv[0][1] += x
    fresh[0][0][1] += x
    assert conv[0].tobytes() == fresh[0][0].tobytes() and ssm[0].tobytes() == fresh[1][0].tobytes()
