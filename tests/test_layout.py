"""Properties of the tiled weight layout (include/moe.h, moe_prepare_weights) that the GEMM epilogues
rely on, checked against the oracle's reading of the plain W1 row order (gate/up interleaved by 8;
"MegaMoE" walk-through section 7.3 and SymmBuffer page section 7.2).  The GPU tests compare the device
re-layout with the same documented permutation, so together they pin the kernel's layout to the
oracle's.

An MFMA output lane j of a 16-column block owns tile column 16b + j of its wave's columns; the
properties are stated per (64- or 128-column group, block b, lane j)."""
import numpy as np
import pytest

from oracle.forward import deinterleave_gate_up
from parity import tile_columns


@pytest.mark.parametrize("which", [1, 2])
def test_tile_permutation_is_a_bijection(which):
    assert np.array_equal(np.sort(tile_columns(which)), np.arange(256))


def test_w1_gate_and_up_of_a_channel_share_a_lane():
    # raw rows of the gate and the up row of each of the 128 channels of a 256-row block, as the oracle
    # reads the interleaved W1
    gate_row, up_row = deinterleave_gate_up(np.arange(256))
    src = tile_columns(1)
    for G in range(4):            # 64-column group = 32 channels = one UE8M0 requant group
        for j in range(16):       # lane
            for k in range(2):
                ch = 32 * G + 2 * j + k
                assert src[64 * G + 16 * k + j] == gate_row[ch]        # block k: gate
                assert src[64 * G + 16 * (k + 2) + j] == up_row[ch]    # block k + 2: up, same lane


def test_w1_group_holds_one_requant_group_with_adjacent_lane_outputs():
    gate_row, _ = deinterleave_gate_up(np.arange(256))
    channel_of_gate_row = {int(r): ch for ch, r in enumerate(gate_row)}
    src = tile_columns(1)
    for G in range(4):
        chans = sorted(channel_of_gate_row[int(src[64 * G + 16 * b + j])] for b in range(2) for j in range(16))
        assert chans == list(range(32 * G, 32 * G + 32))  # the group's gate columns: 32 consecutive channels
        for j in range(16):                                # lane j: channels 2j, 2j + 1 (one 2-byte FP8 store)
            assert [channel_of_gate_row[int(src[64 * G + 16 * k + j])] for k in range(2)] == \
                [32 * G + 2 * j, 32 * G + 2 * j + 1]


def test_w2_lane_holds_adjacent_outputs():
    src = tile_columns(2)
    for S in range(2):            # 128-column span
        for j in range(16):
            cols = [int(src[128 * S + 16 * b + j]) for b in range(8)]
            assert cols == list(range(128 * S + 8 * j, 128 * S + 8 * j + 8))  # one 16-byte BF16 store
            half = [int(src[128 * S + 16 * b + j]) for b in range(4)]          # a 64-column wave: 8 bytes
            assert half == list(range(128 * S + 8 * j, 128 * S + 8 * j + 4))
