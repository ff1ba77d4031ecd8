"""Work and byte counts bench.py reports, on hand-built selections (CPU only)."""
import numpy as np

import bench

UNIT = 16 * 128 * 128 * 4          # one 16-row wave over one 128-key block, QK + PV at d = 128
USEFUL = 128 * 4 * 2 * (128 + 128)  # one list (4 q heads) over one fully visible block


def _case(seq_len, q_len, picks):
    """ids [4 index heads, q_len, 4] with picks {(head, token): [blocks]}, one sequence."""
    ids = np.full((4, q_len, 4), -1, np.int32)
    for (h, t), blocks in picks.items():
        ids[h, t, :len(blocks)] = blocks
    cu = np.array([0, q_len], np.int32)
    _, pos = bench.token_positions(cu, np.array([seq_len], np.int32))
    issued = bench.block_prefill_issued_flops(ids, cu, pos, 16, 2, 4, 128, seq_len // 128)
    useful = bench.block_attention_flops(ids, pos, 16, 4, 128, 128)
    return issued, useful


def test_one_selection_costs_one_wave_block():
    issued, useful = _case(512, 4, {(0, 0): [2]})
    assert issued == UNIT and useful == USEFUL


def test_rows_of_one_wave_share_its_block():
    # tokens 0 and 1 sit in one wave (16 rows = 2 tokens x 8 heads), so both
    # index heads of the kv head selecting block 2 still issue one unit
    issued, useful = _case(512, 4, {(0, 0): [2], (1, 1): [2]})
    assert issued == UNIT and useful == 2 * USEFUL


def test_waves_skip_blocks_none_of_their_rows_selected():
    # wave 0 (tokens 0, 1) takes block 2, wave 1 (tokens 2, 3) block 3: the
    # union is {2, 3} but each wave computes only its own block (token 2, at
    # position 510, sees 127 keys of block 3; the kernel still computes 128)
    issued, useful = _case(512, 4, {(0, 0): [2], (0, 2): [3]})
    assert issued == 2 * UNIT and useful == USEFUL + 127 * 4 * 2 * 256


def test_kv_heads_are_separate_workgroups():
    # index heads 0, 1 belong to kv head 0 and 2, 3 to kv head 1
    issued, _ = _case(512, 4, {(0, 0): [1], (3, 0): [1]})
    assert issued == 2 * UNIT


def test_blocks_past_the_position_are_not_visited():
    # token 0 of a 200-token suffix of 512 sits at position 312: block 3
    # (keys 384..511) holds no key it can see, block 2 only keys 256..312
    issued, useful = _case(512, 200, {(0, 0): [3]})
    assert issued == 0 and useful == 0
    issued, useful = _case(512, 200, {(0, 0): [2]})
    assert issued == UNIT and useful == (312 - 256 + 1) * 4 * 2 * 256


def test_workgroups_hold_32_tokens():
    # tokens 0 and 32 are in different workgroups: two unions, one unit each
    issued, _ = _case(8192, 64, {(0, 0): [5], (0, 32): [5]})
    assert issued == 2 * UNIT


def test_head_groups_that_do_not_divide_a_wave_are_not_modelled():
    ids = np.full((1, 4, 4), -1, np.int32)
    cu = np.array([0, 4], np.int32)
    _, pos = bench.token_positions(cu, np.array([512], np.int32))
    assert bench.block_prefill_issued_flops(ids, cu, pos, 24, 1, 1, 128, 4) is None
