"""Host-side helpers of bench.py (no GPU): algorithmic byte counts."""
import numpy as np

import bench


def test_stage_bytes_decode_32k():
    # one decode query at 32767: 256 representatives, 64 kept blocks of 128 keys
    b = bench.hisa_stage_bytes(np.array([32767]), 128, 64, 2048)
    assert b["block_stage"] == 128 + 256 * 128 + 2 * 64 * 4
    assert b["token_ideal"] == 128 + 64 * 4 + 8192 * 128 + 2048 * 8
    assert b["token_topk"] == 8192 * 4 + 64 * 4 + 2048 * 8
    f = bench.flat_stage_bytes(np.array([32767, 32767]), 2048)
    assert f["flat_scores"] == 2 * (32768 * 132 + 128)
    assert f["flat_topk"] == 2 * (32768 * 4 + 2048 * 8)


def test_stage_bytes_early_queries_are_causal():
    b = bench.hisa_stage_bytes(np.array([0, 200]), 128, 64, 16)
    # query 0 sees one block and one key, query 200 two blocks and 201 keys
    assert b["token_ideal"] == 2 * (128 + 64 * 4 + 16 * 8) + (1 + 201) * 128
