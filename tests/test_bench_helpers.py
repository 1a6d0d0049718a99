"""Host-side helpers of bench.py (no GPU): algorithmic byte counts."""
import numpy as np

import bench


def test_stage_bytes_decode_32k():
    # one decode query at 32767: 256 representatives, 64 kept blocks of 128
    # keys; only inputs read once and the int32 output count (no workspace)
    b = bench.hisa_stage_bytes(np.array([32767]), 128, 64, 2048)
    assert b["block_stage"] == 128 + 256 * 128
    assert b["token_scores"] == 128 + 8192 * 128
    assert b["select_and_scores"] == 128 + 256 * 128 + 8192 * 128
    assert b["token_ideal"] == 128 + 256 * 128 + 8192 * 128 + 2048 * 4
    assert b["token_topk"] == 2048 * 4
    # the 16-sequence decode batch: 17.30 MB of representatives, keys and queries
    b16 = bench.hisa_stage_bytes(np.full(16, 32767), 128, 64, 2048)
    assert b16["select_and_scores"] == 16 * (128 + (256 + 8192) * 128) == 17303552
    f = bench.flat_stage_bytes(np.array([32767, 32767]), 2048)
    assert f["flat_scores"] == 2 * (32768 * 128 + 128)
    assert f["flat_topk"] == 2 * 2048 * 4


def test_stage_bytes_early_queries_are_causal():
    b = bench.hisa_stage_bytes(np.array([0, 200]), 128, 64, 16)
    # query 0 sees one block and one key, query 200 two blocks and 201 keys
    assert b["token_ideal"] == 2 * (128 + 16 * 4) + (1 + 2) * 128 + (1 + 201) * 128


def test_visible_candidates():
    # every causal key while all causal blocks are kept; past that, m-1 whole
    # blocks and the visible part of the query's own block
    c = bench.visible_candidates(np.array([0, 200, 8191, 8192, 10000, 32767]), 128, 64)
    assert c.tolist() == [1, 201, 8192, 63 * 128 + 1, 63 * 128 + 10000 % 128 + 1, 8192]
    # the whole 32K causal prefill: 233,324,544 (query, candidate) pairs
    assert int(bench.visible_candidates(np.arange(32768), 128, 64).sum()) == 233324544


def test_stage_flops_and_bound():
    f = bench.stage_flops(np.array([32767, 200]), 128, 64)
    assert f["block_stage"] == 128 * (256 + 2)
    assert f["token_scores"] == 128 * (8192 + 201)
    assert f["flat_scores"] == 128 * (32768 + 201)
    # few queries: HBM; many: the MFMA tiles
    assert bench.stage_roofline("d/token_scores", 1.0, 16, 1e9, 1e6)[0] == "hbm"
    b, a, p, u, w = bench.stage_roofline("p/token_scores", 1.0, 4096, 1e12, 1e6)
    assert (b, u, w) == ("mfma", "TFLOP/s", 1e12) and abs(a - 1000.0) < 1e-9


def test_row_overlap():
    a = np.array([[0, 1, 2, 3], [5, 6, -1, -1], [-1, -1, -1, -1]])
    f = np.array([[2, 3, 4, 5], [5, 6, -1, -1], [-1, -1, -1, -1]])
    iou, rec = bench.row_overlap(a, f)
    # row 0: 2 shared of 6 distinct, 2 of 4 flat; row 1 identical; row 2 empty on both sides
    assert abs(iou - (2 / 6 + 1 + 1) / 3) < 1e-12
    assert abs(rec - (0.5 + 1 + 1) / 3) < 1e-12


def test_traffic_lookup_takes_the_kernel_the_step_runs(tmp_path):
    src = tmp_path / "long_context_sparse_hisa_amd" / "csrc"
    src.mkdir(parents=True)
    (src / "k.hip").write_text("// kernels\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    sha = bench.kernel_source_hash(str(tmp_path))
    (prof / "w_hbm_traffic.md").write_text(
        "source_sha256 = %s\n" % sha
        + "traffic\tw\tvoid hisa::decode_fused_kernel<1>(x)\t100\n"
        + "traffic\tw\tvoid hisa::decode_step_kernel<1>(x)\t200\n")
    root = str(tmp_path)
    assert bench.measured_traffic(root, "w", "decode/select_and_scores", fused_step=True) == 200.0
    assert bench.measured_traffic(root, "w", "decode/select_and_scores") == 100.0
    assert bench.measured_traffic(root, "other", "decode/select_and_scores") is None
    # a changed kernel source voids the figure
    (src / "k.hip").write_text("// kernels, edited\n")
    assert bench.measured_traffic(root, "w", "decode/select_and_scores", fused_step=True) is None


def test_stage_names_follow_the_library_split():
    # few queries with at most 2048 blocks: stage 1 and the token scores are
    # one kernel (stage 1 of the events); otherwise three stages
    assert bench.hisa_stage_names(16, 32768, 128) == {1: "select_and_scores", 2: "token_topk"}
    assert bench.hisa_stage_names(256, 32768, 128) == {1: "select_and_scores", 2: "token_topk"}
    assert bench.hisa_stage_names(16, 1 << 20, 128) == dict(enumerate(bench.STAGES_HISA))
    assert bench.hisa_stage_names(4096, 32768, 128) == dict(enumerate(bench.STAGES_HISA))


def test_many_row_kernels_carry_their_stage():
    # the many-row forms of the top-k and of the select from scores are
    # looked up under their stages like the plain forms
    assert any("topk_rows_many_kernel" == s for s in bench.STAGE_KERNEL["token_topk"])
    assert any("stage1_select_many_kernel" == s for s in bench.STAGE_KERNEL["block_stage"])
    assert bench.DECODE_FOLD_MAX_SEQS == 64


def test_long_row_kernels_carry_their_stage():
    # the two-walk block selection and the block-major token scores are
    # looked up under their stages, so the line finds their traffic
    assert "block_select_tile_kernel" in bench.STAGE_KERNEL["block_stage"]
    assert "stage2_gather_kernel" in bench.STAGE_KERNEL["token_scores"]
