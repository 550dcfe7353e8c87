"""Values the pages print, as small fixtures under tests/golden/ (CPU)."""
import json
import os

from input_adaptive_reduced_score_amd import accounting as A

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_gemm_flops_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "gemm_flops_worked_example.json")))
    f = A.gemm_flops(g["m"], g["n"], g["k"])
    assert f == g["exact_flops"]
    assert round(f / 1e6) == g["quoted_flops_millions"]


def test_reduced_down_projection_flops():
    # blog section 6.2: the reduced down projection costs 2 * H * active_M per token, i.e. the
    # dense count scaled by the kept fraction of the contraction dimension
    H, M = 1024, 4096
    assert A.linear_flops(1, M // 2, H) == 2 * H * (M // 2)
    assert A.linear_flops(1, M // 2, H) * 2 == A.gemm_flops(1, H, M)


def test_decode_step_bytes_at_the_four_ratios():
    # retained bytes of one decode step (x, c, idx written and read, kept W^T rows, y)
    K, M = 14336, 4096
    got = [A.decode_step_bytes(K, M, int(K * r)) for r in (0.25, 0.5, 0.75, 1.0)]
    assert [round(b / 1e6, 2) for b in got] == [29.49, 58.88, 88.27, 117.66]
