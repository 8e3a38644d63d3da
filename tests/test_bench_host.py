"""Host-side logic of bench.py, on the CPU: the FLOP convention of the
handbook's zigzag work model (section "之字形切分": a diagonal chunk pair
counts half), its agreement with the library's ring plan, the one-GPU
guard, and the traffic figure's tie to the kernel source it was taken for.
"""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_headline_flop_counts():
    # one zigzag rank of 8 at 128K, 32 heads, D = 128: 16 chunk units of
    # 8192^2 pairs (2 per ring step) = 2^44; the Ulysses share (4 heads over
    # the whole causal sequence) is the same 2^44
    assert bench.ring_share_flop(131072, 32, 128, 8, "zigzag", 0) == 2.0 ** 44
    assert bench.ulysses_share_flop(131072, 4, 128) == 2.0 ** 44
    # the whole layer is P times a balanced share
    assert 8 * bench.ring_share_flop(131072, 32, 128, 8, "striped") == 2.0 ** 47
    # contiguous ranks do r + 1/2 units: the 64K P = 4 case, rank 3 vs rank 0
    heavy = bench.ring_share_flop(65536, 32, 128, 4, "contiguous", 3)
    light = bench.ring_share_flop(65536, 32, 128, 4, "contiguous", 0)
    assert heavy / light == 7.0
    assert heavy / bench.ring_share_flop(65536, 32, 128, 4, "zigzag", 3) == 1.75


@pytest.mark.parametrize("layout", ["zigzag", "striped", "contiguous"])
@pytest.mark.parametrize("rank", [0, 3, 7])
def test_plan_flop_matches_closed_form(layout, rank):
    import context_parallelism_cp_amd as cp
    assert bench.plan_flop(cp, 131072, 32, 128, 8, layout, rank) == \
        bench.ring_share_flop(131072, 32, 128, 8, layout, rank)


def test_plan_flop_padded_length_counts_real_rows_only():
    import context_parallelism_cp_amd as cp
    full = bench.plan_flop(cp, 131072, 32, 128, 8, "zigzag", 0)
    short = bench.plan_flop(cp, 131071, 32, 128, 8, "zigzag", 0)
    assert 0.999 * full < short < full


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_recorded_traffic_follows_the_kernel_source_and_workload(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// some kernel\n")
    digest = hashlib.sha256(src.read_bytes()).hexdigest()
    key = bench.workload_key("both", "zigzag", 0, 131072, 8)
    prof = tmp_path / "traffic.md"
    prof.write_text(f"# summary\n\ntraffic_bytes_per_launch: 1234\nworkload_key: {key}\n"
                    f"kernel_source_sha256: {digest}\n")
    assert bench.recorded_traffic(str(prof), str(src), key) == 1234.0
    # another workload of the same kernel: no figure
    for other in (bench.workload_key("ring", "zigzag", 0, 131072, 8),
                  bench.workload_key("both", "striped", 0, 131072, 8),
                  bench.workload_key("both", "zigzag", 3, 131072, 8),
                  bench.workload_key("both", "zigzag", 0, 131071, 8),
                  bench.workload_key("ring", "zigzag", -1, 32768, 8), None):
        assert bench.recorded_traffic(str(prof), str(src), other) is None
    src.write_text("// the kernel changed\n")
    assert bench.recorded_traffic(str(prof), str(src), key) is None
    assert bench.recorded_traffic(str(tmp_path / "missing.md"), str(src), key) is None


def test_work_model_units_of_the_64k_comparison():
    """The per-rank sweep reports work in the handbook's units (C x C chunk
    pairs of the 2P-way split, diagonal half): contiguous [2, 6, 10, 14] and
    zigzag [8, 8, 8, 8] at P = 4, as the page's work snippet prints."""
    import context_parallelism_cp_amd as cp
    import pins
    g = pins.load_golden("work_p4.txt")
    S, P = 65536, 4
    C = S // (2 * P)
    unit = 4.0 * 128 * 32 * C * C
    for layout in ("contiguous", "zigzag"):
        got = [bench.plan_flop(cp, S, 32, 128, P, layout, r) / unit for r in range(P)]
        assert got == [float(x) for x in g[layout]]


def test_bench_argument_guards():
    for extra, msg in ((["--part", "ulysses", "--ring-p", "4"], "--ring-p"),
                       (["--part", "ranks", "--seq", "65535"], "divides"),
                       (["--part", "bwd", "--rank", "-1"], "every rank")):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *extra],
                           capture_output=True, text=True, timeout=120)
        assert r.returncode == 2 and msg in r.stderr, r.stderr


def test_exact_count_closed_forms():
    import context_parallelism_cp_amd as cp
    # contiguous P = 4 on 32 tokens, rank 3: three full 8 x 8 blocks and one
    # causal 8 x 8 diagonal block with 8 * 9 / 2 visible pairs
    assert bench.plan_flop_exact(cp, 32, 1, 1, 4, "contiguous", 3) == 4.0 * (3 * 64 + 36)
    # zigzag rank of 8 at 128K: 15 full 8192^2 chunk pairs and 2 diagonal
    # ones, exceeding the half-diagonal convention by 2 * 8192 / 2 pairs
    exact = bench.plan_flop_exact(cp, 131072, 32, 128, 8, "zigzag", 0)
    half = bench.plan_flop(cp, 131072, 32, 128, 8, "zigzag", 0)
    assert exact - half == 4.0 * 128 * 32 * 8192
    assert bench.plan_flop_exact(cp, 131072, 32, 128, 8, "striped", 0) is None
