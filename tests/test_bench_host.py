"""CPU checks of bench.py's command line (no GPU is touched): several GPUs
are refused with a message, and the help text lists the options."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_contract_options():
    r = subprocess.run([sys.executable, BENCH, "--help"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup"):
        assert opt in r.stdout


def test_cold_set_plan_meets_its_stated_conditions():
    """The timed calls of a cold measurement read each input set once while the sets fit in DISTINCT_BYTES, else
    again only after about DISTINCT_BYTES of other sets; the warm-up set is never read by a timed call; the graphs
    hold the calls the line reports."""
    sys.path.insert(0, ROOT)
    import bench
    for per_set in (82_240 + 1024, 10_526_720 + 4096, 75_800_000, 300_000_000):
        for steps in (20, 60, 120, 600, 1200, 6000):
            calls, n, timed, warm = bench.plan_sets(per_set, steps, cold=True)
            assert calls == min(60, steps) and all(len(g) == calls for g in timed)
            order = [k for r in range(steps // calls) for k in timed[r % len(timed)]]
            assert len(order) == steps and warm not in order
            last = {}
            for i, k in enumerate(order):
                if k in last:
                    assert (i - last[k]) * per_set >= bench.DISTINCT_BYTES - per_set * calls, (per_set, steps)
                last[k] = i
            assert n * per_set <= max(bench.DISTINCT_BYTES, per_set * calls)
            if steps * per_set <= bench.DISTINCT_BYTES:
                assert len(set(order)) == steps
    calls, n, timed, warm = bench.plan_sets(10_530_816, 20, cold=False)
    assert (calls, n, warm) == (20, 1, 0) and timed == [[0] * 20]
