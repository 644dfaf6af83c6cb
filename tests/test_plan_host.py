"""The small-batch FFN launch plan on the host (tests/native/plan_check.cc):
every plan over a sweep of shapes fits the split-K join area, the workload
shapes plan as designed, and plans past the area are refused.  The C ABI runs
the same plan before it enqueues anything (moe_forward returns
MOE_E_UNSUPPORTED for a plan that does not fit), so no over-capacity launch
ever reaches the GPU."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))


def test_split_plan_fits_join_area(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-O2", "-std=c++17", "-Wall", "-Wextra", "-o", exe,
                    os.path.join(HERE, "native", "plan_check.cc")], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    for line in r.stdout.splitlines():
        assert line.split(":")[1].strip().startswith("0 "), line
