"""Host-only checks of the measurement tools (no GPU is touched).

- bench.py refuses more than one GPU and unknown row groups before it
  starts anything;
- the rocprofv3 runs that summarize_profiles.py documents (and that make
  profiles/) stay within what one counter pass can collect on MI355X: at
  most 8 SQ, 4 TCC, 4 TCP, 2 TA, 2 TD and 2 GRBM counters per run, with
  FETCH_SIZE taking 3 TCC counters and WRITE_SIZE 2; a pass asking for more
  fails, so a documented command must never do that.
"""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1",
               CUDA_VISIBLE_DEVICES="-1")
    return subprocess.run([sys.executable, *args], cwd=ROOT, capture_output=True, text=True,
                          timeout=120, env=env)


def test_bench_refuses_more_than_one_gpu():
    r = run("bench.py", "--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_bench_refuses_unknown_row_groups():
    r = run("bench.py", "--rows", "uneven,nonsense")
    assert r.returncode == 2
    assert "unknown row groups ['nonsense']" in r.stderr


# Hardware counters each derived counter uses, by block (the rest count one
# in the block their prefix names).
DERIVED = {"FETCH_SIZE": {"TCC": 3}, "WRITE_SIZE": {"TCC": 2}}
LIMITS = {"SQ": 8, "TCC": 4, "TCP": 4, "TA": 2, "TD": 2, "GRBM": 2}


def test_documented_counter_passes_fit_one_run():
    r = run("summarize_profiles.py", "--commands", "/repo", "/out")
    assert r.returncode == 0, r.stderr
    cmds = r.stdout.strip().splitlines()
    assert len(cmds) == 8
    assert "--kernel-trace" in cmds[0] and "--pmc" not in cmds[0]
    for c in cmds[1:]:
        # one pass per run, under its own kill-timeout, nothing traced beside it
        assert c.startswith("timeout -s KILL ")
        opts = c.split(" rocprofv3 ", 1)[1].split(" -- ", 1)[0]
        assert not re.search(r"--(sys|runtime|hip|hsa|memory-copy|scratch-memory|marker)-trace|"
                             r"(^|\s)-[sr](\s|$)", opts), opts
        names = re.search(r"--pmc (.*?) --output-format", c).group(1).split()
        used = {}
        for n in names:
            for block, k in DERIVED.get(n, {n.split("_")[0]: 1}).items():
                used[block] = used.get(block, 0) + k
        for block, k in used.items():
            assert block in LIMITS, f"unexpected counter block in {names}"
            assert k <= LIMITS[block], f"{k} {block} counters in one pass: {names}"
        # the program itself follows '--', with nothing in between
        assert re.search(r" -- python3 /repo/bench\.py ", c)
