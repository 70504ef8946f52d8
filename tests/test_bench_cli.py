"""bench.py's command line on the CPU: runs on several GPUs are refused with a
message (the codec is measured on one GPU), the defaults finish within the
time a round allows, and every committed counter summary names a call and
carries the source hash bench.py compares before it reports traffic."""
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + args, capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_several_gpus_are_refused():
    r = run_bench(["--gpus", "2"])
    assert r.returncode == 2 and "one GPU" in r.stderr
    r = run_bench([], {"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_defaults():
    r = run_bench(["--help"])
    assert r.returncode == 0
    text = " ".join(r.stdout.split())
    assert "default 100" in text  # warm-up steps
    sys.path.insert(0, ROOT)
    import bench
    assert bench.REDUCE_WARMUP_CALLS >= 250


def test_counter_summaries_are_well_formed():
    sys.path.insert(0, ROOT)
    import bench
    prof = os.path.join(ROOT, "profiles")
    names = [f for f in os.listdir(prof) if f.startswith("traffic_")]
    assert names
    for f in names:
        text = open(os.path.join(prof, f)).read()
        fields = dict(re.findall(r"^(\w+) = (\S+)$", text, re.M))
        assert {"kernel_sha", "call", "workload", "fetch_bytes", "write_bytes"} <= set(fields), f
        assert re.fullmatch(r"[0-9a-f]{16}", fields["kernel_sha"]), f
        assert "# command" in text or "# commands" in text, f  # the command that made it
        call = fields["call"]
        if call in bench.CALL_SOURCES:  # the summaries bench.py reads
            assert int(fields["fetch_bytes"]) > 0 and int(fields["write_bytes"]) > 0, f
