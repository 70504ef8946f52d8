"""bench.py --timeline on the GPU: the instrumented build records every block
of a compress launch, with its role, four stamps in order, and a grid laid
out as the grid planner says (direct blocks only for a launch the device
holds at once; encoder and finalize blocks otherwise), after one call or as
the last of a burst of back-to-back calls."""
import os
import sys

import pytest

from gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    require_gpu()
    sys.path.insert(0, ROOT)
    import bench as b
    return b


@pytest.mark.parametrize("wid, roles, burst", [("1", {"encoder_direct": 128}, 1),
                                               ("2", {"encoder_staged": 7168, "finalize": 448}, 1),
                                               ("2", {"encoder_staged": 7168, "finalize": 448}, 6)])
def test_timeline_records_every_block(bench, wid, roles, burst):
    from lossless_bf16_exponent_amd import workloads, zc
    print("timeline of workload %s, burst %d" % (wid, burst), flush=True)
    rec = bench.timeline(zc, workloads.get(wid), warmup=3, burst=burst)
    assert rec["burst"] == burst
    assert rec["blocks"] == sum(roles.values())
    assert {k: v["blocks"] for k, v in rec["roles"].items()} == roles
    for v in rec["roles"].values():
        assert v["lifetime_median_us"] > 0
        for key in ("stamp_0_1_median_us", "stamp_1_2_median_us", "stamp_2_3_median_us"):
            assert v[key] >= 0
    assert 0 < rec["span_us"] <= rec["event_us"]
    assert rec["tail"]["last_end_us"] == rec["span_us"]
