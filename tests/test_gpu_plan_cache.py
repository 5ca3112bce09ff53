"""The per-thread plan cache of the C ABI: a repeated request reuses its plan, and every
input of the planner -- shape, layout, workspace, the CU cap and the test pins -- keys
it, so that a changed input is never answered with a stale plan."""
import re

import pytest

import moe_grouped_gemm_block_amd as fp8bs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _reset():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    fp8bs.set_num_cus(0)


def _inst(text):
    return int(re.search(r"instance (\d+)", text).group(1))


def _splits(text):
    return int(re.search(r"splits (\d+)", text).group(1))


def test_forced_instance_and_splits_reach_the_plan_through_the_cache():
    shapes = [(64, 7168, 7168), (4096, 7168, 2048), (128, 2112, 7168), (256, 4096, 512)]
    planned = {s: _inst(fp8bs.describe_config(fp8bs.LAYOUT_DENSE, *s)) for s in shapes}
    n_inst = fp8bs.instances()
    staged = [i["instance"] for i in n_inst if i["kind"] == 0][:6]
    # more distinct requests than the cache holds, interleaved, each asked twice
    for rnd in range(2):
        for inst in staged:
            fp8bs.force_instance(inst)
            for s in shapes:
                assert _inst(fp8bs.describe_config(fp8bs.LAYOUT_DENSE, *s)) == inst, (inst, s)
        fp8bs.force_instance(-1)
        for s in shapes:
            assert _inst(fp8bs.describe_config(fp8bs.LAYOUT_DENSE, *s)) == planned[s]
    q0 = fp8bs.plan_query(fp8bs.LAYOUT_DENSE, 64, 7168, 7168)
    fp8bs.force_splits(3)
    assert _splits(fp8bs.describe_config(fp8bs.LAYOUT_DENSE, 64, 7168, 7168)) == 3
    fp8bs.force_splits(0)
    assert fp8bs.plan_query(fp8bs.LAYOUT_DENSE, 64, 7168, 7168) == q0


def test_cu_cap_reaches_the_plan_through_the_cache():
    full = fp8bs.describe_config(fp8bs.LAYOUT_DENSE, 4096, 4096, 7168)
    fp8bs.set_num_cus(64)
    capped = fp8bs.describe_config(fp8bs.LAYOUT_DENSE, 4096, 4096, 7168)
    assert "cus=64" in capped and "cus=64" not in full
    fp8bs.set_num_cus(0)
    assert fp8bs.describe_config(fp8bs.LAYOUT_DENSE, 4096, 4096, 7168) == full
