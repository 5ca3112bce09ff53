"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: every row that must stay untouched is checked bit-exactly,
every valid output for finiteness, and 4096+ sampled outputs per shape against
the oracle computed one by one."""
import sys

import pytest

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import DeviceProblem, check_sampled

pytestmark = pytest.mark.gpu

CASES = [(fam, i) for fam in range(5) for i in range(len(synth.workload_shapes(fam)))]


@pytest.mark.parametrize("fam,i", CASES, ids=[synth.workload_shapes(f)[i]["name"] for f, i in CASES])
def test_full_size_sampled(fam, i):
    fp8bs.force_instance(-1)
    desc = synth.workload_shapes(fam)[i]
    print(f"[gpu] full size {desc['name']}", flush=True)
    sys.stdout.flush()
    p = synth.make(desc)
    dp = DeviceProblem(p)
    dp.run()
    gpu = dp.result()
    del dp
    check_sampled(p, gpu, n_points=4096, seed=fam * 100 + i, what=desc["name"])
