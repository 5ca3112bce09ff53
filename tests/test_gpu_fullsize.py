"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times.  The decode-sized families -- the pages' M=128 shape, the
decode sweep and the masked MoE layout, a few to a hundred GFLOP each -- are
compared with the oracle over the whole output.  The prefill and contiguous
MoE families (up to about 2 TFLOP per shape) check every row that must stay
untouched bit-exactly, every valid output for finiteness, and 4096+ sampled
outputs against the oracle computed one by one."""
import sys

import pytest

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import DeviceProblem, check_full, check_sampled, oracle_full

pytestmark = pytest.mark.gpu

WHOLE = (0, 2, 4)
CASES = [(fam, i) for fam in range(5) for i in range(len(synth.workload_shapes(fam)))]


@pytest.mark.parametrize("fam,i", CASES, ids=[synth.workload_shapes(f)[i]["name"] for f, i in CASES])
def test_full_size(fam, i):
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    desc = synth.workload_shapes(fam)[i]
    print(f"[gpu] full size {desc['name']} ({'whole output' if fam in WHOLE else 'sampled'})",
          flush=True)
    sys.stdout.flush()
    p = synth.make(desc)
    dp = DeviceProblem(p)
    dp.reset()
    dp.run()
    gpu = dp.result()
    del dp
    if fam in WHOLE:
        check_full(p, gpu, oracle_full(p), desc["name"])
    else:
        check_sampled(p, gpu, n_points=4096, seed=fam * 100 + i, what=desc["name"])
