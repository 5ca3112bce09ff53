"""GPU parity of the power-of-two (packed UE8M0) scale variant against the CPU oracle.

The oracle needs no change: it takes the same FP32 scales, here all powers of two, and
the GPU receives them as packed E8M0 exponents.  Every instance compiled for the
variant is exercised for every layout, plus split-K, closed forms and refusals."""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import SENTINEL, check_full, oracle_full, out_shape

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


E8_CAPABLE = [i["instance"] for i in fp8bs.instances() if i["ue8m0"]]


def _run(p, workspace=None):
    dev = "cuda"
    a = torch.from_numpy(p.A).to(dev)
    sfa = fp8bs.sfa_ue8m0_mn_major(torch.from_numpy(p.SA)).to(dev)
    if p.kind == "dense":
        b = torch.from_numpy(np.ascontiguousarray(p.B[0])).to(dev)
        sfb = fp8bs.sfb_ue8m0(torch.from_numpy(np.ascontiguousarray(p.SB[0]))).to(dev)
    else:
        b = torch.from_numpy(p.B).to(dev)
        sfb = fp8bs.sfb_ue8m0(torch.from_numpy(p.SB)).to(dev)
    d = torch.full(out_shape(p), SENTINEL, dtype=torch.int16, device=dev)
    if p.kind == "dense":
        fp8bs.fp8bs_dense_nt_ue8m0(a, sfa, b, sfb, d, workspace=workspace)
    elif p.kind == "contiguous":
        fp8bs.fp8bs_grouped_contiguous_nt_ue8m0(a, sfa, b, sfb, d,
                                                torch.from_numpy(p.layout).to(dev),
                                                workspace=workspace)
    else:
        fp8bs.fp8bs_grouped_masked_nt_ue8m0(a, sfa, b, sfb, d,
                                            torch.from_numpy(p.masked_m).to(dev),
                                            expected_m=p.expected_m, workspace=workspace)
    torch.cuda.synchronize()
    return d.cpu().numpy().view(np.uint16)


def _check(p, what, workspace=None):
    _say(f"[gpu] ue8m0 {what}: {p.kind} M={p.M} N={p.N} K={p.K} G={p.G}")
    return check_full(p, _run(p, workspace), oracle_full(p), what)


@pytest.mark.parametrize("inst", E8_CAPABLE)
def test_dense_every_instance(inst):
    fp8bs.force_instance(inst)
    # K = 5 chunks: a partly used packed word (groups 4..7 hold only group 4)
    _check(synth.make_dense(300, 500, 640, seed=501 + inst, pow2=True), f"dense inst {inst}")


@pytest.mark.parametrize("inst", E8_CAPABLE)
def test_contiguous_every_instance(inst):
    bm = fp8bs.instances()[inst]["block_m"]
    if 128 % bm != 0 and bm != 256:
        pytest.skip("block_m neither divides the 128-row alignment nor spans two blocks")
    fp8bs.force_instance(inst)
    p = synth.make_contiguous(4, 300, 1152, seed=521 + inst, counts=[200, 0, 1, 129], pow2=True)
    _check(p, f"contiguous inst {inst}")


@pytest.mark.parametrize("inst", E8_CAPABLE)
def test_masked_every_instance(inst):
    fp8bs.force_instance(inst)
    p = synth.make_masked(5, 200, 300, 384, seed=541 + inst, masked_m=[0, 200, 1, 77, 129],
                          pow2=True)
    _check(p, f"masked inst {inst}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (129, 2112, 1024), (256, 7168, 512),
                                   (1000, 96, 2048)])
def test_planner_shapes(M, N, K):
    _check(synth.make_dense(M, N, K, seed=M + N + K, outlier_frac=0.01, pow2=True),
           f"dense {M}x{N}x{K}")


def test_split_k():
    fp8bs.force_splits(3)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    _check(synth.make_dense(96, 700, 1280, seed=561, pow2=True), "dense splits 3", workspace=ws)


def test_constant_inputs_bit_exact():
    M, N, K = 200, 300, 7168
    p = synth.make_dense(M, N, K, seed=0, pow2=True)
    p.A[:] = 0x38                                         # 1.0
    p.B[:] = 0x38
    p.SA[:] = 2.0 ** -3
    p.SB[:] = 2.0 ** 2
    gpu = _run(p)
    assert np.all(gpu == 0x4560)                          # 7168 * 2^-1 = 3584


def test_ladder_of_exponents_bit_exact():
    """Each K group its own exponent pair: D = sum_c 128 * 2^(ea_c + eb_c), exact."""
    M, N, K = 64, 128, 1024
    p = synth.make_dense(M, N, K, seed=1, pow2=True)
    p.A[:] = 0x38
    p.B[:] = 0x38
    kb = K // 128
    ea = np.arange(kb) - 4
    eb = np.arange(kb) // 2 - 3
    p.SA[:] = (2.0 ** ea)[None, :].astype(np.float32)
    p.SB[:] = (2.0 ** eb)[None, None, :].astype(np.float32)
    gpu = _run(p)
    assert np.array_equal(gpu, oracle_full(p))


def test_non_power_of_two_scales_are_refused_by_the_helper():
    with pytest.raises(ValueError):
        fp8bs.ue8m0_exponents(torch.tensor([0.75]))


def test_instance_without_the_variant_is_refused():
    no_e8 = [i["instance"] for i in fp8bs.instances() if i["instance"] not in E8_CAPABLE]
    fp8bs.force_instance(no_e8[0])
    p = synth.make_dense(64, 256, 256, seed=2, pow2=True)
    with pytest.raises(fp8bs.FP8BSError):
        _run(p)


def test_queries_with_the_ue8m0_flag_describe_the_launched_plan():
    """workspace_size / describe_config with LAYOUT_UE8M0 plan exactly what the _ue8m0 call
    runs: the decode shape below plans a B-streaming instance for FP32 scales (not compiled
    for UE8M0), so without the flag the sized workspace and the description would be those
    of a plan the call cannot run.  With the flag's workspace the call splits as described
    and matches the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    m, n, k = 64, 7168, 2048
    code = fp8bs.LAYOUT_DENSE | fp8bs.LAYOUT_UE8M0
    q = fp8bs.plan_query(code, m, n, k, 1, 0, cus, 1 << 40)
    assert q["ue8m0"] == 1
    desc = fp8bs.describe_config(code, m, n, k)
    assert f"instance {q['instance']}" in desc and f"splits {q['splits']}" in desc
    assert " ue8m0 " in desc
    ws_bytes = fp8bs.workspace_size(code, m, n, k)
    assert ws_bytes == q["workspace_bytes"]
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    _check(synth.make_dense(m, n, k, seed=590, pow2=True), "dense, flag-sized workspace",
           workspace=ws)
