"""GPU parity of D = C + A B^T (FP32 addend) against the oracle, every layout, with and
without split-K, including ragged tails and rows that must stay untouched."""
import sys

import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import SENTINEL, DeviceProblem, check_full, out_shape

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


def _run(p, splits=0, inst=-1):
    print(f"[gpu] addend {p.kind} M={p.M} N={p.N} K={p.K} splits={splits} inst={inst}", flush=True)
    fp8bs.force_splits(splits)
    fp8bs.force_instance(inst)
    dp = DeviceProblem(p)
    rng = np.random.default_rng(p.seed + 7)
    C = (rng.standard_normal(out_shape(p)) * 4).astype(np.float32)
    c = torch.from_numpy(C).cuda()
    if p.kind == "dense":
        fp8bs.fp8bs_dense_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d)
    elif p.kind == "contiguous":
        fp8bs.fp8bs_grouped_contiguous_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d, dp.layout)
    else:
        fp8bs.fp8bs_grouped_masked_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d, dp.masked_m,
                                        expected_m=p.expected_m)
    gpu = dp.result()
    ref = np.full(out_shape(p), SENTINEL, np.uint16)
    if p.kind == "dense":
        oracle.with_addend("dense", p.A, p.SA, p.B[0], p.SB[0], C, ref)
    elif p.kind == "contiguous":
        oracle.with_addend("contiguous", p.A, p.SA, p.B, p.SB, C, ref, p.layout)
    else:
        oracle.with_addend("masked", p.A, p.SA, p.B, p.SB, C, ref, p.masked_m)
    check_full(p, gpu, ref, f"addend {p.kind}")


@pytest.mark.parametrize("splits", [0, 3])
def test_dense(splits):
    _run(synth.make_dense(300, 502, 640, seed=701), splits)


@pytest.mark.parametrize("inst", [0, 2, 7, 17, 18])
def test_dense_instances(inst):
    _run(synth.make_dense(200, 300, 512, seed=702 + inst), 0, inst)


def test_decode_planner_split():
    _run(synth.make_dense(64, 2048, 7168, seed=703))


@pytest.mark.parametrize("splits", [0, 2])
def test_contiguous(splits):
    _run(synth.make_contiguous(4, 300, 384, seed=704, counts=[200, 0, 1, 129]), splits)


@pytest.mark.parametrize("splits", [0, 4])
def test_masked(splits):
    _run(synth.make_masked(5, 200, 300, 768, seed=705, masked_m=[0, 200, 1, 77, 129]), splits)


def test_misaligned_addend_is_refused():
    p = synth.make_dense(64, 256, 256, seed=706)
    dp = DeviceProblem(p)
    c = torch.zeros(64 * 256 + 1, dtype=torch.float32, device="cuda")[1:].view(64, 256)
    with pytest.raises(fp8bs.FP8BSError):
        fp8bs.fp8bs_dense_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d)
