"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small shapes are compared whole (several tiles and ragged tails in M and N);
every compiled kernel instance is exercised for every layout it supports.
Rows that must not be written are checked bit-exactly against the sentinel.
"""
import sys

import numpy as np
import pytest
import torch

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import (SENTINEL, DeviceProblem, check_full, check_values, oracle_full,
                      bf16_bits_to_f64, out_shape)

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


def _run_and_check(p, what, workspace=True):
    _say(f"[gpu] {what}: {p.kind} M={p.M} N={p.N} K={p.K} G={p.G} workspace={workspace}")
    dp = DeviceProblem(p)
    dp.run(workspace=workspace)
    gpu = dp.result()
    ref = oracle_full(p)
    return check_full(p, gpu, ref, what)


def _instances(layout):
    out = []
    for inst in fp8bs.instances():
        # contiguous: a tile inside one 128-row expert block, or two blocks (two passes)
        if layout == fp8bs.LAYOUT_CONTIGUOUS and 128 % inst["block_m"] != 0 and \
                inst["block_m"] != 256:
            continue
        out.append(inst["instance"])
    return out


N_INST = len(fp8bs.instances())


@pytest.mark.parametrize("inst", range(N_INST))
def test_dense_every_instance(inst):
    fp8bs.force_instance(inst)
    p = synth.make_dense(300, 500, 512, seed=11 + inst)
    _run_and_check(p, f"dense inst {inst}", workspace=False)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (5, 2112, 256), (129, 129, 128), (64, 7168, 384),
                                   (256, 7168, 256), (1000, 96, 1280), (33, 4096, 128)])
def test_dense_planner_shapes(M, N, K):
    p = synth.make_dense(M, N, K, seed=M * 7 + N + K, outlier_frac=0.01)
    _run_and_check(p, f"dense {M}x{N}x{K}")


@pytest.mark.parametrize("inst", range(N_INST))
def test_contiguous_every_instance(inst):
    if inst not in _instances(fp8bs.LAYOUT_CONTIGUOUS):
        pytest.skip("block_m neither divides the 128-row alignment nor spans two blocks")
    fp8bs.force_instance(inst)
    p = synth.make_contiguous(4, 300, 384, seed=31 + inst, counts=[200, 0, 1, 129])
    _run_and_check(p, f"contiguous inst {inst}", workspace=False)


def test_contiguous_planner_multinomial():
    p = synth.make_contiguous(8, 520, 256, seed=41, total_rows=1500)
    _run_and_check(p, "contiguous multinomial")


_TWO_PASS = [i["instance"] for i in fp8bs.instances() if i["block_m"] == 256]


@pytest.mark.parametrize("inst", _TWO_PASS)
@pytest.mark.parametrize("experts", [40, 200])
def test_contiguous_many_two_expert_tiles(inst, experts):
    """256-row tiles over many experts whose segments start at odd 128-row blocks, so that
    many m-blocks hold two experts: with 40 experts 14 do, within the schedule's dense list
    of two-expert m-blocks (at most 64); with 200 experts 75 do, past it (the sparse,
    pass-major order); empty experts and one-row segments included."""
    rng = np.random.default_rng(7000 + experts)
    sizes = [0, 1, 100, 128, 129, 300] if experts == 40 else [0, 1, 100, 129, 300]
    counts = [int(c) for c in rng.choice(sizes, size=experts)]
    counts[experts // 2] = 128 * 3 + 5
    fp8bs.force_instance(inst)
    p = synth.make_contiguous(experts, 136, 256, seed=7100 + experts, counts=counts)
    _run_and_check(p, f"contiguous {experts} experts inst {inst}", workspace=False)


@pytest.mark.parametrize("inst", range(N_INST))
def test_masked_every_instance(inst):
    fp8bs.force_instance(inst)
    p = synth.make_masked(5, 200, 300, 384, seed=51 + inst, masked_m=[0, 200, 1, 77, 129])
    _run_and_check(p, f"masked inst {inst}", workspace=False)


def test_masked_clamps_out_of_range_counts():
    p = synth.make_masked(4, 64, 200, 256, seed=61, masked_m=[-5, 1000, 64, 3])
    _run_and_check(p, "masked clamp")


def test_masked_planner_expected_m():
    p = synth.make_masked(16, 256, 384, 512, seed=62, expected_m=128)
    _run_and_check(p, "masked expected_m")


# ---- split-K (workspace entry points) --------------------------------------------

@pytest.mark.parametrize("inst", range(N_INST))
@pytest.mark.parametrize("splits", [2, 3])
def test_dense_split_k_every_instance(inst, splits):
    """K = 5 chunks: 2 splits give 2 + 3 chunks, 3 splits 1 + 2 + 2."""
    fp8bs.force_instance(inst)
    fp8bs.force_splits(splits)
    p = synth.make_dense(200, 300, 640, seed=81 + inst)
    _run_and_check(p, f"dense inst {inst} splits {splits}")


@pytest.mark.parametrize("inst", range(N_INST))
def test_contiguous_split_k_every_instance(inst):
    if inst not in _instances(fp8bs.LAYOUT_CONTIGUOUS):
        pytest.skip("block_m neither divides the 128-row alignment nor spans two blocks")
    fp8bs.force_instance(inst)
    fp8bs.force_splits(3)
    p = synth.make_contiguous(4, 300, 768, seed=91 + inst, counts=[200, 0, 1, 129])
    if fp8bs.instances()[inst]["block_m"] > 128:
        # two-pass tiles (two expert blocks per tile) are never split: the pin is refused
        with pytest.raises(fp8bs.FP8BSError):
            _run_and_check(p, f"contiguous inst {inst} splits 3")
        return
    _run_and_check(p, f"contiguous inst {inst} splits 3")


@pytest.mark.parametrize("inst", range(N_INST))
def test_masked_split_k_every_instance(inst):
    fp8bs.force_instance(inst)
    fp8bs.force_splits(4)
    p = synth.make_masked(5, 200, 300, 768, seed=101 + inst, masked_m=[0, 200, 1, 77, 129])
    _run_and_check(p, f"masked inst {inst} splits 4")


def test_split_k_one_chunk_per_unit():
    fp8bs.force_splits(8)
    p = synth.make_dense(70, 1000, 1024, seed=111)
    _run_and_check(p, "dense splits 8 of 8 chunks")


def test_split_k_more_splits_than_chunks_is_refused():
    fp8bs.force_splits(3)
    p = synth.make_dense(64, 256, 256, seed=112)
    dp = DeviceProblem(p)
    with pytest.raises(fp8bs.FP8BSError):
        dp.run()


def test_split_k_planner_decode_shape():
    """The planner's own choice for a decode-sized dense GEMM (it splits K when that
    fills the machine) against the oracle."""
    p = synth.make_dense(64, 2048, 7168, seed=113)
    _say(fp8bs.describe_config(fp8bs.LAYOUT_DENSE, 64, 2048, 7168))
    _run_and_check(p, "dense decode planner")


def test_split_k_deterministic_and_close_to_unsplit():
    p = synth.make_dense(96, 700, 2048, seed=114)
    ref = oracle_full(p)
    dp = DeviceProblem(p)
    fp8bs.force_splits(5)
    dp.run()
    d0 = dp.result()
    check_full(p, d0, ref, "splits 5")
    dp.reset()
    dp.run()
    assert np.array_equal(dp.result(), d0), "split-K results differ between runs"
    dp.reset()
    dp.run(workspace=False)
    d1 = dp.result()
    check_full(p, d1, ref, "no split")
    # the two association orders agree with each other to the same bar
    check_values(d0, d1, "splits 5 against no split")


def test_split_k_reuses_a_caller_workspace():
    p = synth.make_dense(64, 512, 1024, seed=115)
    dp = DeviceProblem(p)
    fp8bs.force_splits(4)
    ws = torch.full((64 * 1024 * 1024,), 0xFF, dtype=torch.uint8, device="cuda")   # NaN bytes
    for _ in range(2):
        dp.reset()
        fp8bs.fp8bs_dense_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d, workspace=ws)
        check_full(p, dp.result(), oracle_full(p), "caller workspace")


def test_split_k_workspace_shared_by_calls_of_other_shapes():
    """Split calls of different tile counts and split counts in turn on one workspace
    that starts as garbage: each call's per-tile arrival words overlap what the others
    left there (partials or words), and every result still matches the oracle."""
    ws = torch.randint(0, 256, (64 * 1024 * 1024,), dtype=torch.uint8, device="cuda")
    cases = [(128, 2112, 7168, 7), (64, 512, 1024, 4), (200, 300, 640, 5), (128, 2112, 7168, 7)]
    for n, (m, nn, k, splits) in enumerate(cases):
        _say(f"shared workspace call {n}: {m}x{nn}x{k} splits {splits}")
        p = synth.make_dense(m, nn, k, seed=117 + n)
        dp = DeviceProblem(p)
        fp8bs.force_splits(splits)
        fp8bs.fp8bs_dense_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d, workspace=ws)
        check_full(p, dp.result(), oracle_full(p), f"shared workspace call {n}")


@pytest.mark.parametrize("splits", [2, 3, 5, 7])
def test_pinned_split_runs_in_the_workspace_it_was_sized_for(splits):
    """With only the split count pinned, fp8bs_workspace_size and the call must agree on
    the plan: a workspace of exactly the reported size is accepted."""
    for n, (m, nn, k) in enumerate([(20, 30, 896), (128, 2112, 7168), (64, 4096, 1024),
                                    (256, 700, 2048)]):
        fp8bs.force_splits(splits)
        wsz = fp8bs.workspace_size(fp8bs.LAYOUT_DENSE, m, nn, k)
        _say(f"pinned splits {splits}: {m}x{nn}x{k} workspace {wsz}")
        p = synth.make_dense(m, nn, k, seed=130 + 10 * splits + n)
        dp = DeviceProblem(p)
        ws = torch.empty(max(wsz, 16), dtype=torch.uint8, device="cuda")
        fp8bs.fp8bs_dense_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d, workspace=ws)
        check_full(p, dp.result(), oracle_full(p), f"pinned splits {splits} {m}x{nn}x{k}")


def test_split_k_short_workspace_is_refused_when_pinned():
    p = synth.make_dense(64, 512, 1024, seed=116)
    dp = DeviceProblem(p)
    fp8bs.force_splits(4)
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    with pytest.raises(fp8bs.FP8BSError):
        fp8bs.fp8bs_dense_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d, workspace=ws)
    fp8bs.force_splits(0)                              # planner: falls back to what fits
    fp8bs.fp8bs_dense_nt_ws(dp.a, dp.sfa, dp.b, dp.sfb, dp.d, workspace=ws)
    check_full(p, dp.result(), oracle_full(p), "short workspace")


# ---- closed forms, bit-exact on the GPU too ------------------------------------

def test_constant_inputs_bit_exact():
    M, N, K = 200, 300, 7168
    p = synth.make_dense(M, N, K, seed=0)
    p.A[:] = 0x38                                     # 1.0
    p.B[:] = 0x38
    p.SA[:] = 1.0
    p.SB[:] = 1.0
    dp = DeviceProblem(p)
    dp.run()
    gpu = dp.result()
    assert np.all(gpu == 0x45E0)                      # 7168


def test_one_hot_rows_bit_exact():
    rng = np.random.default_rng(3)
    M, N, K = 40, 300, 1024
    p = synth.make_dense(M, N, K, seed=3)
    pi = rng.choice(K, size=M, replace=False)
    p.A[:] = 0
    p.A[np.arange(M), pi] = 0x38
    p.SA[:] = (2.0 ** rng.integers(-3, 4, size=p.SA.shape)).astype(np.float32)
    p.SB[:] = (2.0 ** rng.integers(-3, 4, size=p.SB.shape)).astype(np.float32)
    dp = DeviceProblem(p)
    dp.run()
    assert np.array_equal(dp.result(), oracle_full(p))


def test_scale_shift_invariance_bit_exact():
    """Doubling every byte value of one 1x128 group and halving its scale leaves D
    unchanged bit for bit (FP32 MFMA sums of FP8 products scale exactly)."""
    p = synth.make_dense(130, 260, 512, seed=5)
    rng = np.random.default_rng(5)
    grp = rng.integers(0, 0x70, size=128, dtype=np.uint8) | (rng.integers(0, 2, 128, dtype=np.uint8) << 7)
    p.A[7, 256:384] = grp                             # exponent field <= 13: doubling stays exact
    dp = DeviceProblem(p)
    dp.run()
    d0 = dp.result()
    v = torch.from_numpy(grp.copy()).view(torch.float8_e4m3fn).to(torch.float32)
    dbl = (v * 2).to(torch.float8_e4m3fn)
    assert torch.equal(dbl.to(torch.float32), v * 2)
    p.A[7, 256:384] = dbl.view(torch.uint8).numpy()
    p.SA[7, 2] /= 2
    dp2 = DeviceProblem(p)
    dp2.run()
    assert np.array_equal(dp2.result(), d0)


def test_constant_inputs_bit_exact_split_k():
    M, N, K = 64, 300, 7168
    p = synth.make_dense(M, N, K, seed=0)
    p.A[:] = 0x38
    p.B[:] = 0x38
    p.SA[:] = 1.0
    p.SB[:] = 1.0
    fp8bs.force_splits(7)
    dp = DeviceProblem(p)
    dp.run()
    assert np.all(dp.result() == 0x45E0)


def test_run_to_run_determinism():
    p = synth.make_dense(512, 1000, 1024, seed=6)
    dp = DeviceProblem(p)
    dp.run()
    d0 = dp.result()
    dp.reset()
    dp.run()
    assert np.array_equal(dp.result(), d0)


def test_poisoned_padding_and_masked_rows_stay_out():
    pc = synth.make_contiguous(3, 200, 256, seed=71, counts=[100, 30, 129])
    pad = pc.layout < 0
    pc.A[pad] = 0x7F                                  # e4m3 NaN
    pc.SA[pad] = np.nan
    dp = DeviceProblem(pc)
    dp.run()
    check_full(pc, dp.result(), oracle_full(pc), "poisoned contiguous")
    pm = synth.make_masked(3, 96, 200, 256, seed=72, masked_m=[5, 96, 40])
    for g, v in enumerate(pm.masked_m):
        pm.A[g, v:] = 0x7F
        pm.SA[g, v:] = np.nan
    dp = DeviceProblem(pm)
    dp.run()
    check_full(pm, dp.result(), oracle_full(pm), "poisoned masked")


def test_stream_argument_is_honoured():
    p = synth.make_dense(64, 256, 256, seed=8)
    dp = DeviceProblem(p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        dp.run(stream=s)
    s.synchronize()
    check_full(p, dp.d.cpu().numpy().view(np.uint16), oracle_full(p), "side stream")


def test_zero_rows_is_a_no_op():
    buf = torch.zeros(64, dtype=torch.float32, device="cuda")
    ptr = buf.data_ptr()
    # m == 0: nothing to do and nothing launched; the pointers are never dereferenced
    assert fp8bs._load().fp8bs_dense_nt(ptr, ptr, ptr, ptr, ptr, 0, 16, 128, None) == 0
    assert fp8bs._load().fp8bs_grouped_masked_nt(ptr, ptr, ptr, ptr, ptr, ptr, 2, 0, 0, 16, 128,
                                                 None) == 0
    torch.cuda.synchronize()


def test_empty_torch_tensors_are_a_no_op():
    """No output rows through the binding: zero-row tensors have NULL data pointers, and
    every entry point takes the call as done (nothing launched, nothing written)."""
    cases = [synth.make_dense(0, 64, 256, seed=11),
             synth.make_contiguous(2, 64, 256, seed=12, counts=[0, 0]),
             synth.make_masked(2, 0, 64, 256, seed=13, masked_m=[0, 0])]
    for p in cases:
        print(f"[gpu] empty {p.kind} M={p.M}", flush=True)
        dp = DeviceProblem(p)
        dp.run(workspace=True)
        dp.run(workspace=False)
        c = torch.zeros(out_shape(p), dtype=torch.float32, device="cuda")
        if p.kind == "dense":
            fp8bs.fp8bs_dense_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d)
        elif p.kind == "contiguous":
            fp8bs.fp8bs_grouped_contiguous_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d, dp.layout)
        else:
            fp8bs.fp8bs_grouped_masked_nt_c(dp.a, dp.sfa, dp.b, dp.sfb, c, dp.d, dp.masked_m)
        torch.cuda.synchronize()
        assert dp.d.numel() == 0 or bool((dp.d == SENTINEL).all())
