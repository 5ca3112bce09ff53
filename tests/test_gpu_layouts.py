"""GPU parity of the dense nn / tn / tt stored forms (MN-major operands read with LDS
transpose loads) against the oracle's stored-form product: every instance compiled for
MN-major operands, ragged tails in M and N, the FP32 addend, split-K, and refusals."""
import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import SENTINEL, check_values

pytestmark = pytest.mark.gpu

FORMS = ["nn", "tn", "tt"]
MN_INSTANCES = [i["instance"] for i in fp8bs.instances() if i["mn"]]


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


def _run(p, form, c=None, workspace=None):
    A, B = synth.stored_operands(p, form)
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(B).cuda()
    sfa = fp8bs.sfa_mn_major(torch.from_numpy(p.SA)).cuda()
    sfb = torch.from_numpy(np.ascontiguousarray(p.SB[0])).cuda()
    d = torch.full((p.M, p.N), SENTINEL, dtype=torch.int16, device="cuda")
    ct = torch.from_numpy(c).cuda() if c is not None else None
    getattr(fp8bs, "fp8bs_dense_" + form)(a, sfa, b, sfb, d, c=ct, workspace=workspace)
    torch.cuda.synchronize()
    return d.cpu().numpy().view(np.uint16)


def _check(p, form, what, c=None, workspace=None):
    print(f"[gpu] form {form} {what}: M={p.M} N={p.N} K={p.K}", flush=True)
    gpu = _run(p, form, c, workspace)
    A, B = synth.stored_operands(p, form)
    ref = oracle.dense_layout(form, A, p.SA, B, p.SB[0], c)
    return check_values(gpu, ref, f"{form} {what}")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("inst", MN_INSTANCES)
def test_every_mn_instance(form, inst):
    fp8bs.force_instance(inst)
    # M = 80, N = 208: ragged against every tile; K = 640: five chunks
    _check(synth.make_dense(80, 208, 640, seed=800 + inst), form, f"inst {inst}")


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("M,N,K", [(16, 16, 128), (256, 512, 1024), (400, 272, 384),
                                   (64, 2112, 2048)])
def test_planner_shapes(form, M, N, K):
    _check(synth.make_dense(M, N, K, seed=M + 3 * N + K, outlier_frac=0.01), form, "planner")


@pytest.mark.parametrize("form", FORMS)
def test_addend_and_split_k(form):
    p = synth.make_dense(96, 336, 1280, seed=851)
    c = (np.random.default_rng(852).standard_normal((96, 336)) * 3).astype(np.float32)
    fp8bs.force_splits(3)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    _check(p, form, "addend, 3 splits", c=c, workspace=ws)
    fp8bs.force_splits(0)
    _check(p, form, "addend", c=c)


def test_forms_agree_with_nt_bit_for_bit_on_exact_inputs():
    """Power-of-two scales and one nonzero K value per row: every output is exact, so
    all four forms must give the same bits as the NT call."""
    M, N, K = 64, 96, 512
    p = synth.make_dense(M, N, K, seed=860)
    rng = np.random.default_rng(861)
    p.A[:] = 0
    p.A[np.arange(M), rng.integers(0, K, M)] = 0x38
    p.SA[:] = 2.0 ** rng.integers(-3, 4, p.SA.shape)
    p.SB[:] = 2.0 ** rng.integers(-3, 4, p.SB.shape)
    ref = oracle.dense(p.A, p.SA, p.B[0], p.SB[0])
    for form in FORMS:
        assert np.array_equal(_run(p, form), ref), form


def test_refusals():
    a = torch.zeros((128, 40), dtype=torch.uint8, device="cuda")      # tn: a is [k][m], m = 40
    b = torch.zeros((128, 64), dtype=torch.uint8, device="cuda")
    sfa = torch.zeros(fp8bs.get_sfa_ld(40), dtype=torch.float32, device="cuda")
    sfb = torch.zeros(1, dtype=torch.float32, device="cuda")
    d = torch.zeros((40, 64), dtype=torch.int16, device="cuda")
    with pytest.raises(fp8bs.FP8BSError):                 # m not a multiple of 16
        fp8bs.fp8bs_dense_tn(a, sfa, b, sfb, d)
    bn = torch.zeros((128, 40), dtype=torch.uint8, device="cuda")   # nn: b is [k][n], n = 40
    an = torch.zeros((64, 128), dtype=torch.uint8, device="cuda")
    sfa64 = torch.zeros(fp8bs.get_sfa_ld(64), dtype=torch.float32, device="cuda")
    dn = torch.zeros((64, 40), dtype=torch.int16, device="cuda")
    with pytest.raises(fp8bs.FP8BSError):                 # n not a multiple of 16
        fp8bs.fp8bs_dense_nn(an, sfa64, bn, sfb, dn)
    no_mn = [i["instance"] for i in fp8bs.instances() if not i["mn"]]
    fp8bs.force_instance(no_mn[0])
    p = synth.make_dense(64, 128, 256, seed=3)
    with pytest.raises(fp8bs.FP8BSError):
        _run(p, "tn")
    torch.cuda.synchronize()


@pytest.mark.parametrize("desc", synth.workload_shapes(6), ids=lambda d: d["name"])
def test_full_size_stored_forms_sampled(desc):
    """The benchmark's stored-form shapes at full size in its launch configuration (the
    planner's plan with its preferred workspace): every output finite, 4100 sampled
    outputs against the oracle."""
    from _helpers import check_sampled
    p = synth.make(desc)
    form = desc["form"]
    print(f"[gpu] full size {desc['name']}", flush=True)
    code = {"nn": fp8bs.LAYOUT_DENSE_NN, "tn": fp8bs.LAYOUT_DENSE_TN,
            "tt": fp8bs.LAYOUT_DENSE_TT}[form]
    ws = torch.empty(max(fp8bs.workspace_size(code, p.M, p.N, p.K), 16), dtype=torch.uint8,
                     device="cuda")
    gpu = _run(p, form, workspace=ws)
    check_sampled(p, gpu, n_points=4096, seed=p.seed, what=desc["name"])


E8_MN_INSTANCES = [i["instance"] for i in fp8bs.instances() if i["mn"] and i["ue8m0"]]


def _run_e8(p, form, workspace=None):
    A, B = synth.stored_operands(p, form)
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(B).cuda()
    sfa = fp8bs.sfa_ue8m0_mn_major(torch.from_numpy(p.SA)).cuda()
    sfb = fp8bs.sfb_ue8m0(torch.from_numpy(np.ascontiguousarray(p.SB[0]))).cuda()
    d = torch.full((p.M, p.N), SENTINEL, dtype=torch.int16, device="cuda")
    getattr(fp8bs, f"fp8bs_dense_{form}_ue8m0")(a, sfa, b, sfb, d, workspace=workspace)
    torch.cuda.synchronize()
    return d.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("form", FORMS)
@pytest.mark.parametrize("inst", E8_MN_INSTANCES)
def test_ue8m0_every_instance(form, inst):
    """Power-of-two scales as packed E8M0 exponents with MN-major operands."""
    fp8bs.force_instance(inst)
    p = synth.make_dense(80, 208, 640, seed=870 + inst, pow2=True)
    print(f"[gpu] form {form} ue8m0 inst {inst}", flush=True)
    A, B = synth.stored_operands(p, form)
    check_values(_run_e8(p, form), oracle.dense_layout(form, A, p.SA, B, p.SB[0]),
                 f"{form} ue8m0 inst {inst}")


@pytest.mark.parametrize("form", FORMS)
def test_ue8m0_planner_and_split_k(form):
    p = synth.make_dense(256, 400, 1536, seed=880, pow2=True)
    A, B = synth.stored_operands(p, form)
    ref = oracle.dense_layout(form, A, p.SA, B, p.SB[0])
    check_values(_run_e8(p, form), ref, f"{form} ue8m0 planner")
    fp8bs.force_splits(3)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    check_values(_run_e8(p, form, workspace=ws), ref, f"{form} ue8m0 3 splits")
