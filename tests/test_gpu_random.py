"""Seeded random parity cases: entry point (workspace or not, FP32 addend, packed UE8M0
scales, the nn / tn / tt stored forms), layout, sizes (ragged and odd, down to one row or
column), instance (forced or the planner's) and K split drawn at random, each checked
against the oracle over the whole output (valid rows to tolerance, the rest untouched);
and the same for the K-grouped weight-gradient call (group sizes with empty groups, FP32
addend in place or apart, UE8M0 scales, split K).  Every case is fixed by the seed, so a
failure names a reproducible case."""
import os

import numpy as np
import pytest
import torch

import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import DeviceProblem, check_full, oracle_full
import test_gpu_addend as addend_t
import test_gpu_kgrouped as kg_t
import test_gpu_layouts as layouts_t
import test_gpu_ue8m0 as ue8m0_t

pytestmark = pytest.mark.gpu

# FP8BS_RANDOM_SEED / FP8BS_RANDOM_CASES draw another (or a longer) series of cases
SEED = int(os.environ.get("FP8BS_RANDOM_SEED", "20261203"))
N_CASES = int(os.environ.get("FP8BS_RANDOM_CASES", "160"))
INSTANCES = fp8bs.instances()
VARIANTS = ["ws", "ws", "nows", "addend", "ue8m0", "form"]


@pytest.fixture(autouse=True)
def _planner_choice():
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)
    yield
    fp8bs.force_instance(-1)
    fp8bs.force_splits(0)


def _case(i):
    rng = np.random.default_rng(SEED + i)
    variant = str(rng.choice(VARIANTS))
    kind = "dense" if variant == "form" else str(rng.choice(["dense", "dense", "contiguous",
                                                            "masked"]))
    form = str(rng.choice(["nn", "tn", "tt"])) if variant == "form" else "nt"
    pow2 = variant == "ue8m0"
    K = 128 * int(rng.integers(1, 9))
    N = int(rng.choice([rng.integers(1, 48), rng.integers(48, 700)]))
    if form in ("nn", "tn"):
        N = 16 * max(1, -(-N // 16))
    if kind == "dense":
        M = int(rng.choice([rng.integers(1, 40), rng.integers(40, 600)]))
        if form in ("tn", "tt"):
            M = 16 * max(1, -(-M // 16))
        p = synth.make_dense(M, N, K, seed=SEED + i, pow2=pow2)
    elif kind == "contiguous":
        G = int(rng.integers(1, 6))
        counts = [int(c) if rng.random() > 0.2 else 0 for c in rng.integers(1, 300, size=G)]
        p = synth.make_contiguous(G, N, K, seed=SEED + i, counts=counts, pow2=pow2)
    else:
        G = int(rng.integers(1, 6))
        max_m = int(rng.integers(1, 300))
        masked_m = rng.integers(-2, max_m + 3, size=G)
        p = synth.make_masked(G, max_m, N, K, seed=SEED + i, masked_m=masked_m,
                              expected_m=int(rng.integers(1, max_m + 1)), pow2=pow2)
    ok = [x["instance"] for x in INSTANCES
          if (kind != "contiguous" or 128 % x["block_m"] == 0 or x["block_m"] == 256)
          and (variant != "ue8m0" or x["ue8m0"]) and (variant != "form" or x["mn"])]
    inst = int(rng.choice(ok)) if rng.random() < 0.7 else -1
    two_pass = (kind == "contiguous" and inst >= 0 and INSTANCES[inst]["block_m"] == 256)
    splits = 1 if two_pass else int(rng.choice([0, 1, 2, 3, 5]))
    splits = min(splits, K // 128)
    return p, inst, splits, variant, form


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_case(i):
    p, inst, splits, variant, form = _case(i)
    what = (f"case {i}: {variant} {form} {p.kind} M={p.M} N={p.N} K={p.K} G={p.G} "
            f"inst={inst} splits={splits}")
    print(f"[gpu] {what}", flush=True)
    if variant == "addend":                         # sets the pins and checks by itself
        addend_t._run(p, splits, inst)
        return
    fp8bs.force_instance(inst)
    fp8bs.force_splits(splits)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    if variant == "ue8m0":
        ue8m0_t._check(p, what, workspace=ws)
    elif variant == "form":
        layouts_t._check(p, form, what, workspace=ws)
    else:
        dp = DeviceProblem(p)
        dp.run(workspace=variant == "ws")
        check_full(p, dp.result(), oracle_full(p), what)


N_KG_CASES = int(os.environ.get("FP8BS_RANDOM_KG_CASES", "40"))


def _kg_case(i):
    rng = np.random.default_rng(SEED + 1000 + i)
    variant = str(rng.choice(["plain", "addend", "in_place", "ue8m0", "split"]))
    G = int(rng.integers(1, 9))
    M = 16 * int(rng.integers(1, 25))
    N = 16 * int(rng.integers(1, 25))
    counts = [int(c) if rng.random() > 0.25 else 0 for c in rng.integers(1, 700, size=G)]
    p = synth.make_k_grouped(G, M, N, seed=SEED + 1000 + i, counts=counts,
                             pow2=variant == "ue8m0")
    pool = kg_t.E8_MN_INSTANCES if variant == "ue8m0" else kg_t.MN_INSTANCES
    inst = int(rng.choice(pool)) if rng.random() < 0.7 else -1
    splits = int(rng.choice([2, 3, 5])) if variant == "split" else 0
    if splits:                                  # a pinned count the call can use
        splits = max(1, min(splits, int(sum(p.ks)) // 128))
    C = None
    if variant in ("addend", "in_place") or rng.random() < 0.3:
        C = (rng.standard_normal((G, M, N)) * 4).astype(np.float32)
    return p, variant, inst, splits, C


@pytest.mark.parametrize("i", range(N_KG_CASES))
def test_random_k_grouped_case(i):
    p, variant, inst, splits, C = _kg_case(i)
    what = (f"k-grouped case {i}: {variant} G={p.G} M={p.M} N={p.N} ks={list(p.ks)} "
            f"inst={inst} splits={splits} addend={C is not None}")
    print(f"[gpu] {what}", flush=True)
    fp8bs.force_instance(inst)
    fp8bs.force_splits(splits)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    if variant == "ue8m0":
        kg_t._full_e8(p, what, C=C, workspace=ws)
    else:
        kg_t._full(p, what, C=C, workspace=ws, in_place=variant == "in_place")
