"""Seeded synthetic inputs for the block-scaled FP8 GEMM.

This module only *draws and prepares inputs*; it holds none of the GEMM's
arithmetic.  Its outputs feed both the HIP path and the CPU oracle, so that
the two sides see byte-identical operands.

Recipe (shapes and value distributions follow the DeepSeek-V3/R1 inference
shapes that the DeepGEMM README repost, lqnn.cn/news/60274, section "性能",
says were measured; the numbers themselves stand in for those workloads):

* PRNG: numpy ``PCG64`` seeded with ``seed``; FP32 standard normals.
* Outlier tokens (decode sweep): ``max(1, round(0.01 * M))`` rows, drawn
  without replacement, are multiplied by 100 before quantisation.
* Quantisation, following the fine-grained recipe ("细粒度量化", "在线量化"
  in "deepseek开源周第三天：DeepGEMM深度分析", pxiaoer.blog): A gets one FP32 scale
  per (row, 128-column group), B one per 128x128 block (the last block of an
  N that is not a multiple of 128 covers only its existing rows).
  ``scale = max(amax, 1e-4) / 448`` in FP32 (the 1e-4 floor is not on the pages;
  it keeps the scale of an all-zero group finite), then
  ``q = e4m3(clamp(x * (448 / max(amax, 1e-4)), -448, 448))`` (each step rounded to
  FP32: the inverse once per group, the product per element) using torch's round-to-nearest-even
  cast to ``float8_e4m3fn`` (OCP e4m3).  The clamp is needed because torch maps
  values beyond the e4m3 range to NaN instead of saturating.
* Contiguous MoE layout: ``counts ~ Multinomial(total, [1/G] * G)``; expert g's
  segment holds ``counts[g]`` rows with group index g followed by padding rows
  (index -1) up to the next multiple of 128 ("Dense và Grouped GEMM" section
  of "DeepGEMM: kernel FP8 GEMM sạch và hiệu quả nhờ scaling chi tiết",
  vi.news.hada.io: each expert segment aligned to the M block size).
* Masked MoE layout: ``masked_m[g] ~ Uniform{1..max_m}``.
* K-grouped (weight-gradient) layout: ``counts ~ Multinomial(total, [1/G] * G)``
  tokens per expert, each group's K range rounded up to a multiple of 128 with
  zero padding tokens; both operands are stored token-major ([K][M], [K][N]) and
  quantised with one scale per feature and 128-token chunk.
* Seeds: shape j of workload family i uses ``seed = 1000 * i + j``.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import numpy as np
import torch

E4M3_MAX = 448.0
SCALE_FLOOR = 1e-4
MK_ALIGNMENT = 128


@dataclasses.dataclass
class Problem:
    """One GEMM problem in logical layouts (host numpy arrays).

    kind:    "dense" | "contiguous" | "masked"
    A:       uint8 [M][K] (dense/contiguous) or [G][max_m][K] (masked)
    SA:      float32, same leading dims as A, last dim K/128
    B:       uint8 [G][N][K] (G = 1 for dense)
    SB:      float32 [G][ceil(N/128)][K/128]
    layout:  int32 [M] group index per row (contiguous only), -1 = padding
    masked_m: int32 [G] valid rows per expert (masked only)
    """
    kind: str
    M: int
    N: int
    K: int
    G: int
    A: np.ndarray
    SA: np.ndarray
    B: np.ndarray
    SB: np.ndarray
    layout: Optional[np.ndarray] = None
    masked_m: Optional[np.ndarray] = None
    max_m: int = 0
    expected_m: int = 0
    seed: int = 0
    name: str = ""

    @property
    def valid_rows(self) -> int:
        if self.kind == "dense":
            return self.M
        if self.kind == "contiguous":
            lay = self.layout
            return int(((lay >= 0) & (lay < self.G)).sum())
        return int(np.clip(self.masked_m, 0, self.max_m).sum())

    @property
    def active_groups(self) -> int:
        if self.kind == "dense":
            return 1
        if self.kind == "contiguous":
            lay = self.layout
            return int(np.unique(lay[(lay >= 0) & (lay < self.G)]).size)
        return int((np.clip(self.masked_m, 0, self.max_m) > 0).sum())

    def flops(self) -> float:
        """Algorithmic FLOP: 2 * valid rows * N * K (padding/masked rows excluded)."""
        return 2.0 * self.valid_rows * self.N * self.K

    def algorithmic_bytes(self) -> float:
        """A (valid rows) + B (groups with work) + SFA + SFB + D (valid rows), each once."""
        kb = self.K // 128
        nb = (self.N + 127) // 128
        rows = self.valid_rows
        return float(rows * self.K + self.active_groups * self.N * self.K
                     + rows * kb * 4 + self.active_groups * nb * kb * 4 + rows * self.N * 2)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _to_e4m3_bytes(q: torch.Tensor) -> np.ndarray:
    return q.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _pow2_scale(amax: torch.Tensor):
    """Power-of-two scale (UE8M0): the smallest 2^e >= amax / 448, and its inverse."""
    e = torch.ceil(torch.log2(amax.double() / E4M3_MAX))
    # log2 of a float32 ratio near a power of two: nudge so that 2^e >= amax/448 holds exactly
    e = torch.where(torch.exp2(e) * E4M3_MAX < amax.double(), e + 1, e)
    e = torch.where(torch.exp2(e - 1) * E4M3_MAX >= amax.double(), e - 1, e)
    return torch.exp2(e).float(), torch.exp2(-e).float()


def quantize_rows_1x128(x: np.ndarray, pow2: bool = False):
    """x float32 [..., K] -> (uint8 e4m3 [..., K], float32 scales [..., K/128]).
    pow2: scales rounded up to powers of two (the UE8M0 variant); x * 2^-e is exact."""
    K = x.shape[-1]
    assert K % 128 == 0
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    g = t.reshape(*t.shape[:-1], K // 128, 128)
    amax = g.abs().amax(dim=-1).clamp_min(SCALE_FLOOR)
    if pow2:
        s, inv = _pow2_scale(amax)
    else:
        s = amax / E4M3_MAX
        inv = E4M3_MAX / amax
    q = (g * inv.unsqueeze(-1)).clamp(-E4M3_MAX, E4M3_MAX).reshape(t.shape)
    return _to_e4m3_bytes(q), s.numpy().astype(np.float32)


def quantize_blocks_128x128(x: np.ndarray, pow2: bool = False):
    """x float32 [G][N][K] -> (uint8 [G][N][K], float32 [G][ceil(N/128)][K/128])."""
    G, N, K = x.shape
    assert K % 128 == 0
    nb = (N + 127) // 128
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    pad = nb * 128 - N
    tp = torch.nn.functional.pad(t, (0, 0, 0, pad)) if pad else t   # zero rows never raise amax
    blocks = tp.reshape(G, nb, 128, K // 128, 128)
    amax = blocks.abs().amax(dim=(2, 4)).clamp_min(SCALE_FLOOR)      # [G][nb][kb]
    if pow2:
        s, inv = _pow2_scale(amax)
    else:
        s = amax / E4M3_MAX
        inv = E4M3_MAX / amax
    q = (blocks * inv[:, :, None, :, None]).clamp(-E4M3_MAX, E4M3_MAX)
    q = q.reshape(G, nb * 128, K)[:, :N, :]
    return _to_e4m3_bytes(q.contiguous()), s.numpy().astype(np.float32)


def _normals(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def _weights(rng, G, N, K, pow2=False):
    Bf = _normals(rng, (G, N, K))
    B, SB = quantize_blocks_128x128(Bf, pow2)
    return B, SB


def make_dense(M: int, N: int, K: int, seed: int, outlier_frac: float = 0.0,
               name: str = "", pow2: bool = False) -> Problem:
    rng = _rng(seed)
    Af = _normals(rng, (M, K))
    if outlier_frac > 0.0 and M > 0:
        n_out = max(1, int(round(outlier_frac * M)))
        rows = rng.choice(M, size=n_out, replace=False)
        Af[rows] *= 100.0
    A, SA = quantize_rows_1x128(Af, pow2)
    B, SB = _weights(rng, 1, N, K, pow2)
    return Problem("dense", M, N, K, 1, A, SA, B, SB, seed=seed, name=name)


def contiguous_layout(counts, align: int = MK_ALIGNMENT) -> np.ndarray:
    """Group index per row: segment g = counts[g] rows of g, then -1 up to a multiple of align."""
    parts = []
    for g, c in enumerate(counts):
        c = int(c)
        padded = (c + align - 1) // align * align
        seg = np.full(padded, -1, dtype=np.int32)
        seg[:c] = g
        parts.append(seg)
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int32)


def make_contiguous(G: int, N: int, K: int, seed: int, total_rows: int = 32768,
                    counts=None, name: str = "", pow2: bool = False) -> Problem:
    rng = _rng(seed)
    if counts is None:
        counts = rng.multinomial(total_rows, [1.0 / G] * G)
    layout = contiguous_layout(counts)
    M = int(layout.shape[0])
    Af = _normals(rng, (M, K))
    A, SA = quantize_rows_1x128(Af, pow2)
    B, SB = _weights(rng, G, N, K, pow2)
    return Problem("contiguous", M, N, K, G, A, SA, B, SB, layout=layout, seed=seed, name=name)


def make_masked(G: int, max_m: int, N: int, K: int, seed: int, expected_m: int = 0,
                masked_m=None, name: str = "", pow2: bool = False) -> Problem:
    rng = _rng(seed)
    if masked_m is None:
        masked_m = rng.integers(1, max_m + 1, size=G)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    Af = _normals(rng, (G, max_m, K))
    A, SA = quantize_rows_1x128(Af, pow2)
    B, SB = _weights(rng, G, N, K, pow2)
    return Problem("masked", G * max_m, N, K, G, A, SA, B, SB, masked_m=masked_m, max_m=max_m,
                   expected_m=expected_m or max_m, seed=seed, name=name)


def stored_operands(p: Problem, ab: str):
    """A and B of a dense problem in the stored form ab ("nt", "nn", "tn", "tt"): A as
    [M][K] ("n") or [K][M] ("t"), B as [N][K] ("t") or [K][N] ("n").  Same values; the
    scales keep their layouts."""
    assert p.kind == "dense" and ab in ("nt", "nn", "tn", "tt")
    A = p.A if ab[0] == "n" else np.ascontiguousarray(p.A.T)
    B = p.B[0] if ab[1] == "t" else np.ascontiguousarray(p.B[0].T)
    return np.ascontiguousarray(A), np.ascontiguousarray(B)


@dataclasses.dataclass
class KGroupedProblem:
    """K-grouped (weight-gradient) problem, host numpy arrays in logical layouts.

    A:  uint8 [K_total][M]   (per token: the output gradient's M features)
    B:  uint8 [K_total][N]   (per token: the layer input's N features)
    SA: float32 [M][K_total/128], SB: float32 [N][K_total/128]
        (one scale per feature and 128-token chunk)
    ks: int64 [G] tokens per group along K, multiples of 128 (padding tokens are zero)
    counts: int64 [G] real tokens per group (ks is counts rounded up to 128)
    """
    M: int
    N: int
    G: int
    A: np.ndarray
    SA: np.ndarray
    B: np.ndarray
    SB: np.ndarray
    ks: np.ndarray
    counts: np.ndarray
    seed: int = 0
    name: str = ""
    kind: str = "k_grouped"

    @property
    def K(self) -> int:
        return int(self.ks.sum())

    def flops(self) -> float:
        """2 * M * N * (real tokens): padding tokens are not counted."""
        return 2.0 * self.M * self.N * float(self.counts.sum())

    def algorithmic_bytes(self, with_c: bool = False) -> float:
        """A + B + SA + SB once, D (FP32, every group) once, plus C when it is read."""
        K = self.K
        d = self.G * self.M * self.N * 4
        return float(K * (self.M + self.N) + (K // 128) * (self.M + self.N) * 4 + d
                     + (d if with_c else 0))


def _quantize_along_k(x: np.ndarray, pow2: bool = False):
    """x float32 [K][F] (K outermost) -> (uint8 [K][F], float32 [F][K/128]): one scale
    per feature and 128-row chunk, the 1x128 recipe applied along K."""
    q, s = quantize_rows_1x128(np.ascontiguousarray(x.T), pow2)
    return np.ascontiguousarray(q.T), s


def make_k_grouped(G: int, M: int, N: int, seed: int, total_tokens: int = 32768, counts=None,
                   name: str = "", pow2: bool = False) -> KGroupedProblem:
    rng = _rng(seed)
    if counts is None:
        counts = rng.multinomial(total_tokens, [1.0 / G] * G)
    counts = np.asarray(counts, dtype=np.int64)
    ks = (counts + MK_ALIGNMENT - 1) // MK_ALIGNMENT * MK_ALIGNMENT
    K = int(ks.sum())
    real = np.zeros(K, dtype=bool)                 # token rows that are not padding
    k0 = 0
    for c, k in zip(counts, ks):
        real[k0:k0 + c] = True
        k0 += int(k)
    Xa = _normals(rng, (K, M))
    Xb = _normals(rng, (K, N))
    Xa[~real] = 0.0
    Xb[~real] = 0.0
    A, SA = _quantize_along_k(Xa, pow2)
    B, SB = _quantize_along_k(Xb, pow2)
    return KGroupedProblem(M, N, G, A, SA, B, SB, ks, counts, seed=seed, name=name)


# ---- the workload families -------------------------------------------------

DENSE_PREFILL_NK = [(2112, 7168), (24576, 1536), (32768, 512), (7168, 16384), (4096, 7168),
                    (7168, 2048)]
DECODE_M = [64, 128, 256]
DECODE_NK = [(7168, 7168), (7168, 2048), (4096, 7168)]
MOE_NK = [(4096, 7168), (7168, 2048)]
# weight gradients of the two MoE projections above: dW [N_fwd][K_fwd] = dY^T X
KGROUPED_MN = [(4096, 7168), (7168, 2048)]


def workload_shapes(family: int) -> List[dict]:
    """Shape descriptors (no data) for workload family 0..6 (5: K-grouped weight
    gradients; 6: the dense nn / tn / tt stored forms, "form" naming how A and B are
    stored)."""
    out = []
    if family == 0:
        out.append(dict(kind="dense", M=128, N=2112, K=7168, seed=0, name="dense_m128_n2112_k7168"))
    elif family == 1:
        for j, (n, k) in enumerate(DENSE_PREFILL_NK):
            out.append(dict(kind="dense", M=4096, N=n, K=k, seed=1000 + j,
                            name=f"dense_m4096_n{n}_k{k}"))
    elif family == 2:
        j = 0
        for m in DECODE_M:
            for n, k in DECODE_NK:
                out.append(dict(kind="dense", M=m, N=n, K=k, seed=2000 + j, outlier_frac=0.01,
                                name=f"decode_m{m}_n{n}_k{k}"))
                j += 1
    elif family == 3:
        for j, (n, k) in enumerate(MOE_NK):
            out.append(dict(kind="contiguous", G=8, N=n, K=k, seed=3000 + j,
                            name=f"contig_g8_n{n}_k{k}"))
    elif family == 4:
        for j, (n, k) in enumerate(MOE_NK):
            out.append(dict(kind="masked", G=16, max_m=256, N=n, K=k, expected_m=128,
                            seed=4000 + j, name=f"masked_g16_m256_n{n}_k{k}"))
    elif family == 6:
        for j, form in enumerate(("nn", "tn", "tt")):
            out.append(dict(kind="dense", M=4096, N=4096, K=7168, seed=6000 + j, form=form,
                            name=f"dense_{form}_m4096_n4096_k7168"))
    elif family == 5:
        for j, (m, n) in enumerate(KGROUPED_MN):
            out.append(dict(kind="k_grouped", G=8, M=m, N=n, seed=5000 + j,
                            name=f"kgrouped_g8_m{m}_n{n}"))
    else:
        raise ValueError(family)
    return out


def make(desc: dict) -> Problem:
    d = dict(desc)
    kind = d.pop("kind")
    if kind == "dense":
        return make_dense(d["M"], d["N"], d["K"], d["seed"], d.get("outlier_frac", 0.0),
                          name=d.get("name", ""))
    if kind == "contiguous":
        return make_contiguous(d["G"], d["N"], d["K"], d["seed"], d.get("total_rows", 32768),
                               counts=d.get("counts"), name=d.get("name", ""))
    if kind == "masked":
        return make_masked(d["G"], d["max_m"], d["N"], d["K"], d["seed"], d.get("expected_m", 0),
                           masked_m=d.get("masked_m"), name=d.get("name", ""))
    if kind == "k_grouped":
        return make_k_grouped(d["G"], d["M"], d["N"], d["seed"], d.get("total_tokens", 32768),
                              counts=d.get("counts"), name=d.get("name", ""))
    raise ValueError(kind)
