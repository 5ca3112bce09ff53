"""Host checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

from moe_grouped_gemm_block_amd import synth


def _dec(b):
    return torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_same_seed_same_bytes_and_different_seed_differs():
    p1 = synth.make_dense(64, 300, 256, seed=5, outlier_frac=0.01)
    p2 = synth.make_dense(64, 300, 256, seed=5, outlier_frac=0.01)
    p3 = synth.make_dense(64, 300, 256, seed=6, outlier_frac=0.01)
    for f in ("A", "SA", "B", "SB"):
        assert np.array_equal(getattr(p1, f), getattr(p2, f))
    assert not np.array_equal(p1.A, p3.A)


def test_quantised_bytes_are_finite_and_each_group_reaches_448():
    p = synth.make_dense(32, 200, 384, seed=1)
    for q, shape in ((p.A, (32, 3, 128)), (p.B[0], None)):
        v = _dec(q)
        assert np.all(np.isfinite(v)) and np.abs(v).max() <= 448.0
    a = np.abs(_dec(p.A)).reshape(32, 3, 128).max(axis=2)
    assert np.all(a == 448.0)
    # B: 128x128 blocks, the last one partial (200 = 128 + 72 rows)
    b = np.abs(_dec(p.B[0]))
    for j, (r0, r1) in enumerate(((0, 128), (128, 200))):
        for c in range(3):
            assert b[r0:r1, 128 * c:128 * c + 128].max() == 448.0
    assert p.SB.shape == (1, 2, 3) and p.SA.shape == (32, 3)


def test_dequantised_values_track_the_normals():
    rng = np.random.Generator(np.random.PCG64(3))
    x = rng.standard_normal((16, 256), dtype=np.float32)
    q, s = synth.quantize_rows_1x128(x)
    deq = _dec(q).reshape(16, 2, 128) * s[:, :, None]
    rel = np.abs(deq.reshape(16, 256) - x) / (np.abs(x) + 1e-3)
    assert np.median(rel) < 0.04          # e4m3 keeps 4 significant bits


def test_outlier_rows():
    p = synth.make_dense(256, 128, 128, seed=2, outlier_frac=0.01)
    big = np.nonzero(p.SA[:, 0] > 10 * np.median(p.SA[:, 0]))[0]
    assert big.size == 3                   # round(0.01 * 256)


def test_contiguous_layout_alignment_and_counts():
    p = synth.make_contiguous(8, 256, 128, seed=3000, total_rows=4096)
    lay = p.layout
    assert p.M % 128 == 0 and lay.shape == (p.M,)
    counts = [(lay == g).sum() for g in range(8)]
    assert sum(counts) == 4096
    for blk in range(p.M // 128):
        ids = lay[128 * blk:128 * blk + 128]
        valid = ids[ids >= 0]
        assert np.unique(valid).size <= 1          # one expert per aligned block
        if valid.size:
            assert np.all(ids[:valid.size] == valid[0]) and np.all(ids[valid.size:] == -1)


def test_masked_counts_in_range():
    p = synth.make_masked(16, 256, 128, 128, seed=4000, expected_m=128)
    assert p.A.shape == (16, 256, 128) and p.SA.shape == (16, 256, 1)
    assert p.masked_m.min() >= 1 and p.masked_m.max() <= 256


def test_workload_families_cover_the_shapes():
    n = [len(synth.workload_shapes(i)) for i in range(5)]
    assert n == [1, 6, 9, 2, 2]


def test_k_grouped_segments_padding_and_scales():
    p = synth.make_k_grouped(4, 48, 40, seed=5000, total_tokens=700)
    assert p.counts.sum() == 700 and np.all(p.ks % 128 == 0)
    assert np.all(p.ks - p.counts >= 0) and np.all(p.ks - p.counts < 128)
    K = int(p.ks.sum())
    assert p.A.shape == (K, 48) and p.B.shape == (K, 40)
    assert p.SA.shape == (48, K // 128) and p.SB.shape == (40, K // 128)
    k0 = 0
    for c, k in zip(p.counts, p.ks):
        assert np.all(p.A[k0 + c:k0 + k] == 0) and np.all(p.B[k0 + c:k0 + k] == 0)
        k0 += int(k)
    # one scale per feature and 128-token chunk: every chunk of a feature with real tokens
    # reaches the e4m3 maximum once
    for c in range(K // 128):
        col = p.A[128 * c:128 * c + 128, :]
        if np.any(col):
            assert np.all((col & 0x7F).max(axis=0) == 0x7E)
    assert [len(synth.workload_shapes(5))] == [2]


def test_stored_operands_are_transposes():
    p = synth.make_dense(40, 70, 256, seed=1)
    for ab in ("nt", "nn", "tn", "tt"):
        A, B = synth.stored_operands(p, ab)
        assert np.array_equal(A if ab[0] == "n" else A.T, p.A)
        assert np.array_equal(B if ab[1] == "t" else B.T, p.B[0])
