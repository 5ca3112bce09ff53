"""Pins for the oracle's quantiser (the step that turns FP32 activations / weights into
e4m3 bytes plus FP32 block scales), checked against things other than itself:

* the e4m3 encoder against torch's float8_e4m3fn cast (a library routine) on every
  code value, every tie between neighbouring codes, values one ulp either side of
  the ties, and a million random values;
* the block quantisers against the input generator's torch implementation of the
  same recipe (written independently, in torch ops);
* closed forms: constant blocks, all-zero blocks, power-of-two ladders.
"""
import numpy as np
import pytest
import torch

import oracle
from moe_grouped_gemm_block_amd import synth


def _torch_e4m3(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def _enc(x: np.ndarray) -> np.ndarray:
    return np.array([oracle.enc_e4m3(float(v)) for v in x.ravel()], dtype=np.uint8).reshape(x.shape)


def _code_values():
    return np.array([oracle.dec_e4m3(c) for c in range(127)], dtype=np.float64)


def test_every_code_value_round_trips():
    vals = _code_values().astype(np.float32)
    assert np.array_equal(_enc(vals), np.arange(127, dtype=np.uint8))
    assert np.array_equal(_enc(-vals), (np.arange(127) | 0x80).astype(np.uint8))
    assert np.array_equal(_enc(vals), _torch_e4m3(vals))


def test_ties_go_to_the_even_code_like_torch():
    vals = _code_values()
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)      # exact in FP32
    assert np.array_equal(mids.astype(np.float64), (vals[:-1] + vals[1:]) / 2)
    ours = _enc(mids)
    assert np.all(ours % 2 == 0)
    assert np.array_equal(ours, _torch_e4m3(mids))
    for side in (np.float32(np.inf), np.float32(0.0)):
        near = np.nextafter(mids, side).astype(np.float32)
        assert np.array_equal(_enc(near), _torch_e4m3(near))
        assert np.array_equal(_enc(-near), _torch_e4m3(-near))


def test_random_values_match_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.uniform(-448, 448, 200_000),
        rng.standard_normal(200_000) * 4,
        np.exp2(rng.uniform(-14, 8.8, 200_000)) * rng.choice([-1, 1], 200_000),
    ]).astype(np.float32)
    x = np.clip(x, -448, 448)
    sub = x[::7]                                                   # keep the pure-Python loop short
    assert np.array_equal(_enc(sub), _torch_e4m3(sub))


def test_activation_quantiser_matches_the_generator():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((48, 512)).astype(np.float32)
    x[3] *= 100.0                                                  # an outlier row
    x[5, 128:256] = 0.0                                            # an all-zero group: the floor
    x[7, :128] *= 1e-6                                             # codes in the subnormal range
    x[9, 256:384] = -x[9, 256:384]
    q, s = oracle.quant_1x128(x)
    q_ref, s_ref = synth.quantize_rows_1x128(x)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


def test_weight_quantiser_matches_the_generator():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 200, 384)).astype(np.float32)     # N = 200: a partial last block
    x[1, 150:200, :] *= 30.0                                       # the partial block's own amax
    q, s = oracle.quant_128x128(x)
    q_ref, s_ref = synth.quantize_blocks_128x128(x)
    assert q.shape == (2, 200, 384) and s.shape == (2, 2, 3)
    assert np.array_equal(q, q_ref)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))


@pytest.mark.parametrize("c", [1.0, 3.0, 0.37, 1234.5, -2.5])
def test_constant_group_is_all_max_code(c):
    x = np.full((1, 128), c, dtype=np.float32)
    q, s = oracle.quant_1x128(x)
    code = 0x7E | (0x80 if c < 0 else 0)
    assert np.all(q == code)
    assert s[0, 0] == np.float32(np.float32(abs(c)) / np.float32(448.0))


def test_zero_group_uses_the_floor():
    q, s = oracle.quant_1x128(np.zeros((2, 256), dtype=np.float32))
    assert np.all(q == 0)
    assert np.all(s == np.float32(np.float32(1e-4) / np.float32(448.0)))


def test_power_of_two_ladder_is_exact():
    # x = 2^(k+8), k in [-6, 0]: amax 2^8, inv = 448/256 = 1.75 exactly, and every product
    # 1.75 * 2^(k+8) is exact and an e4m3 value (7 .. 448)
    k = np.arange(-6, 1)
    x = np.zeros((1, 128), dtype=np.float32)
    x[0, :k.size] = np.exp2(k + 8).astype(np.float32)
    q, s = oracle.quant_1x128(x)
    assert s[0, 0] == np.float32(256.0 / 448.0)
    for i, kk in enumerate(k):
        assert oracle.dec_e4m3(int(q[0, i])) == 1.75 * 2.0 ** (kk + 8)


def test_weight_block_scale_covers_only_existing_rows():
    x = np.ones((1, 130, 128), dtype=np.float32)
    x[0, 129, 5] = 7.0                                             # only in the second row block
    q, s = oracle.quant_128x128(x)
    assert s[0, 0, 0] == np.float32(1.0 / 448.0)
    assert s[0, 1, 0] == np.float32(np.float32(7.0) / np.float32(448.0))
    assert np.all(q[0, :128] == 0x7E)
