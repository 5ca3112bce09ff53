"""GPU parity of the quantisers (through the C ABI) against the CPU oracle: e4m3 codes
bit-exact, FP32 scales bit-exact, MN-major SFA placement exact, alignment padding and
rows outside the problem untouched; and the quantiser's output fed to the GEMM."""
import sys

import numpy as np
import pytest
import torch

import oracle
import moe_grouped_gemm_block_amd as fp8bs
from moe_grouped_gemm_block_amd import synth
from _helpers import check_full, oracle_full, SENTINEL

pytestmark = pytest.mark.gpu

PAD = np.float32(-12345.0)


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(shape, seed, dtype):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    flat = x.reshape(-1, shape[-1])
    flat[0, :128] = 0.0                                   # an all-zero group (scale floor)
    if flat.shape[0] > 1:
        flat[1, :128] *= 1e-6                             # subnormal e4m3 codes
    if flat.shape[0] > 2:
        flat[2] *= 300.0                                  # an outlier row
    t = torch.from_numpy(x)
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
        x = t.to(torch.float32).numpy()                   # exact widening, what the GPU sees
    return t, x


def _sfa_logical(sfa_dev, rows):
    """MN-major [(G,) k/128, ld] -> logical [(G,) rows, k/128]; also returns the padding."""
    s = sfa_dev.cpu().numpy()
    return np.swapaxes(s[..., :rows], -1, -2), s[..., rows:]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,rows,k", [(1, 1, 128), (1, 63, 256), (1, 64, 512), (1, 65, 384),
                                      (1, 300, 1024), (3, 70, 256)])
def test_activation_quantiser_bit_exact(dtype, G, rows, k):
    _say(f"[gpu] quantize_1x128 {dtype} G={G} rows={rows} k={k}")
    shape = (rows, k) if G == 1 else (G, rows, k)
    t, x = _inputs(shape, 100 + rows + k + G, dtype)
    xd = t.cuda()
    q = torch.full(shape, 0xAB, dtype=torch.uint8, device="cuda")
    ld = fp8bs.get_sfa_ld(rows)
    sshape = (k // 128, ld) if G == 1 else (G, k // 128, ld)
    sfa = torch.full(sshape, float(PAD), dtype=torch.float32, device="cuda")
    fp8bs.fp8bs_quantize_1x128(xd, q, sfa)
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_1x128(x.reshape(-1, k))
    assert np.array_equal(q.cpu().numpy().reshape(-1, k), q_ref)
    s_log, pad = _sfa_logical(sfa, rows)
    assert np.array_equal(s_log.reshape(-1, k // 128).view(np.uint32), s_ref.view(np.uint32))
    assert np.all(pad == PAD)


def test_activation_quantiser_ties_and_signs():
    # amax = 448 -> inv = 1 exactly, so every input is its own product: e4m3 midpoints
    # (ties), values one ulp either side, negative zero and tiny negatives
    vals = np.array([oracle.dec_e4m3(c) for c in range(127)])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    row = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf))])
    row = np.concatenate([row, -row])
    n = (row.size + 127) // 128 * 128
    x = np.zeros((1, n), dtype=np.float32)
    x[0, :row.size] = row
    for c in range(n // 128):                           # every group gets amax exactly 448
        x[0, 128 * c + 127] = 448.0
    x[0, 0] = -0.0
    x[0, 1] = -1e-30
    q, sfa = fp8bs.quantize_1x128(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_1x128(x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert q_ref[0, 0] == 0x80 and q_ref[0, 1] == 0x80


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("G,n,k", [(1, 200, 384), (2, 128, 256), (1, 1, 128), (3, 300, 512)])
def test_weight_quantiser_bit_exact(dtype, G, n, k):
    _say(f"[gpu] quantize_128x128 {dtype} G={G} n={n} k={k}")
    shape = (n, k) if G == 1 else (G, n, k)
    t, x = _inputs(shape, 200 + n + k + G, dtype)
    q, sfb = fp8bs.quantize_128x128(t.cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_128x128(x.reshape(G, n, k))
    assert np.array_equal(q.cpu().numpy().reshape(G, n, k), q_ref)
    assert np.array_equal(sfb.cpu().numpy().reshape(s_ref.shape).view(np.uint32),
                          s_ref.view(np.uint32))


def test_activation_quantiser_full_size_sampled_rows():
    rows, k = 4096, 7168
    _say(f"[gpu] quantize_1x128 bf16 full size {rows}x{k}")
    t, x = _inputs((rows, k), 300, "bf16")
    q, sfa = fp8bs.quantize_1x128(t.cuda())
    torch.cuda.synchronize()
    pick = np.random.default_rng(301).choice(rows, size=192, replace=False)
    pick = np.concatenate([pick, [0, 1, 2, rows - 1]])
    q_ref, s_ref = oracle.quant_1x128(x[pick])
    assert np.array_equal(q.cpu().numpy()[pick], q_ref)
    s_log, _ = _sfa_logical(sfa, rows)
    assert np.array_equal(s_log[pick].view(np.uint32), s_ref.view(np.uint32))


def test_quantiser_output_feeds_the_gemm():
    """FP32 activations and weights quantised on the GPU, multiplied by the GEMM, against
    the oracle's quantiser followed by the oracle's GEMM."""
    M, N, K = 200, 300, 640
    rng = np.random.default_rng(400)
    xa = rng.standard_normal((M, K)).astype(np.float32)
    xb = rng.standard_normal((N, K)).astype(np.float32)
    a, sfa = fp8bs.quantize_1x128(torch.from_numpy(xa).cuda())
    b, sfb = fp8bs.quantize_128x128(torch.from_numpy(xb).cuda())
    d = torch.full((M, N), SENTINEL, dtype=torch.int16, device="cuda")
    fp8bs.dense_nt(a, sfa, b, sfb, d)
    torch.cuda.synchronize()
    A, SA = oracle.quant_1x128(xa)
    B, SB = oracle.quant_128x128(xb[None])
    p = synth.Problem("dense", M, N, K, 1, A, SA, B, SB)
    check_full(p, d.cpu().numpy().view(np.uint16), oracle_full(p), "quantised then multiplied")


def test_quantiser_validation():
    lib = fp8bs._load()
    buf = torch.zeros(4096, dtype=torch.float32, device="cuda")
    ptr = buf.data_ptr()
    assert lib.fp8bs_quantize_1x128(ptr, 0, ptr, ptr, 1, 4, 100, None) == 1      # K not 128k
    assert lib.fp8bs_quantize_1x128(ptr, 7, ptr, ptr, 1, 4, 128, None) == 3      # dtype
    assert lib.fp8bs_quantize_1x128(ptr + 4, 0, ptr, ptr, 1, 4, 128, None) == 2  # alignment
    assert lib.fp8bs_quantize_1x128(ptr, 0, ptr, ptr, 1, 0, 128, None) == 0      # nothing to do
    assert lib.fp8bs_quantize_128x128(ptr, 0, ptr, ptr, 1, 0, 128, None) == 1
    torch.cuda.synchronize()


def test_nan_inputs_keep_their_sign_on_the_nan_code():
    """NaN never raises a block's maximum and becomes the NaN code with its sign; the rest
    of the group (converted by the hardware instruction) stays bit-exact."""
    rng = np.random.default_rng(500)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    x[0, 5] = np.nan
    x[1, 130] = -np.nan
    x[2, 0] = np.float32(np.copysign(np.nan, -1.0))
    q, sfa = fp8bs.quantize_1x128(torch.from_numpy(x).cuda())
    torch.cuda.synchronize()
    q_ref, s_ref = oracle.quant_1x128(x)
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert (q_ref[0, 5] & 0x7F) == 0x7F and (q_ref[2, 0] == 0xFF)
    s_log, _ = _sfa_logical(sfa, 3)
    assert np.array_equal(s_log.view(np.uint32), s_ref.view(np.uint32))
