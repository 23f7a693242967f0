"""GPU parity of the weight-only INT4 entry points against the oracle:
the quantizer bit for bit (codes and fp32 scales), and the GEMV against
the oracle's binary64 GEMV over the oracle's dequantized weights
(fp16(code * scale)) within the fp32 summation bound."""
import numpy as np
import pytest

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import request_decode_amd as rd
    rd.lib()
    return rd


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


@pytest.mark.parametrize("N,K", [(1, 128), (7, 256), (333, 2176), (1000, 2048), (4096, 2048), (2048, 5632),
                                 (16384, 4096), (100, 8192)])
def test_q4_quantize_and_gemv_vs_oracle(rd, orc, N, K):
    import torch
    print(f"q4 N={N} K={K}", flush=True)
    W, X = synth.gemv_inputs(N, K, 1, seed_w=N + 2 * K, seed_x=K + 5)
    if N >= 7:
        W[3, 128:256] = 0                      # an all-zero group
        W[5, :128] *= np.float16(200)          # a group of large weights
    Wd, Xd = dev(W), dev(X)
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((N, K // 128), dtype=torch.float32, device="cuda")
    rd.rd_q4_quantize(Wd.data_ptr(), N, K, codes.data_ptr(), scales.data_ptr())
    y = torch.full((N,), float("nan"), dtype=torch.float32, device="cuda")
    rd.rd_gemv_q4(codes.data_ptr(), scales.data_ptr(), Xd.data_ptr(), y.data_ptr(), N, K)
    torch.cuda.synchronize()
    rc, rs = orc.q4_quant(W)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs)
    Wq = orc.q4_dequant(rc, rs)
    ref = orc.gemv(Wq, X[0].astype(np.float64))
    got = y.cpu().numpy().astype(np.float64)
    # two fp32 chains per lane of 8 v_dot2_f32_f16 steps per 2048-column
    # chunk (a step: at most 37 * 2^-24 of its terms, as for the fp16
    # GEMV), then 6 fp32 adds across the wave
    mag = np.abs(Wq.astype(np.float64)) @ np.abs(X[0].astype(np.float64))
    bound = (37 * 8 * -(-K // 2048) + 6) * 2.0 ** -24 * mag + 1e-30
    err = np.abs(got - ref)
    assert np.all(err <= bound), float(np.nanmax(err / bound))
