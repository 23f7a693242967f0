"""Delta quantization of K/V segments on the GPU (rd_delta_seal,
rd_delta_restore) against the oracle ("Grok-3 v3.2.4 hot update deep dive",
§3.2): anchor rows, codes and (scale, zp) bit for bit, and the restored rows
bit for bit (the same binary32 operations in the same order)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def rd():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import request_decode_amd as rd
    rd.lib()
    return rd


def _run(rd, x):
    """x: uint16 [n_seg, n, hd] -> (anchor, codes, meta, restored) from the GPU."""
    import torch
    n_seg, n, hd = x.shape
    xin = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    anchor = torch.empty((n_seg, hd), dtype=torch.int16, device="cuda")
    codes = torch.empty((n_seg, max(n - 1, 1), hd), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_seg, 2), dtype=torch.float32, device="cuda")
    out = torch.empty((n_seg, n, hd), dtype=torch.float32, device="cuda")
    rd.rd_delta_seal(xin.data_ptr(), n_seg, n, hd, anchor.data_ptr(), codes.data_ptr(), meta.data_ptr())
    rd.rd_delta_restore(anchor.data_ptr(), codes.data_ptr(), meta.data_ptr(), n_seg, n, hd, out.data_ptr())
    torch.cuda.synchronize()
    return (anchor.cpu().numpy().view(np.uint16), codes.cpu().numpy()[:, : n - 1], meta.cpu().numpy(),
            out.cpu().numpy())


def _check(orc, x, got, idx=None):
    anchor, codes, meta, out = got
    for i in (range(x.shape[0]) if idx is None else idx):
        ra, rc, rs, rz = orc.delta_seal(x[i])
        assert np.array_equal(anchor[i], ra), i
        assert meta[i, 0] == rs and meta[i, 1] == rz, (i, meta[i], rs, rz)
        assert np.array_equal(codes[i], rc), i
        assert np.array_equal(out[i], orc.delta_restore(ra, rc, rs, rz)), i


def _walks(rng, n_seg, n, hd, step=0.05):
    x = np.cumsum(rng.normal(0, step, size=(n_seg, n, hd)), axis=1) + rng.normal(0, 1, size=(n_seg, 1, hd))
    return x.astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("n,hd", [(128, 128), (128, 64), (37, 96), (2, 8), (1, 128), (300, 64)])
def test_delta_bit_exact(rd, orc, n, hd):
    rng = np.random.default_rng(100 + n + hd)
    x = _walks(rng, 6, n, hd)
    if n > 2:
        xf = x.view(np.float16).astype(np.float32)
        xf[1, n // 2:] += 8.0                                      # an abrupt token
        xf[2] = np.arange(hd)[None, :] / 8.0 + np.arange(n)[:, None] * 0.25   # one constant step
        xf[3] = 0.0                                                # all zero: scale 1
        xf[4] = -1.5                                               # one repeated value
        x = xf.astype(np.float16).view(np.uint16)
    _check(orc, x, _run(rd, x))


def test_delta_full_size_sampled(rd, orc):
    # the K and V segments of every layer of the 2B cache at 8192 keys: 24
    # layers x 2 x 8 kv heads x 64 segments of 128 rows x 128; inputs drawn
    # on the device (seeded), sampled segments checked against the oracle
    import torch
    n_seg, n, hd = 24 * 2 * 8 * 64, 128, 128
    g = torch.Generator(device="cuda").manual_seed(17)
    x = torch.randn((n_seg, 1, hd), generator=g, device="cuda")
    x = (x + torch.cumsum(0.05 * torch.randn((n_seg, n, hd), generator=g, device="cuda"), dim=1)).half()
    anchor = torch.empty((n_seg, hd), dtype=torch.int16, device="cuda")
    codes = torch.empty((n_seg, n - 1, hd), dtype=torch.uint8, device="cuda")
    meta = torch.empty((n_seg, 2), dtype=torch.float32, device="cuda")
    out = torch.empty((n_seg, n, hd), dtype=torch.float32, device="cuda")
    rd.rd_delta_seal(x.data_ptr(), n_seg, n, hd, anchor.data_ptr(), codes.data_ptr(), meta.data_ptr())
    rd.rd_delta_restore(anchor.data_ptr(), codes.data_ptr(), meta.data_ptr(), n_seg, n, hd, out.data_ptr())
    torch.cuda.synchronize()
    idx = [0, 1, 4095, 12345, n_seg - 2, n_seg - 1] + list(np.random.default_rng(3).integers(0, n_seg, 26))
    sel = torch.tensor(idx, device="cuda")
    xs = x[sel].cpu().numpy().view(np.uint16)
    got = (anchor[sel].cpu().numpy().view(np.uint16), codes[sel].cpu().numpy(), meta[sel].cpu().numpy(),
           out[sel].cpu().numpy())
    _check(orc, xs, got)


def test_delta_errors(rd):
    import request_decode_amd as r
    for args in [(1, 0, 128), (1, 4097, 128), (1, 128, 0), (1, 128, 1025), (-1, 128, 128), (1, 128, 12)]:
        with pytest.raises(r.RdError):
            rd.rd_delta_seal(16, args[0], args[1], args[2], 16, 16, 16)
        with pytest.raises(r.RdError):
            rd.rd_delta_restore(16, 16, 16, args[0], args[1], args[2], 16)
    with pytest.raises(r.RdError):
        rd.rd_delta_seal(0, 1, 128, 128, 16, 16, 16)
