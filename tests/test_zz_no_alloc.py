"""rd_attention_noalloc (the entry point that allocates nothing) against
rd_attention, through the C ABI: bit-identical outputs (the same kernels in
the same order), on two calls in a row, the second with a smaller input,
and a request past the fixed scratch rejected before anything runs."""
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


def _case(H, Hk, hd, L, kv, seed):
    import torch
    rng = np.random.default_rng(seed)
    ld = L + 5
    q = torch.from_numpy(rng.standard_normal((H, hd)).astype(np.float32)).cuda()
    d = {"q": q}
    if kv == "fp16":
        d["K"] = torch.from_numpy(rng.standard_normal((Hk, ld, hd)).astype(np.float16)).cuda()
        d["V"] = torch.from_numpy(rng.standard_normal((Hk, ld, hd)).astype(np.float16)).cuda()
    else:
        nseg = -(-ld // 128)
        for n in ("K", "V"):
            d[n] = torch.from_numpy(rng.integers(0, 256, (Hk, ld, hd), dtype=np.uint8)).cuda()
            d[n + "s"] = torch.from_numpy(rng.standard_normal((Hk, 128, hd)).astype(np.float16)).cuda()
            m = np.empty((Hk, nseg, 2), np.float32)
            m[..., 0] = rng.uniform(0.005, 0.02, (Hk, nseg))
            m[..., 1] = rng.integers(50, 200, (Hk, nseg))
            d[n + "m"] = torch.from_numpy(m).cuda()
    return d, ld


def _run(rd, fn, d, H, Hk, hd, L, ld, kv, splits):
    import torch
    out = torch.full((H, hd), float("nan"), dtype=torch.float32, device="cuda")
    extra = {}
    if kv == "int8":
        extra = dict(k_stage=d["Ks"].data_ptr(), v_stage=d["Vs"].data_ptr(), k_meta=d["Km"].data_ptr(),
                     v_meta=d["Vm"].data_ptr())
    fn(d["q"].data_ptr(), d["K"].data_ptr(), d["V"].data_ptr(), out.data_ptr(), H, Hk, hd, L, ld, kv,
       float(1.0 / np.sqrt(hd)), splits, **extra)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("kv", ["fp16", "int8"])
def test_noalloc_matches_rd_attention(rd, kv):
    for (H, Hk, hd, L, splits) in [(16, 8, 128, 3000, 32), (4, 2, 64, 200, 7)]:   # second call smaller
        print(f"noalloc {kv} H={H} Hk={Hk} hd={hd} L={L} S={splits}", flush=True)
        d, ld = _case(H, Hk, hd, L, kv, seed=L)
        ref = _run(rd, rd.rd_attention, d, H, Hk, hd, L, ld, kv, splits)
        got = _run(rd, rd.rd_attention_noalloc, d, H, Hk, hd, L, ld, kv, splits)
        assert np.all(np.isfinite(ref))
        assert np.array_equal(got, ref), (kv, H, L)


def test_noalloc_rejects_past_its_scratch(rd):
    import torch
    d, ld = _case(128, 16, 128, 64, "fp16", seed=1)
    out = torch.zeros((128, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(rd.RdError) as e:
        rd.rd_attention_noalloc(d["q"].data_ptr(), d["K"].data_ptr(), d["V"].data_ptr(), out.data_ptr(), 128, 16,
                                128, 64, ld, "fp16", 0.088, 256)   # 128 * 256 * 130 * 4 B > 4 MiB
    assert e.value.status == rd.RD_ERR_INVALID_ARG and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy() == 0)
