"""hpa_kv_pack_pages through the C ABI: row-major [pages, Hkv, 64, 128] pages turned
into the tiled blocks the attention kernels read. The packed bytes must equal the
input generator's tiling bit for bit (whole pool, a page list, in place), and
attention over a cache packed on the GPU must match the oracle and the run on the
generator's own tiled cache."""

import numpy as np
import pytest

from load_balanced_split_amd import _lib, inputs
from oracle import attention as oa
from tests.helpers import assert_within, ensure_built

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ensure_built()
    _lib.lib()


def _dev(a):
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.to("cuda")


def _host(t, dtype):
    return t.cpu().numpy().view(dtype)


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_pack_equals_generator_tiling(kv_dtype):
    rng = np.random.default_rng(11)
    P, hkv = 37, 2
    dtype = np.uint16 if kv_dtype == "bf16" else np.uint8
    top = 65536 if kv_dtype == "bf16" else 256
    k = rng.integers(0, top, size=(P, hkv, 64, 128)).astype(dtype)
    v = rng.integers(0, top, size=(P, hkv, 64, 128)).astype(dtype)
    want_k, want_v = inputs.tile_k(k, kv_dtype), inputs.tile_v(v, kv_dtype)
    desc = _lib.make_desc(1, hkv, hkv, 1, P, kv_dtype)
    kr, vr = _dev(k), _dev(v)
    # whole pool into separate caches
    kc, vc = torch.zeros_like(kr), torch.zeros_like(vr)
    print(f"pack {kv_dtype} whole pool", flush=True)
    _lib.hpa_kv_pack_pages(desc, kr, vr, None, kc, vc)
    torch.cuda.synchronize()
    assert np.array_equal(_host(kc, dtype).reshape(P, hkv, -1), want_k)
    assert np.array_equal(_host(vc, dtype).reshape(P, hkv, -1), want_v)
    # a page list: 9 source pages to scattered blocks, every other block untouched
    dst = rng.permutation(P)[:9].astype(np.int32)
    kc.fill_(0)
    vc.fill_(0)
    print(f"pack {kv_dtype} page list", flush=True)
    _lib.hpa_kv_pack_pages(desc, kr[:9].contiguous(), vr[:9].contiguous(), _dev(dst), kc, vc)
    torch.cuda.synchronize()
    gk, gv = _host(kc, dtype).reshape(P, hkv, -1), _host(vc, dtype).reshape(P, hkv, -1)
    assert np.array_equal(gk[dst], want_k[:9]) and np.array_equal(gv[dst], want_v[:9])
    rest = np.setdiff1d(np.arange(P), dst)
    assert not gk[rest].any() and not gv[rest].any()
    # in place over the whole pool
    print(f"pack {kv_dtype} in place", flush=True)
    _lib.hpa_kv_pack_pages(desc, kr, vr, None, kr, vr)
    torch.cuda.synchronize()
    assert np.array_equal(_host(kr, dtype).reshape(P, hkv, -1), want_k)
    assert np.array_equal(_host(vr, dtype).reshape(P, hkv, -1), want_v)


def test_pack_reports_bad_page_ids():
    desc = _lib.make_desc(1, 8, 1, 1, 4, "bf16")
    rows = torch.ones((2, 1, 64, 128), dtype=torch.int16, device="cuda")
    kc = torch.zeros((4, 1, 8192), dtype=torch.int16, device="cuda")
    vc = torch.zeros_like(kc)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    _lib.hpa_kv_pack_pages(desc, rows, rows, _dev(np.array([2, 9], np.int32)), kc, vc, err)
    torch.cuda.synchronize()
    assert int(err.item()) & _lib.DEVERR_PAGE_ID
    assert bool(torch.all(kc[2] == 1)) and not bool(kc[[0, 1, 3]].any())


@pytest.mark.parametrize("cfg", [0, 2])
def test_attention_over_a_cache_packed_on_the_gpu(cfg):
    """The workload's cache handed over row-major (the generator's tiling undone),
    packed in place on the GPU, then attended: the oracle's output within tolerance
    and the same bits as the run on the generator's tiled cache."""
    from load_balanced_split_amd.runner import DeviceStep
    w = inputs.config_workload(cfg)
    d = DeviceStep(w)
    d.step("fused")
    torch.cuda.synchronize()
    want = d.out.clone()
    d.k_cache.copy_(_dev(inputs.untile_k(w.k_cache, w.kv_dtype)).view(d.k_cache.shape))
    d.v_cache.copy_(_dev(inputs.untile_v(w.v_cache, w.kv_dtype)).view(d.v_cache.shape))
    print(f"pack cfg{cfg} in place, then attention", flush=True)
    _lib.hpa_kv_pack_pages(d.desc, d.k_cache, d.v_cache, None, d.k_cache, d.v_cache)
    d.out.zero_()
    d.step("fused")
    torch.cuda.synchronize()
    assert d.device_error() == 0
    assert torch.equal(d.out, want)
    ref = oa.decode_attention(w.q, w.k_cache, w.v_cache, w.seq_lens, w.page_table, w.hkv, w.sm_scale)
    assert_within(d.output_f64(), ref, "bf16", f"cfg{cfg} packed on the GPU")
