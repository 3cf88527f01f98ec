"""GPU: the kernels' E4M3 decoding and kv_append_quant against the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import cases
from tests.gpu_util import dev, device_cache, host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def test_e4m3_to_f16_all_codes(plc):
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8).cuda()
    got = host(plc.debug_e4m3_to_f16(codes)).astype(np.float64)
    ref = np.array([oracle.e4m3_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _compare_caches(c_gpu, c_ref, dtype):
    if dtype == "fp16":
        assert np.array_equal(host(c_gpu.k).view(np.uint16), c_ref.k)
        assert np.array_equal(host(c_gpu.v).view(np.uint16), c_ref.v)
    else:
        assert np.array_equal(host(c_gpu.k).view(np.uint8), c_ref.k.view(np.uint8))
        assert np.array_equal(host(c_gpu.v).view(np.uint8), c_ref.v.view(np.uint8))
    if dtype == "int8":
        assert np.array_equal(host(c_gpu.k_scale).view(np.uint32), c_ref.k_tok_scale.view(np.uint32))
        assert np.array_equal(host(c_gpu.v_scale).view(np.uint32), c_ref.v_tok_scale.view(np.uint32))


@pytest.mark.parametrize("dtype", ["fp16", "e4m3", "int8"])
@pytest.mark.parametrize("ctx,hkv", [([1], 1), ([17, 40, 3], 2), ([512], 1), ([300, 1000, 77, 16], 4)])
def test_append_bit_exact(plc, dtype, ctx, hkv):
    w = synthetic.generate(cases.spec(ctx, ctx, hq=hkv * 2, hkv=hkv, seed=101 + len(ctx)))
    c_gpu, _ = device_cache(plc, w, dtype)
    torch.cuda.synchronize()
    _compare_caches(c_gpu, cases.oracle_cache(w, dtype), dtype)


@pytest.mark.parametrize("dtype", ["e4m3", "int8"])
def test_append_in_chunks_matches_oracle(plc, dtype):
    # prefix first, then the new chunk at start_pos (the chunked-prefill write pattern)
    w = synthetic.generate(cases.spec([200, 45], [37, 45], hq=8, hkv=1, seed=7))
    c_gpu, bt = device_cache(plc, w, dtype, upto="prefix")
    kn, vn = w.new_kv()
    plc.kv_append_quant(c_gpu, dev(kn), dev(vn), bt, dev(w.cu_q_lens), dev(w.start_pos))
    torch.cuda.synchronize()
    _compare_caches(c_gpu, cases.oracle_cache(w, dtype), dtype)


@pytest.mark.parametrize("scale", [1.0, 0.37109375, 1.0 / 448.0, 3.0e-3, 150.0])
def test_e4m3_encoder_on_every_f16_value(plc, scale):
    f16 = np.arange(65536, dtype=np.uint16).view(np.float16)
    f16 = f16[np.isfinite(f16)]
    pad = (-f16.size) % 128
    x = np.concatenate([f16, np.zeros(pad, np.float16)]).reshape(-1, 1, 128)
    T = x.shape[0]
    spec = cases.spec([T], [T], hq=1, hkv=1, seed=1)
    w = synthetic.generate(spec)
    w.k[:] = x
    w.v[:] = -x
    w.k_scale_head[:] = np.float32(scale)
    w.v_scale_head[:] = np.float32(scale)
    c_gpu, _ = device_cache(plc, w, "e4m3")
    torch.cuda.synchronize()
    _compare_caches(c_gpu, cases.oracle_cache(w, "e4m3"), "e4m3")


def test_int8_rows_with_zeros_and_ties(plc):
    spec = cases.spec([64], [64], hq=1, hkv=1, seed=3)
    w = synthetic.generate(spec)
    w.k[0] = 0                                   # all-zero row: sigma 0, codes 0
    w.k[1, 0, :] = 0
    w.k[1, 0, 0] = 127
    w.k[1, 0, 1:7] = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5]
    w.v[2] = np.float16(65504)                   # largest fp16
    c_gpu, _ = device_cache(plc, w, "int8")
    torch.cuda.synchronize()
    _compare_caches(c_gpu, cases.oracle_cache(w, "int8"), "int8")


def test_append_leaves_unowned_slots_untouched(plc):
    w = synthetic.generate(cases.spec([5, 21], [5, 21], hq=1, hkv=1, seed=9))
    c_gpu, _ = device_cache(plc, w, "e4m3")
    torch.cuda.synchronize()
    k = host(c_gpu.k)
    owned = np.zeros(k.shape[:3], bool)
    for b in range(2):
        for j in range(int(w.context_lens[b])):
            owned[w.block_tables[b, j // 16], :, j % 16] = True
    assert np.all(k[~owned] == synthetic.POISON_CODE_8BIT)
