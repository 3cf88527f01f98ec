"""The C-ABI library loads, exports what include/plc.h declares, and refuses bad
arguments on the host before touching the GPU (CPU only: no kernel runs)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "plc.h")


@pytest.fixture(scope="module")
def plc():
    import paged_long_context_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(plc_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["plc_kv_append_quant", "plc_attn_prefill_paged", "plc_attn_decode_paged",
              "plc_lse_merge", "plc_attn_decode_partials", "plc_decode_workspace_size",
              "plc_attn_verify_paged", "plc_verify_workspace_size",
              "plc_abi_version", "plc_last_error"]:
        assert n in names


def test_library_exports_every_declared_symbol(plc):
    lib = ctypes.CDLL(plc.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing


def test_abi_version(plc):
    assert plc.lib().plc_abi_version() == plc.ABI_VERSION == 3
    assert plc.verify_max_query_tokens() == plc.VERIFY_MAX_Q_LEN == 16


def _desc(plc, dtype=1, head_dim=128, block_size=16, num_blocks=10, hkv=1, scales=True):
    fake = 0x1000  # never dereferenced: every call below fails validation first
    return plc.plc_kv_cache(fake, fake, fake if scales else None, fake if scales else None,
                            num_blocks, block_size, hkv, head_dim, dtype)


def _decode(plc, desc, hq=8, max_blocks=4, max_ctx=64, part=0, ws_bytes=1 << 20, ws=0x2000,
            q=0x3000):
    return plc.lib().plc_attn_decode_paged(q, hq, ctypes.byref(desc), 0x4000, max_blocks, 0x5000, 2,
                                           max_ctx, part, 0.088, 0x6000, 0x7000, ws, ws_bytes, None)


def _err(plc):
    return plc.lib().plc_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(dtype=7), -2, "dtype"),
    (dict(head_dim=64), -2, "head_dim"),
    (dict(block_size=32), -2, "block_size"),
    (dict(scales=False), -1, "never assumed 1.0"),
    (dict(num_blocks=0), -1, "num_blocks"),
])
def test_cache_descriptor_is_validated(plc, kw, code, msg):
    assert _decode(plc, _desc(plc, **kw)) == code
    assert msg in _err(plc)


def test_fp16_cache_needs_no_scales(plc):
    # fails later, on the workspace, proving the scale check passed
    assert _decode(plc, _desc(plc, dtype=0, scales=False), ws=None) == -3


def test_int8_cache_needs_scales(plc):
    assert _decode(plc, _desc(plc, dtype=2, scales=False)) == -1


@pytest.mark.parametrize("hq,code", [(12, -1), (3, -2), (24, -2), (32, -2)])
def test_group_size_is_validated(plc, hq, code):
    assert _decode(plc, _desc(plc, hkv=1 if hq != 12 else 8), hq=hq) == code


def test_context_longer_than_table_is_refused(plc):
    assert _decode(plc, _desc(plc), max_blocks=4, max_ctx=65) == -1
    assert "capacity" in _err(plc)


def test_partition_must_be_block_multiple(plc):
    assert _decode(plc, _desc(plc), part=24) == -1
    assert "multiple" in _err(plc)


def test_workspace_too_small(plc):
    need = plc.decode_workspace_size(2, 8, 128, 64, 0)
    assert need > 0
    assert _decode(plc, _desc(plc), ws_bytes=need - 1) == -3
    assert "needed" in _err(plc)


def test_null_query_refused(plc):
    assert _decode(plc, _desc(plc), q=None) == -1


def test_workspace_size_formula(plc):
    # rows * nparts * D floats, then rows * nparts floats, each 256-byte aligned
    def want(rows, nparts):
        return ((rows * nparts * 128 * 4 + 255) // 256) * 256 + ((rows * nparts * 4 + 255) // 256) * 256
    # 8 sequences x 16 partitions fill half the chip: room for each partition
    # split over two workgroups (32 partials per row)
    assert plc.decode_workspace_size(8, 8, 128, 32768, 2048) == want(8 * 8, 32)
    # 32 sequences x 16 partitions already fill it: no split, 16 per row
    assert plc.decode_workspace_size(32, 8, 128, 32768, 2048) == want(32 * 8, 16)


def test_default_partition_choice(plc):
    p = plc.decode_partition_tokens(8, 1, 32768, 0)
    assert p % 16 == 0 and 512 <= p <= 4096
    assert plc.decode_partition_tokens(8, 1, 32768, 2048) == 2048


def test_prefill_and_merge_and_append_validation(plc):
    L = plc.lib()
    d = _desc(plc)
    assert L.plc_attn_prefill_paged(0x1, 8, ctypes.byref(d), 0x1, 4, 0x1, 0x1, 1, 10, 100, 64,
                                    0.1, 0x1, 0x1, None) == -1      # max_q_len > max_context_len
    assert L.plc_attn_prefill_paged(None, 8, ctypes.byref(d), 0x1, 4, 0x1, 0x1, 1, 10, 10, 64,
                                    0.1, 0x1, 0x1, None) == -1      # null q
    assert L.plc_lse_merge(0x1, 0x1, 4, 0, 128, 0x1, 0x1, None) == -1
    assert L.plc_lse_merge(0x1, 0x1, 4, 2, 1024, 0x1, 0x1, None) == -1
    assert L.plc_lse_merge(None, 0x1, 4, 2, 128, 0x1, 0x1, None) == -1
    assert L.plc_lse_merge(None, None, 0, 2, 128, None, None, None) == 0   # nothing to do
    assert L.plc_kv_append_quant(ctypes.byref(d), None, 0x1, 0x1, 4, 0x1, 0x1, 1, 5, None) == -1
    assert L.plc_kv_append_quant(ctypes.byref(d), None, None, None, 4, None, None, 1, 0, None) == 0
    assert L.plc_kv_append_quant(ctypes.byref(d), 0x1, 0x1, 0x1, 4, 0x1, 0x1, 0, 5, None) == -1


def _verify(plc, desc, hq=8, max_q=4, max_ctx=64, total=8, part=0, ws_bytes=1 << 20, ws=0x2000,
            q=0x3000):
    return plc.lib().plc_attn_verify_paged(q, hq, ctypes.byref(desc), 0x4000, 4, 0x4800, 0x5000, 2,
                                           total, max_q, max_ctx, part, 0.088, 0x6000, 0x7000, ws,
                                           ws_bytes, None)


def test_verify_validation(plc):
    d = _desc(plc)
    assert _verify(plc, d, max_q=0) == -1 and "max_q_len" in _err(plc)
    assert _verify(plc, d, max_q=plc.VERIFY_MAX_Q_LEN + 1) == -1 and "prefill" in _err(plc)
    assert _verify(plc, d, max_q=8, max_ctx=4) == -1                 # more queries than keys
    assert _verify(plc, d, part=24) == -1 and "multiple" in _err(plc)
    assert _verify(plc, d, q=None) == -1
    assert _verify(plc, d, total=0, q=None) == 0                     # nothing to do
    need = plc.verify_workspace_size(2, 8, 8, 1, 128, 4, 64, 0)
    assert need > 0
    assert _verify(plc, d, ws_bytes=need - 1) == -3 and "needed" in _err(plc)
    assert _verify(plc, _desc(plc, dtype=1, scales=False)) == -1       # E4M3 needs its scales


def test_verify_workspace_size_formula(plc):
    # 8 sequences x 4 tokens x 8 heads = 256 rows, 16 partitions of 2048;
    # 4 x 8 = 32 rows per (sequence, KV head) = 2 row groups of 16, which one
    # workgroup takes together: 8 units x 16 partitions = 128 workgroups, so
    # room for each partition streamed as two halves (32 partials per row)
    def want(rows, nparts):
        return ((rows * nparts * 128 * 4 + 255) // 256) * 256 + ((rows * nparts * 4 + 255) // 256) * 256
    assert plc.verify_workspace_size(8, 32, 8, 1, 128, 4, 32768, 2048) == want(8 * 4 * 8, 32)
    # 16 drafts: 8 row groups, two per workgroup: 8 x 4 x 16 = 512 workgroups,
    # no split
    assert plc.verify_workspace_size(8, 128, 8, 1, 128, 16, 32768, 2048) == want(8 * 16 * 8, 16)
    assert plc.verify_workspace_size(8, 32, 8, 1, 128, 0, 32768, 2048) == 0
    assert plc.verify_workspace_size(8, 32, 8, 1, 128, 17, 32768, 2048) == 0



def test_head_dim_256_entry_points(plc):
    # head dim 256 is taken by every entry point with a group of up to 16
    # query heads (six here); other widths are refused before touching memory
    d = _desc(plc, head_dim=256, hkv=2)
    assert _decode(plc, d, hq=12, ws=None) == -3                      # validation passed up to the workspace
    assert _decode(plc, d, hq=12 * 3) == -2 and "1..16" in _err(plc)  # group of 18
    assert _decode(plc, _desc(plc, head_dim=128, hkv=2), hq=12) == -2  # G = 6 needs head dim 256
    L = plc.lib()
    assert L.plc_attn_prefill_paged(None, 12, ctypes.byref(d), 0x1, 4, 0x1, 0x1, 1, 10, 10, 64,
                                    0.1, 0x1, 0x1, None) == -1      # validated up to the null q
    assert _verify(plc, d, hq=12, ws=None) == -3                      # validation passed up to the workspace
    assert _decode(plc, _desc(plc, head_dim=192)) == -2 and "head_dim" in _err(plc)


def test_misaligned_output_or_workspace_refused(plc):
    # the kernels store 16-byte vectors into out and the workspace
    d = _desc(plc)
    assert _decode(plc, d, ws=0x2004) == -1 and "aligned" in _err(plc)
    assert plc.lib().plc_attn_decode_paged(0x3000, 8, ctypes.byref(d), 0x4000, 4, 0x5000, 2, 64, 0, 0.088,
                                           0x6008, 0x7000, 0x2000, 1 << 20, None) == -1
    assert "out" in _err(plc) and "aligned" in _err(plc)
    assert _verify(plc, d, ws=0x2008) == -1 and "aligned" in _err(plc)


def test_no_alloc_refuses_more_than_its_scratch(plc):
    # 1024 sequences x 32 heads x 16 partitions of partials need ~270 MB,
    # beyond the 16 MiB scratch: refused on the host before any launch
    d = _desc(plc, hkv=4)
    L = plc.lib()
    assert L.plc_attn_decode_append_noalloc(0x3000, 0x3100, 0x3200, 32, ctypes.byref(d), 0x4000, 8192,
                                            0x5000, 1024, 131072, 8192, 0.088, 0x6000, 0x7000,
                                            None) == -3
    assert "scratch" in _err(plc) and str(16 << 20) in _err(plc)
    assert plc.NOALLOC_SCRATCH_BYTES == 16 << 20
