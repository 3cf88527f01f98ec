"""CPU: the bench's algorithmic numerators against their closed forms.

The roofline fractions divide these byte and FLOP counts by measured times, so
they are pinned here to values computed by hand from the workload shapes."""
import numpy as np

import bench
import synthetic

SPECS = synthetic.named_specs()


def test_c2_decode_bytes():
    w = synthetic.generate(SPECS["c2"])
    # KV codes 8 x 32768 tokens x 1 head x 128 x (K + V), block-table entries
    # (2048 pages per sequence), E4M3 scales (2 x 4 B), queries (fp16),
    # outputs (fp32 o and lse)
    kv = 8 * 32768 * 128 * 2
    tables = 8 * 2048 * 4
    q = 8 * 8 * 128 * 2
    outs = 8 * 8 * (128 + 1) * 4
    assert bench.decode_bytes(w, "e4m3") == kv + tables + 8 + q + outs == 67223816
    # the appended step token: fp16 K/V in (8 x 128 x 2 x 2 B), codes out, and
    # cu_q_lens / start_pos / context lengths (3 x 8 + 1 int32)
    assert bench.append_bytes(w, "e4m3") == 8 * 128 * 2 * 2 + 8 * 128 * 2 + (3 * 8 + 1) * 4


def test_c4_decode_bytes():
    w = synthetic.generate(SPECS["c4"])
    kv = (2 * 524288 + 4 * 262144) * 128 * 2
    tables = (2 * 524288 + 4 * 262144) // 16 * 4
    q = 6 * 8 * 128 * 2
    outs = 6 * 8 * 129 * 4
    assert bench.decode_bytes(w, "e4m3") == kv + tables + 8 + q + outs == 537432264


def test_c5_int8_and_fp16_bytes_follow_the_lengths():
    w = synthetic.generate(SPECS["c5"])
    L = w.context_lens.astype(np.int64)
    pages = int(((L + 15) // 16).sum())
    base = pages * 4 + 32 * 32 * 128 * 2 + 32 * 32 * 129 * 4
    assert bench.decode_bytes(w, "fp16") == int(L.sum()) * 4 * 128 * 2 * 2 + base
    assert bench.decode_bytes(w, "int8") == int(L.sum()) * 4 * (128 * 2 + 2 * 4) + base


def test_c3_prefill_flops():
    w = synthetic.generate(SPECS["c3"])
    # 4 D Hq per visible (query, key) pair: 8192 queries over a 122,880 prefix
    # plus the causal triangle of the chunk
    pairs = 8192 * 122880 + 8192 * 8193 // 2
    assert bench.prefill_flops(w) == 4 * 128 * 8 * pairs == 4260624334848


def test_d256_numerators():
    w = synthetic.generate(SPECS["d256"])
    assert bench.decode_bytes(w, "e4m3") == (8 * 32768 * 2 * 256 * 2 + 8 * 2048 * 4 + 2 * 2 * 4 +
                                             8 * 12 * 256 * 2 + 8 * 12 * 257 * 4)
    wp = synthetic.generate(SPECS["d256_prefill"])
    assert bench.prefill_flops(wp) == 4 * 256 * 12 * (8192 * 122880 + 8192 * 8193 // 2)


def test_accuracy_summary():
    ro = np.zeros((3, 2, 4), np.float32)
    rl = np.array([[0.5, 100.0], [2.0, -1.0], [0.0, 0.0]], np.float32)
    o = ro.copy()
    o[1, 1, 3] = 1.5e-3
    l = rl.copy()
    l[0, 1] += 0.02                    # 2e-4 relative at |lse| = 100
    a = bench.accuracy(o, l, ro, rl)
    assert a["rows_checked"] == 6 and abs(a["max_abs_do"] - 1.5e-3) < 1e-9
    assert abs(a["max_rel_dlse"] - 2e-4) < 1e-6 and not a["within_tolerance"]
    a = bench.accuracy(o, l, ro, rl, rows=np.array([2, 3, 4]))
    assert a["rows_checked"] == 3 and a["max_abs_do"] == np.float32(1.5e-3) and a["within_tolerance"]


def test_smi_flattening_keeps_clocks_and_power():
    sample = [{"gpu": 0, "power": {"socket_power": {"value": 612, "unit": "W"}, "gfx_voltage": "N/A"},
               "clock": {"gfx_0": {"clk": {"value": 2100, "unit": "MHz"}},
                         "mem_0": {"clk": {"value": 1900, "unit": "MHz"}}}}]
    f = bench.smi_filter(sample)
    assert f["0.power.socket_power"] == 612 and "0.clock.gfx_0.max_clk" not in f
    assert f["0.clock.gfx_0.clk"] == 2100 and f["0.clock.mem_0.clk"] == 1900
    assert "0.power.gfx_voltage" not in f
