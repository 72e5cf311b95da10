"""Host-side accounting of bench.py: the algorithmic flops and bytes its roofline figures divide
by, the guard that drops stored traffic figures once a kernel source changes, and the refusal of
multi-GPU runs.  No GPU needed."""
import json
import os
import subprocess
import sys

import numpy as np

import harness
import synth

sys.path.insert(0, harness.ROOT)
import bench  # noqa: E402


def test_chunk_flops_by_hand():
    """c1: every query sees the 2072 persistent keys, 2 x 4680 history keys and the whole
    current chunk (causal block = chunk): 4 H D n (P + W n + n)."""
    w = synth.get_workload("c1")
    n = w.chunk
    assert bench.attention_flops(w) == 4.0 * 24 * 128 * n * (2072 + 2 * n + n)
    # c4: frame-causal blocks of 3120 inside a 9360-token chunk
    w4 = synth.get_workload("c4")
    vis = sum(2072 + 2 * 9360 + 3120 * (b + 1) for b in range(3)) * 3120
    assert bench.attention_flops(w4) == 4.0 * 32 * 128 * vis


def test_decoder_flops_by_hand():
    """d1: 10 windows of 512 rows over 5 + 3 x 512 keys, 5 windows of 416 rows over 5 + 3 x 416,
    and 5 global rows over 5 + 7200 keys, 16 heads x 128."""
    w = synth.get_decoder_workload("d1")
    f_win, f_glob = bench.decoder_flops(w)
    assert f_win == 4.0 * 16 * 128 * (10 * 512 * 1541 + 5 * 416 * (5 + 3 * 416))
    assert f_glob == 4.0 * 16 * 128 * 5 * (5 + 7200)
    assert bench.global_bytes(w) == 2 * 16 * 128 * (2 * (5 + 7200) + 2 * 5)


def test_append_bytes_by_hand():
    w = synth.get_workload("c1")
    pages = -(-4680 // 128)
    assert bench.append_bytes(w) == 2 * 24 * 128 * 2 * (4680 + pages * 128)
    kpage = 13312  # MXFP6 keys of one 128-token page at D = 128: 4 blocks x 3200 B, whole KiB
    assert bench.append_bytes(w, mx=True) == 2 * 24 * 128 * 2 * 4680 + 24 * pages * (kpage + 128 * 128)


def test_traffic_guard(tmp_path, monkeypatch):
    """A stored traffic figure is reported only while the kernel source it was measured on is
    unchanged."""
    if bench.measured_traffic("c1") is not None:
        t = bench.TRAFFIC["c1"]
        assert bench.measured_traffic("c1") == (2.0 * t["fetch_kib"] + t["write_kib"]) * 1024.0
    edited = tmp_path / "attention.hip"
    edited.write_bytes(open(bench.ATTENTION_SRC, "rb").read() + b"\n")
    monkeypatch.setattr(bench, "ATTENTION_SRC", str(edited))
    assert bench.measured_traffic("c1") is None and bench.measured_traffic("d1") is None
    assert bench.measured_traffic("no-such-workload") is None


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(harness.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]


def test_peaks():
    assert abs(bench.PEAK_BF16_TFLOPS - 256 * 4096 * 2.4e9 / 1e12) < 0.1
    assert abs(bench.PEAK_MX_TFLOPS - 2.0 / (1.0 / 10100.0 + 1.0 / 5000.0)) < 0.1
    assert bench.PEAK_HBM_GBS == 8000.0 and np.isclose(bench.PEAK_F32_TFLOPS, 157.3)


def test_attention_bytes_by_hand():
    """c1: Q and O (4680 x 24 x 128 bf16 each) once, K and V of the 16112 visible keys once."""
    w = synth.get_workload("c1")
    assert bench.attention_bytes(w) == 2 * 24 * 128 * (2 * 4680 + 2 * 16112)
    assert abs(bench.attention_bytes(w) / 1e6 - 255.5) < 0.1


def test_counter_csv_means(tmp_path):
    """--counters averages each counter over the dispatches of the named kernel only, and the
    dispatch durations from the timestamps."""
    head = ('"Correlation_Id","Dispatch_Id","Agent_Id","Queue_Id","Process_Id","Thread_Id","Grid_Size","Kernel_Id",'
            '"Kernel_Name","Workgroup_Size","LDS_Block_Size","Scratch_Size","VGPR_Count","Accum_VGPR_Count","SGPR_Count",'
            '"Counter_Name","Counter_Value","Start_Timestamp","End_Timestamp"')
    rows = [(1, "void sr::chunk_attention_kernel<G>(A)", "FETCH_SIZE", 100.0, 1000, 3000),
            (2, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 131072.0, 5000, 6000),
            (3, "void sr::chunk_attention_kernel<G>(A)", "FETCH_SIZE", 300.0, 7000, 11000)]
    p = tmp_path / "p_counter_collection.csv"
    p.write_text(head + "\n" + "\n".join(
        f'{d},{d},"Agent 1",1,1,1,1,1,"{k}",512,0,0,0,0,0,"{c}",{v},{s},{e}' for d, k, c, v, s, e in rows) + "\n")
    means, dur, n = bench._counter_means(str(p), "chunk_attention_kernel")
    assert means == {"FETCH_SIZE": 200.0} and dur == 3000.0 and n == 2
    means, dur, n = bench._counter_means(str(p), bench.COPY_KERNEL)
    assert means == {"FETCH_SIZE": 131072.0} and n == 1


def test_counter_passes_fit_the_hardware():
    """Each pass holds at most 8 SQ, 4 TCC (FETCH_SIZE uses 3, WRITE_SIZE 2) and 2 GRBM counters."""
    tcc_cost = {"FETCH_SIZE": 3, "WRITE_SIZE": 2}
    for name, ctrs in bench.COUNTER_PASSES:
        assert sum(c.startswith("SQ_") for c in ctrs) <= 8, name
        assert sum(tcc_cost.get(c, 1) for c in ctrs if c.startswith("TCC_") or c in tcc_cost) <= 4, name
        assert sum(c.startswith("GRBM_") for c in ctrs) <= 2, name
