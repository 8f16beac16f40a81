"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic byte counts the roofline
divides by, and the HBM-traffic summary written from rocprofv3 counter files and read back."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import kvsynth  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert r.stdout.strip() == ""                      # no JSON line
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def test_algorithmic_bytes_per_unit():
    """Per kept token-head: 512 B of fp16 K+V rows, 256 B of int8 codes, 64 B of fp16 scales,
    for encode (in) and decode (out); the scorer reads 256 B per token-head of K. Positions and
    the rotary table are counted once per launch."""
    w = kvsynth.workload(1)
    n = 13108
    b = bench.algorithmic_bytes(w, n)
    kept = w.compressed_layers * w.kv_heads * n
    extra = w.compressed_layers * n * 4 + w.tokens * 512
    assert b["encode"] == kept * 832 + extra
    assert b["decode"] == kept * 832 + extra
    assert b["score_evict"] == (w.compressed_layers * w.kv_heads * w.tokens * 256
                                + w.compressed_layers * w.tokens * 16 + w.compressed_layers * n * 4)
    # the totals quoted for this workload: ~4.95 GB for scoring + encode, 2.81 GB for decode
    assert abs(b["score_evict"] + b["encode"] - 4.949e9) / 4.949e9 < 0.01
    assert abs(b["decode"] - 2.810e9) / 2.810e9 < 0.001


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for k, c, v in rows:
            f.write(f'"{k}",{c},{v}\n')


def test_traffic_summary_round_trip(tmp_path, monkeypatch):
    """Counters are scaled by what a copy of known size reads; per-phase sums are written with
    the source hash and read back; a different hash reads as absent."""
    w = kvsynth.workload(1)
    out = tmp_path / "traffic.md"
    monkeypatch.setattr(bench, "traffic_path", lambda _w, decode_step=False: str(out))
    copy = bench.COPY_KERNEL
    # the copy of 1 MiB reads 512 KiB by FETCH_SIZE (factor 2) and 1024 KiB by WRITE_SIZE
    _counter_csv(tmp_path / "f", [(copy, "FETCH_SIZE", 512),
                                  ("nq::k_encode(nq::CodecArgs)", "FETCH_SIZE", 100),
                                  ("nq::k_encode(nq::CodecArgs)", "FETCH_SIZE", 300),
                                  ("nq::k_decode(nq::CodecArgs)", "FETCH_SIZE", 50),
                                  ("nq::k_decode_reset(unsigned int*, long, unsigned int*)",
                                   "FETCH_SIZE", 1),
                                  ("void nq::k_select_reg<32>(double const*, int, int, int, int*)",
                                   "FETCH_SIZE", 7),
                                  ("other::kernel()", "FETCH_SIZE", 999)])
    _counter_csv(tmp_path / "w", [(copy, "WRITE_SIZE", 1024),
                                  ("nq::k_encode(nq::CodecArgs)", "WRITE_SIZE", 40),
                                  ("nq::k_decode(nq::CodecArgs)", "WRITE_SIZE", 60),
                                  ("nq::k_decode_reset(unsigned int*, long, unsigned int*)",
                                   "WRITE_SIZE", 3)])

    class A:
        summarize_pmc = (str(tmp_path / "f"), str(tmp_path / "w"))
        copy_calibration = 1
        pmc_command = "(test)"
    bench.summarize_pmc(A, w)
    assert bench.read_traffic(str(out), "encode") == (200 * 2 + 40) * 1024
    assert bench.read_traffic(str(out), "decode") == ((50 + 1) * 2 + 60 + 3) * 1024
    assert bench.read_traffic(str(out), "score_evict") == 7 * 2 * 1024
    txt = out.read_text().replace(bench.kernel_source_hash(), "0" * 16)
    out.write_text(txt)
    assert bench.read_traffic(str(out), "encode") is None
    assert bench.read_traffic(str(tmp_path / "missing.md"), "encode") is None


def test_decode_step_traffic_and_copy_calibration(tmp_path, monkeypatch):
    """The fused decode step's summary sums its own kernels; the calibration uses the largest
    copy dispatch (the runtime's copy kernel also stages smaller input uploads)."""
    w = kvsynth.workload(2)
    out = tmp_path / "ds.md"
    seen = []
    monkeypatch.setattr(bench, "traffic_path",
                        lambda _w, decode_step=False: seen.append(decode_step) or str(out))
    copy = bench.COPY_KERNEL
    _counter_csv(tmp_path / "f", [(copy, "FETCH_SIZE", 3), (copy, "FETCH_SIZE", 512),
                                  ("void nq::k_decode_attend<4>(nq::FusedArgs)", "FETCH_SIZE", 80),
                                  ("void nq::k_decode_attend_merge<4>(nq::FusedArgs)",
                                   "FETCH_SIZE", 4),
                                  ("nq::k_decode(nq::CodecArgs)", "FETCH_SIZE", 999)])
    _counter_csv(tmp_path / "w", [(copy, "WRITE_SIZE", 1), (copy, "WRITE_SIZE", 1024),
                                  ("void nq::k_decode_attend<4>(nq::FusedArgs)", "WRITE_SIZE", 6),
                                  ("nq::k_decode_reset(unsigned int*, long, unsigned int*)",
                                   "WRITE_SIZE", 2)])

    class A:
        summarize_pmc = (str(tmp_path / "f"), str(tmp_path / "w"))
        copy_calibration = 1
        pmc_command = "(test)"
    bench.summarize_pmc(A, w, decode_step=True)
    assert seen == [True]
    assert bench.read_traffic(str(out), "decode_attend") == ((80 + 4) * 2 + 6 + 2) * 1024
    assert bench.read_traffic(str(out), "encode") is None
