"""The profile summaries bench.py writes under profiles/ (CPU, synthetic rocprofv3 CSVs):
the traffic of each decode layout is scaled by the largest copy dispatch of the run and set
against that layout's algorithmic bytes from the same run's JSON line; decode kernels are
told apart by their template arguments; SQ counts are averaged per position of the period
in dispatch order; the source hash ties a traffic summary to the kernel it was taken on."""
import csv
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

K4 = ("void pace::(anonymous namespace)::decode_kernel<128, 8, 0, 4, 1, 64, 0, true, false, false>"
      "(pace::DecodeParams, pace::(anonymous namespace)::OrderArg<false>)")
K48M = ("void pace::(anonymous namespace)::decode_kernel<128, 8, 1, 0, 1, 32, 1, true, false, false>"
        "(pace::DecodeParams, pace::(anonymous namespace)::OrderArg<false>)")
K4ORD = K4.replace("true, false, false>", "true, true, false>")
KBF = "void pace::(anonymous namespace)::decode_kernel<128, 8, 0, 4, 1, 128, 0, true, false, true>(x)"


def _write(path, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_decode_layout_from_template_arguments():
    assert bench.decode_layout(K4) == "pace4"
    assert bench.decode_layout(K48M) == "pace48-mixed"
    assert bench.decode_layout(K48M.replace("<128, 8, 1, 0", "<128, 8, 0, 0")) == "pace48-int8"
    assert bench.decode_layout(KBF) == "bf16-periodic"
    assert bench.decode_layout(K4ORD) is None              # ordered launches are not a layout leg
    assert bench.decode_layout("__amd_rocclr_copyBuffer") is None


def test_traffic_summary_per_layout(tmp_path):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    for d, c, copy_kib in ((fetch, "FETCH_SIZE", 2 * 1048576.0), (write, "WRITE_SIZE", 1048576.0)):
        rows = [dict(Dispatch_Id=1, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=c, Counter_Value=copy_kib),
                # a small copy of the same kernel name must not set the calibration
                dict(Dispatch_Id=2, Kernel_Name="__amd_rocclr_copyBuffer", Counter_Name=c, Counter_Value=64.0)]
        rows += [dict(Dispatch_Id=10 + i, Kernel_Name=K4, Counter_Name=c, Counter_Value=20000.0 + 2000.0 * (i % 2))
                 for i in range(4)]
        rows += [dict(Dispatch_Id=20, Kernel_Name=K48M, Counter_Name=c, Counter_Value=30000.0),
                 dict(Dispatch_Id=21, Kernel_Name=K4ORD, Counter_Name=c, Counter_Value=99999.0)]
        _write(os.path.join(d, "run_counter_collection.csv"), rows)
    log = tmp_path / "bench.log"
    log.write_text("[bench] noise\n" + json.dumps({
        "config": {"global_batch": 64}, "roofline": {"bytes_per_launch": 23489024},
        "variants": {"pace48-mixed": {"bytes_per_launch": 30948864}}}) + "\n")
    src = tmp_path / "k.hip"
    src.write_text("kernel source")
    out = bench.summarize_traffic(fetch, write, str(log), 1 << 30, str(src), ["cmd f", "cmd w"])
    assert sorted(out) == ["pace48-mixed_b64", "pace4_b64"]
    fields = dict(l.split(":", 1) for l in out["pace4_b64"].splitlines() if ":" in l)
    # FETCH reads twice the copy's bytes (factor 1/2), WRITE reads them once (factor 1)
    assert "factor 0.5000" in fields["copy_fetch_KiB"] and "factor 1.0000" in fields["copy_write_KiB"]
    fb, wb = float(fields["fetch_bytes_per_launch"]), float(fields["write_bytes_per_launch"])
    assert fb == pytest.approx(21000.0 * 1024 * 0.5) and wb == pytest.approx(21000.0 * 1024)
    assert float(fields["traffic_over_algorithmic"]) == pytest.approx((fb + wb) / 23489024, rel=1e-4)
    import hashlib
    assert fields["kernel_source_sha256"].strip() == hashlib.sha256(b"kernel source").hexdigest()


def test_sq_summary_per_period_position(tmp_path):
    d = str(tmp_path / "sq")
    rows = [dict(Dispatch_Id=1, Kernel_Name="prefill", Counter_Name="SQ_WAVES", Counter_Value=5)]
    for i in range(16):                                  # two periods of dP = 8
        for c, v in (("SQ_WAVES", 4096), ("SQ_INSTS_VALU", 4096 * (400 + i % 8 + (1000 if i % 8 == 7 else 0)))):
            rows.append(dict(Dispatch_Id=100 + i, Kernel_Name=K4, Counter_Name=c, Counter_Value=v))
    _write(os.path.join(d, "run_counter_collection.csv"), rows)
    txt = bench.summarize_sq(d, 8, "cmd")
    per = {int(l.split()[0]): float(l.split()[1]) for l in txt.splitlines()[4:]}
    assert per == {t: 400.0 + t + (1000.0 if t == 7 else 0.0) for t in range(8)}
