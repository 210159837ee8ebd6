"""Host-side parts of bench.py that need no GPU: the one-GPU refusal and the
profile summaries it writes from rocprofv3 output."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_stats_summary_names_kernels(tmp_path):
    csv = tmp_path / "run_kernel_stats.csv"
    csv.write_text(
        '"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n'
        '"void (anonymous namespace)::split16_kernel<1, true, false>(SplitArgs)",10,1000000,100000,50,90000,'
        '110000,1\n'
        '"void (anonymous namespace)::combine_kernel<16>(float const*)",10,200000,20000,10,19000,21000,1\n'
        '"void (anonymous namespace)::wide_kernel<3, false>(SplitArgs)",2,400000,200000,20,190000,210000,1\n'
        '"void at::native::vectorized_elementwise_kernel<4>(int)",5,100,20,1,10,30,1\n')
    out = tmp_path / "kernel_stats_x.txt"
    bench.summarize_stats("x", str(csv), str(out), "--only layer --workload 3")
    text = out.read_text()
    assert "split16_kernel<1> paged" in text
    assert "combine_kernel<16>" in text
    assert "wide_kernel<3>" in text
    assert "at::" not in text
    assert "--only layer --workload 3" in text
    rows = [l for l in text.splitlines() if not l.startswith("#")][1:]
    assert rows[0].startswith("split16_kernel<1> paged")  # sorted by total time


def _counter_csv(path, counter, partial_kib, copy_kib):
    lines = ['"Dispatch_Id","Kernel_Name","Counter_Name","Counter_Value"']
    # two partial dispatches whose counter is split over two instances each
    for d, v in ((1, partial_kib), (2, partial_kib)):
        lines.append(f'{d},"void (anonymous namespace)::split16_kernel<2, false, false>(SplitArgs)",'
                     f'"{counter}",{v / 2}')
        lines.append(f'{d},"void (anonymous namespace)::split16_kernel<2, false, false>(SplitArgs)",'
                     f'"{counter}",{v / 2}')
    lines.append(f'3,"__amd_rocclr_copyBuffer","{counter}",{copy_kib}')
    lines.append(f'4,"__amd_rocclr_copyBuffer","{counter}",{copy_kib}')
    lines.append(f'5,"__amd_rocclr_copyBuffer","{counter}",1.0')  # a small copy, ignored
    path.write_text("\n".join(lines) + "\n")


def test_pmc_summary_scales_by_the_copy(tmp_path):
    from mla_latent_kv_cache_amd import workloads as W
    fetch, write = tmp_path / "f.csv", tmp_path / "w.csv"
    # the copy reads 1 GiB as 524288 KiB of FETCH_SIZE (factor 2) and writes it as 1048576 KiB (factor 1)
    _counter_csv(fetch, "FETCH_SIZE", 300000.0, 524288.0)
    _counter_csv(write, "WRITE_SIZE", 20000.0, 1048576.0)
    out = tmp_path / "pmc.txt"
    bench.summarize_pmc(2, None, None, 0, str(fetch), str(write), str(out))
    text = out.read_text()
    vals = dict(l.split(": ", 1) for l in text.splitlines() if l and not l.startswith("#"))
    assert float(vals["copy_fetch_factor"]) == pytest.approx(2.0)
    assert float(vals["copy_write_factor"]) == pytest.approx(1.0)
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx(300000.0 * 1024 * 2 + 20000.0 * 1024)
    w = W.WORKLOADS[2]
    algo = (W.lengths(2) + 1).sum() * bench.row_bytes(w.fmt)
    assert float(vals["algorithmic_bytes_per_launch"]) == pytest.approx(algo)
    assert vals["kernel_source_sha256_16"] == bench.kernel_sha()
    assert vals["partial_dispatches"] == "2"
