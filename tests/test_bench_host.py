"""Host-side logic of bench.py (no GPU): the byte counts behind the roofline, the
one-GPU guard and the counter-summary reader."""
import os
import subprocess
import sys

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_call_bytes_match_the_hand_count():
    # x once, phi once (fp32), alpha, bias; hIn, hPost, hRes; invRms, hMix, hPre and
    # 2*20 Sinkhorn planes of sums and matrices, for T=16384, n=4, D=7168
    T, n, D, M, it = 16384, 4, 7168, 24, 20
    K = n * D
    want = (T * 2 * K + M * K * 4 + 3 * 4 + M * 4 + T * D * 2 + T * n * 4 + T * n * n * 4
            + T * (4 + 4 * M + 4 * n) + 2 * it * T * (4 * n + 4 * n * n))
    assert bench.algorithmic_bytes(synth.WORKLOADS["large_prefill_bwd"], intermediates=True) == want
    assert want == 1_232_797_804


def test_stage_bytes_cover_the_call():
    # the kernels' own counts add up to the call's, plus one more read of x by the hIn
    # kernel (without pre_mix), plus alpha and bias (tiny; read by the epilogue)
    for name, wl in synth.WORKLOADS.items():
        stages = sum(bench.stage_bytes(wl, s) for s in ("projection", "epilogue", "hin"))
        call = bench.algorithmic_bytes(wl, intermediates=wl.need_backward)
        extra_x = 0 if wl.pre_mix else wl.T * 2 * wl.K
        gamma = wl.K * 4 if wl.gamma else 0
        assert stages - extra_x + wl.n_alpha * 4 + wl.M * 4 + gamma == call, name


def test_single_read_stage_bytes_cover_the_call():
    # on the single-read path x is read once: the projection stage reads x and writes hIn,
    # the hIn stage moves nothing
    for name, wl in synth.WORKLOADS.items():
        if wl.pre_mix:
            continue
        stages = sum(bench.stage_bytes(wl, s, True) for s in ("projection", "epilogue", "hin"))
        call = bench.algorithmic_bytes(wl, intermediates=wl.need_backward)
        gamma = wl.K * 4 if wl.gamma else 0
        assert bench.stage_bytes(wl, "hin", True) == 0
        assert stages + wl.n_alpha * 4 + wl.M * 4 + gamma == call, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_counter_summary_reader(tmp_path, monkeypatch):
    # missing file -> None; stale source hash -> None; matching hash -> scaled bytes
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    (tmp_path / "profiles").mkdir()
    assert bench.counter_traffic("proj_kernel", "w")[0] is None
    for rel in bench.KERNEL_SOURCES:
        p = tmp_path / rel
        p.parent.mkdir(parents=True, exist_ok=True)
        p.write_text("kernel v1")
    sha = bench.kernel_source_sha()
    f = tmp_path / "profiles" / "proj_kernel_w_counters.md"
    body = ("source_sha256: {}\nfetch_kib_per_dispatch: 2048\nwrite_kib_per_dispatch: 1024\n"
            "fetch_factor: 2.0\nwrite_factor: 1.0\n")
    f.write_text(body.format(sha))
    traffic, src = bench.counter_traffic("proj_kernel", "w")
    assert traffic == 1024 * 1024 + 1024 * 1024
    f.write_text(body.format("0" * 64))
    assert bench.counter_traffic("proj_kernel", "w")[0] is None
