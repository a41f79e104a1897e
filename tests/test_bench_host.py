"""bench.py's host logic, without a GPU: the metric strings of each line, the
FLOP counts, the committed traffic summary lookup and the digest it is keyed
on, and the refusal of more than one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import fa_inputs as fi  # noqa: E402


def test_metric_strings_name_their_workload():
    assert bench.metric_for(2, 32, 8192, 128, fi.BF16, False) == bench.METRIC
    assert bench.metric_for(4, 16, 2048, 64, fi.F16, True) == \
        "attention fwd TFLOP/s + % of MFMA peak (d=64, N=2048, f16, causal)"
    assert bench.metric_for(4, 16, 8192, 128, fi.FP8_E4M3, False) == \
        "attention fwd TFLOP/s + % of MFMA peak (d=128, N=8192, fp8_e4m3)"
    assert bench.metric_bwd_for(128, 8192, fi.BF16, True).endswith("(d=128, N=8192, bf16, causal)")
    assert len({bench.metric_for(*w[:6]) for w in bench.WORKLOADS.values()}) == len(bench.WORKLOADS)


def test_flop_counts():
    # forward: two products of 2*N*N*d each per head, halved by the causal mask
    assert bench.attention_flops(2, 32, 8192, 128, False) == 4 * 2 * 32 * 8192 ** 2 * 128
    assert bench.attention_flops(2, 32, 8192, 128, True) == 2 * 2 * 32 * 8192 ** 2 * 128
    # backward: five products
    assert bench.backward_flops(2, 32, 8192, 128, False) == 10 * 2 * 32 * 8192 ** 2 * 128
    assert bench.backward_flops(2, 32, 8192, 128, True) == 5 * 2 * 32 * 8192 ** 2 * 128


def test_traffic_summary_follows_the_kernel_source(tmp_path, monkeypatch):
    # the committed summary is read while its digest matches the source ...
    t = bench.read_traffic(bench.DEFAULT)
    assert t is None or abs(t / bench.algorithmic_bytes(2, 32, 8192, 128, 2, 2) - 1.0) < 0.05
    # ... and ignored once the source no longer matches
    monkeypatch.setattr(bench, "source_digest", lambda: "0000000000000000")
    assert bench.read_traffic(bench.DEFAULT) is None


def test_digest_covers_the_shared_header(monkeypatch, tmp_path):
    # bench.py and the summary writer agree on the forward kernel's digest ...
    import profile_summary
    assert bench.source_digest() == profile_summary.source_digest("fa_fwd_kernel")
    # ... and it changes with fa_common.h, which the kernel sources include
    csrc = tmp_path / "csrc"
    csrc.mkdir()
    src = os.path.join(ROOT, "io_aware_softmax_fa_amd", "csrc")
    for name in ("fa_fwd.hip", "fa_common.h"):
        (csrc / name).write_bytes(open(os.path.join(src, name), "rb").read())
    monkeypatch.setattr(bench, "KERNEL_SOURCE", str(csrc / "fa_fwd.hip"))
    before = bench.source_digest()
    assert before == profile_summary.source_digest("fa_fwd_kernel")
    (csrc / "fa_common.h").write_bytes((csrc / "fa_common.h").read_bytes() + b"\n")
    assert bench.source_digest() != before


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_coissue_probe_rejects_bad_arguments_before_any_launch():
    """The co-issue probe's argument checks run on the host: no GPU needed."""
    import ctypes
    from io_aware_softmax_fa_amd import build as fab
    if not os.path.exists(fab.PROBE_OUT):
        import pytest
        pytest.skip("probe library not built")
    probe = ctypes.CDLL(fab.PROBE_OUT)
    f = probe.fa_probe_coissue
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    fake = ctypes.c_void_p(16)   # never dereferenced: every call below returns first
    assert f(None, 1, 8, 0, 2, None) == -1
    assert f(fake, 0, 8, 0, 2, None) == -1
    assert f(fake, 1, 7, 0, 2, None) == -1          # iters not a multiple of 8
    assert f(fake, 1, 8, 0, 3, None) == -2          # (op, K) not built
    assert f(fake, 1, 8, 9, 1, None) == -2
    assert {(op, k) for op, k, _, _ in bench.COISSUE} == {
        (0, 2), (0, 4), (0, 8), (1, 2), (1, 4), (2, 1), (2, 2), (2, 3)}


def test_fp8_ceiling_probe_rejects_bad_arguments_before_any_launch():
    import ctypes
    from io_aware_softmax_fa_amd import build as fab
    if not os.path.exists(fab.PROBE_OUT):
        import pytest
        pytest.skip("probe library not built")
    f = ctypes.CDLL(fab.PROBE_OUT).fa_probe_mfma_fp8
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    fake = ctypes.c_void_p(16)   # never dereferenced: every call below returns first
    assert f(None, 1, 8, None) == -1
    assert f(fake, -1, 8, None) == -1
    assert f(fake, 1, 12, None) == -1


def test_16x16x32_ceiling_probe_rejects_bad_arguments_before_any_launch():
    import ctypes
    from io_aware_softmax_fa_amd import build as fab
    if not os.path.exists(fab.PROBE_OUT):
        import pytest
        pytest.skip("probe library not built")
    f = ctypes.CDLL(fab.PROBE_OUT).fa_probe_mfma16
    f.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    fake = ctypes.c_void_p(16)   # never dereferenced: every call below returns first
    assert f(None, 1, 8, None) == -1
    assert f(fake, 0, 8, None) == -1
    assert f(fake, 1, 0, None) == -1
    assert f(fake, 1, 12, None) == -1
