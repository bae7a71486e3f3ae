"""bench.py's command-line contract, checked on the CPU: a request for more
than one GPU ends with a message and a non-zero status before any device
work (this build measures one GPU)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")],
                       capture_output=True, text=True, timeout=300, cwd=ROOT, env=env)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_every_recorded_kernel_has_bench_byte_figures():
    # every kernel name the library records for a call (rec_kernel in the C
    # ABI) must have algorithmic bytes in bench.py, or a --workload run that
    # launches it fails before printing its line
    import re
    sys.path.insert(0, ROOT)
    import bench
    from fft_spectral_convolution_amd.inputs import CONFIGS
    names = set()
    for fname in os.listdir(os.path.join(ROOT, "fft_spectral_convolution_amd", "csrc")):
        if fname.endswith(".hip"):
            src = open(os.path.join(ROOT, "fft_spectral_convolution_amd", "csrc", fname)).read()
            for call in re.findall(r"rec_kernel\(([^;]*?), \w+\);", src):
                names.update(re.findall(r'"([a-z0-9_]+)"', call))
    assert {"conv_fused", "fwd2d", "mix_mfma", "inv2d", "rows_fwd", "rows_inv"} <= names
    # the weight preparation of the linear convolution (zero-padding the
    # spatial kernel, turning its spectrum into a weight) runs once before
    # the timed steps, never inside them
    names -= {"pad", "spec_to_weight"}
    for name in sorted(names):
        for cfg in (CONFIGS["c1"], CONFIGS["c4"]):
            assert bench.kernel_bytes(name, cfg) > 0, name
            bench.compulsory_share(name, cfg)
