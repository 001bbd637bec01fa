"""The benchmark's command-line contract that needs no GPU: more than one
GPU is refused with a message (this library runs on one GPU), before any
GPU or torch work; the byte accounting of the step matches the record
layouts."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), (["--gpus", "8", "--steps", "1"], {}), ([], {"WORLD_SIZE": "4"})):
        r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                           timeout=120, env={**os.environ, **env})
        assert r.returncode == 2, (args, env, r.stdout, r.stderr)
        assert "one GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_element():
    sys.path.insert(0, ROOT)
    import bench
    # reads and writes of each kernel, from the record layouts: bf16 tensors
    # 2 B/element, bit-planes and masks 1/8, NVFP4 scale bytes 1/16
    assert bench.BYTES_PER_ELEM == {"tensor_scale": 2.0, "capture": 2.1875, "guided_fwd": 4.3125,
                                    "rne_fwd": 4.1875, "ste_bwd": 4.125}
    assert bench.NEXT_BYTES_PER_ELEM["capture_codes"] == 2.6875
    assert bench.NEXT_BYTES_PER_ELEM["full_info_fwd"] == 4.6875
    assert bench.MOE_BYTES_PER_ELEM["gather_records"] == 0.375
