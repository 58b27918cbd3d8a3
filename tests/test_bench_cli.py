"""Host-side checks of bench.py: the multi-GPU request is refused with a message (the path is
one GPU's share), and the algorithmic work table counts what the design notes state."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_work_matches_the_stated_bytes_and_flops():
    import bench
    T, H, I, k, El, E = 4096, 2048, 768, 8, 128, 128
    R = T * k
    b, f = bench.kernel_work("bwd_dWgu", T, H, I, k, R, El, E)
    assert b == R * (2 * H + 4 * I) + El * 4 * H * I        # Xp + dG|dU + dW_gate|dW_up
    assert f == 4.0 * R * H * I
    b, f = bench.kernel_work("fwd_gateup", T, H, I, k, R, El, E)
    assert b == R * 2 * H + El * 4 * H * I + R * 6 * I       # Xp + W_gate|W_up + G|U + A
    b, f = bench.kernel_work("router_logits", T, H, I, k, R, El, E)
    assert f == 2.0 * T * H * E
    assert bench.kernel_work("no_such_kernel", T, H, I, k, R, El, E) == (0.0, 0.0)
