"""Host-side checks of bench.py's command-line contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_attended_pairs_matches_a_direct_count():
    """The bench's exact pair count (own block causal plus min(c, K) history
    blocks of b keys) against a loop over a small shape."""
    sys.path.insert(0, ROOT)
    import bench
    N, block, topk, Hq, B = 200, 16, 3, 2, 1
    want = 0
    for t in range(N):
        c = t // block
        want += (t % block + 1) + block * (c if topk is None else min(c, topk))
    assert bench.attended_pairs(N, block, topk, Hq, B) == want * Hq * B
    full = sum((t % block + 1) + block * (t // block) for t in range(N))
    assert bench.attended_pairs(N, block, None, Hq, B) == full * Hq * B
