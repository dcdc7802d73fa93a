"""bench.py's command line on the CPU: the path runs on one GPU, so a request for
several GPUs (or a launch with several ranks) ends with a message and status 2
before anything touches a device."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(args, env=None):
    e = dict(os.environ)
    e.update(env or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, env=e, timeout=300)


def test_several_gpus_are_refused_with_a_message():
    r = _bench(["--gpus", "2", "--steps", "1", "--warmup", "0"])
    assert r.returncode == 2, r.stdout
    assert "one GPU" in r.stdout and "not supported" in r.stdout


def test_several_ranks_are_refused_with_a_message():
    r = _bench(["--steps", "1", "--warmup", "0"], env={"WORLD_SIZE": "2", "RANK": "0", "LOCAL_RANK": "0"})
    assert r.returncode == 2, r.stdout
    assert "one GPU" in r.stdout


def test_reused_activations_equal_full_draws():
    """The bench draws the prefill activations once and reuses them for the
    LayerNorm and headwise prefill workloads, whose draws are the same; what it
    hands those legs must equal their own full draws (checked on 64 tokens)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import bench
    from layerwise_qk_norm_amd import inputs
    cache = {}
    bench.host_inputs(inputs.PREFILL.with_T(64), cache)
    for w in (inputs.LN_PREFILL, inputs.HW_PREFILL, inputs.PREFILL_E4M3, inputs.GQA):
        got, want = bench.host_inputs(w.with_T(64), cache), inputs.make_host(w.with_T(64))
        assert sorted(got) == sorted(want)
        for key in got:
            assert np.array_equal(got[key], want[key]), (w.name, key)
