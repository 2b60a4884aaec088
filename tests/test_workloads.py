"""Host checks of the seeded input generator (no GPU)."""
import numpy as np
import torch

from flash_attention_transformers_amd import workloads as W


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000, dtype=np.float32) * 7
    x[:4] = [1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 65504.0]  # ties to even
    bits = W.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)


def test_inputs_are_seeded_and_ordered():
    w = W.WORKLOADS["tiny_mha_f32"]
    a, b = W.make_inputs(w), W.make_inputs(w)
    for n in ("q", "k", "v", "do"):
        np.testing.assert_array_equal(a.vals[n], b.vals[n])
    rng = np.random.default_rng(w.seed)
    np.testing.assert_array_equal(a.vals["q"], rng.standard_normal((1, 2, 128, 64), dtype=np.float32))


def test_dit_self_qk_multiplier_before_rounding():
    w = W.WORKLOADS["dit_self"].with_shape(Sq=64, Skv=64, Hq=1, Hkv=1)
    inp = W.make_inputs(w)
    rng = np.random.default_rng(w.seed)
    q = rng.standard_normal((1, 1, 64, 128), dtype=np.float32) * np.float32(1 / np.sqrt(2))
    np.testing.assert_array_equal(inp.bits["q"], W.round_to_bf16_bits(q))


def test_credited_flops():
    w = W.WORKLOADS["gqa_causal"]
    assert w.fwd_flop() == 4 * 4 * 32 * 4096 * 4096 * 128 / 2
    assert w.bwd_flop() == 2.5 * w.fwd_flop()
    assert W.WORKLOADS["dit_self"].fwd_flop() == 4 * 10 * 32760 ** 2 * 128


def test_bench_roofline_kernels_have_sources():
    # Every kernel the bench line can name has a source entry, so a committed
    # counter summary for it can be matched against the current source.
    import bench

    for dtype in ("bf16", "f32"):
        for stage in ("fwd", "dkdv", "dq"):
            assert bench.roofline_kernel(stage, dtype) in bench.KERNEL_SOURCES
    assert bench.roofline_kernel("fwd", "bf16") == "fwd_bf16_kernel"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; asking for more exits with a message, before
    touching any GPU."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
