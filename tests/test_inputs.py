"""The seeded workload generator: shapes, determinism, planted structure (CPU only)."""

import torch

from differentiable_adaptive_block_amd import inputs


def test_prefill_is_deterministic_and_shaped():
    a = inputs.make_prefill(1, 2, 256, 32, "bf16", True, (1, 3), seed=5)
    b = inputs.make_prefill(1, 2, 256, 32, "bf16", True, (1, 3), seed=5)
    for key in ["q", "k", "v", "dout"]:
        assert a[key].shape == (1, 2, 256, 32) and a[key].dtype == torch.bfloat16
        assert torch.equal(a[key], b[key])
    c = inputs.make_prefill(1, 2, 256, 32, "bf16", True, (1, 3), seed=6)
    assert not torch.equal(a["q"], c["q"])


def test_planted_queries_lean_toward_earlier_blocks():
    w = inputs.make_prefill(1, 1, 1024, 64, "fp32", True, (1, 1), seed=1)
    q, k = w["q"][0, 0].double(), w["k"][0, 0].double()
    kb = k.view(16, 64, 64).mean(1)
    unit = kb / kb.norm(dim=1, keepdim=True)
    s = q @ unit.T  # [T, nb]
    for i in range(64, 1024, 97):
        c = i // 64
        # one planted earlier block: it has the largest alignment, and it lies before the row's block
        assert int(s[i, :c].argmax()) == int(s[i].argmax()) or s[i, :c].max() > 0.7


def test_decode_shapes():
    w = inputs.make_decode(2, 2, 256, 32, "bf16", (1, 2), seed=3)
    assert w["q"].shape == (2, 2, 32) and w["k"].shape == (2, 2, 256, 32)


def test_named_configs_exist():
    for name in ["tiny512", "tiny512_sc16", "prefill16k", "prefill64k", "prefill64k_sc7", "decode96k", "decode96k_sc5", "train16k"]:
        assert name in inputs.CONFIGS
