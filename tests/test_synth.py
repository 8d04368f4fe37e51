"""The seeded generator: bf16 rounding, determinism, block-range independence."""
import numpy as np
import torch

from synth import make_workload, round_to_bf16, token_values, WORKLOADS


def test_round_to_bf16_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.01171875, -2.00390625, 0.0]   # exact ties
    vals, bits = round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16)
    assert np.array_equal(bits.view(np.int16), ref.view(torch.int16).numpy())
    assert np.array_equal(vals, ref.float().numpy())


def test_token_ranges_are_independent_of_split():
    key = (99, 0)
    whole = token_values(key, 0, 0, 3000, 2, 8, 0.5, "bf16")
    part = token_values(key, 0, 1000, 2100, 2, 8, 0.5, "bf16")
    assert np.array_equal(whole[1000:2100], part)


def test_named_workloads_structure():
    for name in WORKLOADS:
        w = make_workload(name)
        bt = w.block_table()
        used = bt[bt >= 0]
        assert len(np.unique(used)) == len(used) and used.max() < w.num_blocks
    w = make_workload("mixed_budget2048")
    assert sum(r.launch[1] for r in w.requests) == 2048
    lens = [r.n_ctx for r in w.requests[:64]]
    assert min(lens) >= 512 and max(lens) <= 8192
