"""The seeded synthetic generator: determinism, slicing, rounding, structure (CPU only)."""
import numpy as np
import pytest

from workload import WORKLOADS, Workload, make_decode, make_prompt, round_to_dtype, unit_vector


def test_named_workloads_shapes():
    w = WORKLOADS["opt6.7b_layer"]
    assert (w.batch, w.heads, w.head_dim, w.dtype, w.prompt_len, w.k, w.steps) == \
        (64, 32, 128, "bf16", 1024, 256, 512)
    assert WORKLOADS["opt30b_layer"].k == 410 and WORKLOADS["opt30b_layer"].sink == 4.0
    assert WORKLOADS["long_context"].alpha == 1.2 and WORKLOADS["long_context"].k == 2048
    assert WORKLOADS["large_batch_f16"].dtype == "f16"
    assert WORKLOADS["tiny_f32"].dtype == "f32" and WORKLOADS["tiny_f32"].head_dim == 64


def test_subset_and_prefix_are_slices_of_full_generation():
    wl = Workload("t", 2, 3, 16, "bf16", 20, 4, 4, 12, 1.5, 4.0, 3)
    Q, K, V = make_prompt(wl)
    q, k, v = make_decode(wl)
    Qs, Ks, Vs = make_prompt(wl, heads=[4, 1])
    qs, ks, vs = make_decode(wl, heads=[4, 1], steps=5)
    for full, sub in [(Q, Qs), (K, Ks), (V, Vs)]:
        assert np.array_equal(full[[4, 1]], sub)
    for full, sub in [(q, qs), (k, ks), (v, vs)]:
        assert np.array_equal(full[[4, 1], :5], sub)
    Q2, _, _ = make_prompt(wl)
    assert np.array_equal(Q, Q2)
    Q3, _, _ = make_prompt(wl, seed=4)
    assert not np.array_equal(Q, Q3)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_rounding_is_exact_in_dtype(dtype):
    import torch
    x = np.random.default_rng(0).standard_normal(10000).astype(np.float32) * 3
    r = round_to_dtype(x, dtype)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    back = torch.from_numpy(r).to(tdt).to(torch.float32).numpy()
    assert np.array_equal(back, r)  # representable
    ref = torch.from_numpy(x).to(tdt).to(torch.float32).numpy()
    assert np.array_equal(ref, r)   # same rounding as torch (round to nearest even)


def test_structure_of_keys_and_queries():
    wl = Workload("s", 1, 64, 64, "f32", 256, 8, 8, 4, 1.5, 4.0, 9)
    u = unit_vector(wl)
    assert abs(np.linalg.norm(u) - 1) < 1e-6
    Q, K, _ = make_prompt(wl)
    # query mean along u is 2, key coefficient along u is noise + clipped Pareto in [1, 4]
    assert abs((Q @ u).mean() - 2.0) < 0.05
    proj = K[:, 1:] @ u
    assert 1.0 < proj.mean() < 4.0
    # position 0 carries the sink offset 4u on top of the Pareto coefficient
    assert (K[:, 0] @ u).mean() > proj.mean() + 3.0
