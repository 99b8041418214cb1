"""The allocation-free split decode step, h2o_decode_step_split_noalloc, against
h2o_decode_step_split through the C ABI (GPU).

Both run the same kernels with the same chunking, so every output, eviction
and cache array must be bit-identical: two caches are prefilled alike and
stepped side by side, the reference with a caller-allocated workspace and
the other on the library's own array. The calls come in a row on two shapes,
the second smaller than the first, so the second reuses an array whose
contents the first left behind.
"""
import pytest
import torch

from h2o_harness import TORCH_DTYPE, log, to_device
from kv_cache_eviction_decode_amd import H2OCache
from workload import Workload, make_decode, make_prompt

pytestmark = pytest.mark.gpu

CASES = [
    # name, B, H, d, dtype, n, k_heavy, k_recent, T, chunk_rows
    ("noalloc_larger", 2, 16, 128, "bf16", 1500, 512, 512, 5, 0),
    ("noalloc_smaller", 1, 3, 64, "f16", 300, 40, 41, 5, 64),
]


def _prefilled_pair(wl, dev):
    B, H, n, d = wl.batch, wl.heads, wl.prompt_len, wl.head_dim
    Q, K, V = (to_device(x, wl.dtype, dev).view(B, H, n, d) for x in make_prompt(wl))
    caches = []
    for _ in range(2):
        c = H2OCache(B, H, d, wl.k_heavy, wl.k_recent, TORCH_DTYPE[wl.dtype], wl.scale, dev)
        c.prefill_select(Q, K, V)
        caches.append(c)
    return caches


def test_noalloc_split_matches_split_on_two_shapes(gpu):
    dev = torch.device("cuda")
    for name, B, H, d, dt, n, kh, kr, T, chunk in CASES:
        wl = Workload(name, B, H, d, dt, n, kh, kr, T, 1.5, 0.0, seed=61)
        log(f"[no-alloc] {wl.describe()} chunk_rows={chunk}")
        ref, got = _prefilled_pair(wl, dev)
        q, k, v = (to_device(x.transpose(1, 0, 2), dt, dev).view(T, B, H, d) for x in make_decode(wl))
        out_r = torch.empty(B, H, d, dtype=torch.float32, device=dev)
        out_g = torch.full_like(out_r, float("nan"))
        ev_r = torch.empty(B, H, dtype=torch.int32, device=dev)
        ev_g = torch.full_like(ev_r, 12345)
        for t in range(T):
            ref.decode_step_split(q[t], k[t], v[t], out_r, ev_r, chunk)
            got.decode_step_split_noalloc(q[t], k[t], v[t], out_g, ev_g, chunk)
            torch.cuda.synchronize()
            assert torch.equal(out_g, out_r), f"{name} step {t}: outputs differ"
            assert torch.equal(ev_g, ev_r), f"{name} step {t}: evictions differ"
            for what in ("score", "pos", "K", "V"):
                assert torch.equal(getattr(got, what), getattr(ref, what)), f"{name} step {t}: {what} differs"
        assert got.t_next == ref.t_next == n + T
        full = n + T > wl.k
        if full:
            assert (ev_r.cpu().numpy() >= 0).all()
        log(f"[no-alloc] {name}: {T} steps bit-identical to h2o_decode_step_split")
