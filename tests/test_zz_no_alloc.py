"""The allocation-free decode entry point (rdt_decode_step_noalloc, for
callers that cannot allocate device memory) against rdt_decode_step with a
caller workspace: same inputs, same kernels, so outputs, halt counts and the
cache positions each step appends must match bit for bit.  Two calls in a
row share the library's scratch array, the second with fewer sequences; a
step whose workspace would not fit the array is refused up front."""

import numpy as np
import pytest

from workloads import configs, generate

from gpu_support import fill_cache, kv_capacity, to_np

pytestmark = pytest.mark.gpu


def _decode_pair(cfg, W, e, h0, blk):
    """rdt_decode_step with a torch workspace, then rdt_decode_step_noalloc,
    each on its own freshly seeded cache; returns both results."""
    import torch
    from recurrent_depth_moe_amd import binding
    B, n = e.shape[0], cfg["n_loops"]
    cap = kv_capacity(cfg)
    et = torch.from_numpy(np.ascontiguousarray(e)).cuda()
    ht = torch.from_numpy(np.ascontiguousarray(h0)).cuda()
    out = []
    for noalloc in (False, True):
        kv = torch.zeros(binding.kv_cache_bytes(cfg, B, cap, n), dtype=torch.uint8, device="cuda")
        for t in range(n):
            fill_cache(cfg, None, kv, t, generate.make_cache_loop(cfg, t, "k", (0, B)),
                       generate.make_cache_loop(cfg, t, "v", (0, B)))
        h_out = torch.full_like(et, float("nan"))
        halt = torch.full((B, 1), -1, dtype=torch.int32, device="cuda")
        if noalloc:
            binding.decode_step_noalloc(blk, et, ht, cfg["start_pos"], n, cfg["act_threshold"], kv, cap, h_out, halt)
        else:
            blk.decode_step(et, ht, cfg["start_pos"], n, cfg["act_threshold"], kv, cap, h_out=h_out,
                            halt_counts=halt)
        torch.cuda.synchronize()
        out.append((to_np(h_out), to_np(halt), kv.cpu().numpy()))
    return out


@pytest.mark.parametrize("name, over", [
    ("small_bf16_decode", {}),                                   # bf16: skinny GEMMs, split-KV attention, side stream
    ("small_bf16_decode", dict(act_threshold=0.99)),             # ACT on
    ("tiny_gqa", dict(start_pos=9, seq=1, batch=5)),             # fp32: generic attention
])
def test_noalloc_decode_matches_workspace_decode(name, over):
    from recurrent_depth_moe_amd import binding
    cfg = configs.get(name, **over)
    W = generate.make_weights(cfg)
    blk = binding.Block(cfg, binding.weights_to_device(W))
    for B in (cfg["batch"], max(1, cfg["batch"] - 2)):        # the second call is smaller
        c = dict(cfg, batch=B)
        e, h0 = generate.make_inputs(c)
        print(f"[noalloc] {name} {over} B={B} pos={c['start_pos']} loops={c['n_loops']}", flush=True)
        (o1, h1, kv1), (o2, h2, kv2) = _decode_pair(c, W, e, h0, blk)
        assert np.all(np.isfinite(o1))
        np.testing.assert_array_equal(o2, o1)
        np.testing.assert_array_equal(h2, h1)
        np.testing.assert_array_equal(kv2, kv1)


def test_noalloc_refuses_a_step_beyond_its_scratch():
    import torch
    from recurrent_depth_moe_amd import binding
    cfg = configs.get("small_bf16_decode")
    W = generate.make_weights(cfg)
    blk = binding.Block(cfg, binding.weights_to_device(W))
    B = 1
    while binding.workspace_bytes(cfg, B, 1) <= 32 << 20:
        B *= 2
    e = torch.zeros((B, 1, cfg["dim"]), dtype=torch.float32, device="cuda")
    cap = kv_capacity(cfg)
    kv = torch.zeros(binding.kv_cache_bytes(cfg, B, cap, cfg["n_loops"]), dtype=torch.uint8, device="cuda")
    h_out = torch.empty_like(e)
    halt = torch.empty((B, 1), dtype=torch.int32, device="cuda")
    with pytest.raises(binding.RdtError) as ex:
        binding.decode_step_noalloc(blk, e, e, cfg["start_pos"], cfg["n_loops"], 0.0, kv, cap, h_out, halt)
    assert ex.value.status == 6
    assert "scratch" in str(ex.value)
