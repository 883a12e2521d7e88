"""Host-side checks of the C ABI (no GPU): the library loads, exports every
function include/rdt.h declares, and rejects bad arguments before any HIP
call."""

import ctypes
import os
import re

import pytest

from workloads import configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "recurrent_depth_moe_amd", "librdt.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="librdt.so not built (run __graft_entry__.build())")


def _declared():
    src = open(os.path.join(ROOT, "include", "rdt.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(rdt_[A-Za-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    names = _declared()
    assert len(names) >= 18
    for n in names:
        assert hasattr(L, n), n
    assert L.rdt_abi_version() == 1


def _cfg(name="tiny_gqa", **kw):
    from recurrent_depth_moe_amd import binding
    c = binding.make_config(configs.get(name))
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _status(fn, *args):
    from recurrent_depth_moe_amd import binding
    return fn(*args)


@pytest.mark.parametrize("field,value", [
    ("dim", 0), ("dim", 250), ("n_kv_heads", 3), ("head_dim", 31), ("top_k", 0), ("top_k", 9),
    ("n_experts", 0), ("lora_rank", 0), ("lora_rank", 64), ("loop_dim", 6), ("loop_dim", 300),
    ("max_seq_len", 0), ("norm_eps", 0.0), ("weight_dtype", 7), ("attn", 5)])
def test_bad_config_rejected(field, value):
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    c = _cfg(**{field: value})
    st = L.rdt_check_config(ctypes.byref(c))
    assert st in (1, 2), (field, value, st)
    assert L.rdt_last_error()


def test_unsupported_combinations():
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    c = _cfg("small_bf16", head_dim=64, n_heads=8)       # bf16 attention is built for d=128
    assert L.rdt_check_config(ctypes.byref(c)) == 2
    c = _cfg("tiny_mla", weight_dtype=1)                  # MLA is fp32 only
    assert L.rdt_check_config(ctypes.byref(c)) == 2
    for name in ("tiny_gqa", "tiny_mla", "small_bf16", "small_bf16_k3", "mythos_1b", "mythos_3b",
                 "mythos_10b_decode"):
        assert L.rdt_check_config(ctypes.byref(_cfg(name))) == 0, name


def test_generic_attention_lds_bound_refused_up_front():
    """Configurations that reach the generic attention kernel keep the query
    row and one score per visible key in 64 KB of LDS: a longer max_seq_len
    is refused by the config check (UNSUPPORTED) before any device work,
    and a wide MLA latent (kv_lora_rank 512 + rope 16 query slots in decode)
    is accepted while it fits."""
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    assert L.rdt_check_config(ctypes.byref(_cfg("tiny_gqa", max_seq_len=16000))) == 0
    assert L.rdt_check_config(ctypes.byref(_cfg("tiny_gqa", max_seq_len=16380))) == 2
    assert "LDS" in L.rdt_last_error().decode()
    assert L.rdt_check_config(ctypes.byref(_cfg("tiny_mla", kv_lora_rank=512, max_seq_len=15800))) == 0
    assert L.rdt_check_config(ctypes.byref(_cfg("tiny_mla", kv_lora_rank=512, max_seq_len=15900))) == 2
    # bf16 GQA with at most 16 query heads per KV head never uses it
    assert L.rdt_check_config(ctypes.byref(_cfg("mythos_3b", max_seq_len=1 << 20))) == 0


def test_call_checks():
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    cfg = configs.get("small_bf16")
    c = binding.make_config(cfg)
    ws = binding.workspace_bytes(cfg, 2, 200)
    kvb = binding.kv_cache_bytes(cfg, 2, 256, 3)
    ok = lambda *a: L.rdt_check_call(ctypes.byref(c), *a)
    #        B  T   sp  nl thr   kv cap  kvb  ws  decode
    assert ok(2, 200, 0, 3, 0.99, 0, 0, 0, ws, 0) == 0
    assert ok(0, 200, 0, 3, 0.99, 0, 0, 0, ws, 0) == 1
    assert ok(2, 0, 0, 3, 0.99, 0, 0, 0, ws, 0) == 1
    assert ok(2, 200, 0, 0, 0.99, 0, 0, 0, ws, 0) == 1
    assert ok(2, 200, 0, 5000, 0.99, 0, 0, 0, ws, 0) == 1
    assert ok(2, 200, 0, 3, 1.5, 0, 0, 0, ws, 0) == 1
    assert ok(2, 200, 0, 3, -0.1, 0, 0, 0, ws, 0) == 1
    assert ok(2, 200, 0, 3, 0.99, 0, 0, 0, ws - 1, 0) == 6
    assert ok(2, 200, 400, 3, 0.99, 0, 0, 0, ws, 0) == 1       # past max_seq_len
    assert ok(2, 200, 0, 3, 0.99, 1, 256, kvb, ws, 0) == 0
    assert ok(2, 200, 100, 3, 0.99, 1, 256, kvb, ws, 0) == 1   # past kv capacity
    assert ok(2, 200, 0, 4, 0.99, 1, 256, kvb, ws, 0) == 1     # cache holds 3 loops
    wsd = binding.workspace_bytes(cfg, 2, 1)
    assert ok(2, 1, 10, 3, 0.0, 0, 0, 0, wsd, 1) == 5          # decode without cache
    assert ok(2, 1, 10, 4, 0.0, 1, 256, kvb, wsd, 1) == 5      # more loops than cached
    assert ok(2, 1, 10, 3, 0.0, 1, 256, kvb, wsd, 1) == 0


def test_workspace_layout_is_disjoint_and_aligned():
    from recurrent_depth_moe_amd import binding
    cfg = configs.get("mythos_3b")
    total = binding.workspace_bytes(cfg, 2, 4096)
    spans = []
    for name in ("h", "c", "a", "q", "k", "vt", "o", "x1", "f", "logits", "sel", "gate", "tile_counts",
                 "offsets", "mt_start", "tile_row0", "tile_grp", "perm", "inv", "act", "y", "act_s", "y_s", "cum"):
        off, n = binding.workspace_offset(cfg, 2, 4096, name)
        assert off % 256 == 0 and off + n <= total
        spans.append((off, off + n))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    with pytest.raises(binding.RdtError):
        binding.workspace_offset(cfg, 2, 4096, "nope")


def test_mla_decode_plan_has_latent_buffers():
    """MLA decode steps (T = 1) attend over the cached latent: the plan
    carries the latent query / key / value / output buffers, sized from the
    ranks, and a prefill plan does not."""
    from recurrent_depth_moe_amd import binding
    cfg = configs.get("tiny_mla")
    B, H, kvl, rope = 3, cfg["n_heads"], cfg["kv_lora_rank"], cfg["qk_rope_head_dim"]
    P = cfg["max_seq_len"]
    want = {"q_lat": B * H * (kvl + rope), "k_lat": B * P * (kvl + rope), "vt_lat": B * kvl * P, "o_lat": B * H * kvl}
    for name, n in want.items():
        assert binding.workspace_offset(cfg, B, 1, name)[1] == 4 * n
        assert binding.workspace_offset(cfg, B, 8, name)[1] == 0


def test_kv_cache_size_formula():
    from recurrent_depth_moe_amd import binding
    cfg = configs.get("mythos_10b_decode")
    n = binding.kv_cache_bytes(cfg, 32, 8193, 24)
    P = 8256   # 8193 rounded up to a multiple of 64
    assert n == 24 * 2 * 32 * 8 * P * 128 * 2


def test_injected_allocation_failure(monkeypatch):
    """RDT_FAULT_ALLOC=1 makes create fail with OUT_OF_MEMORY before any
    device call (host-forced failure path)."""
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    monkeypatch.setenv("RDT_FAULT_ALLOC", "1")
    c = _cfg("tiny_gqa")
    arr = (ctypes.c_void_p * len(binding.WEIGHT_NAMES))(*([1] * len(binding.WEIGHT_NAMES)))
    h = ctypes.c_void_p(123)
    st = L.rdt_block_create(ctypes.byref(c), arr, None, ctypes.byref(h))
    assert st == 3 and not h.value
    assert b"RDT_FAULT_ALLOC" in L.rdt_last_error()
    arr[5] = None
    assert L.rdt_block_create(ctypes.byref(c), arr, None, ctypes.byref(h)) == 1   # NULL weight


def test_null_and_status_strings():
    from recurrent_depth_moe_amd import binding
    L = binding.lib()
    for s in range(7):
        assert L.rdt_status_string(s)
    assert L.rdt_block_destroy(None) == 0
    assert L.rdt_block_create(None, None, None, None) == 1
