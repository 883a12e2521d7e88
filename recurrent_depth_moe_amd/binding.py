"""ctypes binding of librdt.so (include/rdt.h).

Argument marshalling only: torch tensors provide device memory and the
stream; every step of the block runs in the HIP kernels behind the C ABI.
There is no fallback: if the library is missing or a call fails, this
raises.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librdt.so")

RDT_F32, RDT_BF16 = 0, 1
RDT_ATTN_GQA, RDT_ATTN_MLA = 0, 1
STATUS = {0: "RDT_OK", 1: "RDT_E_INVALID_ARG", 2: "RDT_E_UNSUPPORTED", 3: "RDT_E_OUT_OF_MEMORY",
          4: "RDT_E_HIP", 5: "RDT_E_BAD_STATE", 6: "RDT_E_WORKSPACE_TOO_SMALL"}

STAGES = ["loop_head", "qkv", "attention", "o_proj", "ffn_norm", "router", "dispatch", "expert_gate_up",
          "expert_down", "shared_gate_up", "shared_down", "tail"]

WEIGHT_NAMES = ["g_rec", "g_attn", "g_ffn", "wq", "wk", "wv", "wo", "wdq", "gq", "wuq", "wdkv", "gkv", "wukv",
                "router_w", "router_bias", "w_gate", "w_up", "w_down", "s_gate", "s_up", "s_down",
                "lora_down", "lora_B", "lora_scale", "log_A", "log_dt", "B", "halt_w", "halt_b"]


class RdtConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("dim", "n_heads", "n_kv_heads", "head_dim", "attn",
                                               "q_lora_rank", "kv_lora_rank", "qk_rope_head_dim",
                                               "qk_nope_head_dim", "v_head_dim", "n_experts",
                                               "n_shared_experts", "top_k", "expert_dim", "lora_rank",
                                               "max_loop_iters", "loop_dim", "max_seq_len")] + \
        [("rope_theta", ctypes.c_float), ("loop_theta", ctypes.c_float), ("norm_eps", ctypes.c_float),
         ("weight_dtype", ctypes.c_int32)]


class RdtError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float
    cfgp = ctypes.POINTER(RdtConfig)
    sig = {
        "rdt_abi_version": ([], i32),
        "rdt_status_string": ([i32], ctypes.c_char_p),
        "rdt_last_error": ([], ctypes.c_char_p),
        "rdt_check_config": ([cfgp], i32),
        "rdt_workspace_bytes_cfg": ([cfgp, i32, i32, ctypes.POINTER(sz)], i32),
        "rdt_kv_cache_bytes_cfg": ([cfgp, i32, i32, i32, ctypes.POINTER(sz)], i32),
        "rdt_workspace_offset_cfg": ([cfgp, i32, i32, ctypes.c_char_p, ctypes.POINTER(sz), ctypes.POINTER(sz)], i32),
        "rdt_check_call": ([cfgp, i32, i32, i32, i32, f32, i32, i32, sz, sz, i32], i32),
        "rdt_block_create": ([cfgp, ctypes.POINTER(vp), vp, ctypes.POINTER(vp)], i32),
        "rdt_block_destroy": ([vp], i32),
        "rdt_param_count": ([vp, ctypes.POINTER(ctypes.c_int64)], i32),
        "rdt_workspace_bytes": ([vp, i32, i32, ctypes.POINTER(sz)], i32),
        "rdt_kv_cache_bytes": ([vp, i32, i32, i32, ctypes.POINTER(sz)], i32),
        "rdt_workspace_offset": ([vp, i32, i32, ctypes.c_char_p, ctypes.POINTER(sz), ctypes.POINTER(sz)], i32),
        "rdt_recurrent_forward": ([vp, vp, vp, i32, i32, i32, i32, f32, vp, i32, sz, vp, sz, vp, vp, vp], i32),
        "rdt_decode_step": ([vp, vp, vp, i32, i32, i32, f32, vp, i32, sz, vp, sz, vp, vp, vp], i32),
        "rdt_get_A": ([vp, vp], i32),
        "rdt_set_capture": ([vp, vp, vp, vp, i32], i32),
        "rdt_set_timing": ([vp, i32], i32),
        "rdt_set_timing_stages": ([vp, ctypes.c_uint32], i32),
        "rdt_read_timing": ([vp, vp, vp], i32),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    _lib = L
    return L


def check(status):
    if status != 0:
        raise RdtError(status, lib().rdt_last_error().decode())


def make_config(cfg):
    """rdt_config from a workload dictionary (workloads.configs)."""
    c = RdtConfig()
    for f in ("dim", "n_heads", "head_dim", "q_lora_rank", "kv_lora_rank", "qk_rope_head_dim",
              "qk_nope_head_dim", "v_head_dim", "n_experts", "n_shared_experts", "top_k", "expert_dim",
              "lora_rank", "max_loop_iters", "loop_dim", "max_seq_len"):
        setattr(c, f, int(cfg[f]))
    c.n_kv_heads = int(cfg["n_kv_heads"])
    c.attn = RDT_ATTN_GQA if cfg["attn"] == "gqa" else RDT_ATTN_MLA
    c.rope_theta = float(cfg["rope_theta"])
    c.loop_theta = float(cfg["loop_theta"])
    c.norm_eps = float(cfg["norm_eps"])
    c.weight_dtype = RDT_BF16 if cfg["dtype"] == "bf16" else RDT_F32
    return c


def _ptr(t):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(cfg, B, T):
    n = ctypes.c_size_t()
    check(lib().rdt_workspace_bytes_cfg(ctypes.byref(make_config(cfg)), B, T, ctypes.byref(n)))
    return n.value


def kv_cache_bytes(cfg, B, capacity, n_loops):
    n = ctypes.c_size_t()
    check(lib().rdt_kv_cache_bytes_cfg(ctypes.byref(make_config(cfg)), B, capacity, n_loops, ctypes.byref(n)))
    return n.value


def workspace_offset(cfg, B, T, name):
    off, n = ctypes.c_size_t(), ctypes.c_size_t()
    check(lib().rdt_workspace_offset_cfg(ctypes.byref(make_config(cfg)), B, T, name.encode(),
                                         ctypes.byref(off), ctypes.byref(n)))
    return off.value, n.value


class Block:
    """Owns an rdt_block handle.  ``weights`` maps names to device tensors."""

    def __init__(self, cfg, weights, stream=None):
        self.cfg = cfg
        self._c = make_config(cfg)
        arr = (ctypes.c_void_p * len(WEIGHT_NAMES))()
        for i, n in enumerate(WEIGHT_NAMES):
            t = weights.get(n)
            if t is not None:
                assert t.is_cuda and t.is_contiguous(), n
                arr[i] = t.data_ptr()
        h = ctypes.c_void_p()
        check(lib().rdt_block_create(ctypes.byref(self._c), arr, _stream(stream), ctypes.byref(h)))
        self._h = h

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            check(lib().rdt_block_destroy(self._h))
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def param_count(self):
        n = ctypes.c_int64()
        check(lib().rdt_param_count(self._h, ctypes.byref(n)))
        return n.value

    def workspace_bytes(self, B, T):
        n = ctypes.c_size_t()
        check(lib().rdt_workspace_bytes(self._h, B, T, ctypes.byref(n)))
        return n.value

    def kv_cache_bytes(self, B, capacity, n_loops):
        n = ctypes.c_size_t()
        check(lib().rdt_kv_cache_bytes(self._h, B, capacity, n_loops, ctypes.byref(n)))
        return n.value

    def new_workspace(self, B, T):
        return torch.empty(self.workspace_bytes(B, T), dtype=torch.uint8, device="cuda")

    def workspace_view(self, ws, B, T, name, dtype, shape=None):
        off, n = ctypes.c_size_t(), ctypes.c_size_t()
        check(lib().rdt_workspace_offset(self._h, B, T, name.encode(), ctypes.byref(off), ctypes.byref(n)))
        v = ws[off.value:off.value + n.value].view(dtype)
        return v if shape is None else v[:int(torch.Size(shape).numel())].view(shape)

    def get_A(self):
        out = torch.empty(self.cfg["dim"], dtype=torch.float32)
        check(lib().rdt_get_A(self._h, ctypes.c_void_p(out.data_ptr())))
        return out

    def set_capture(self, h_loops=None, sel_loops=None, p_loops=None, max_loops=0):
        check(lib().rdt_set_capture(self._h, _ptr(h_loops), _ptr(sel_loops), _ptr(p_loops), max_loops))
        self._capture = (h_loops, sel_loops, p_loops)

    def set_timing(self, enable=True):
        check(lib().rdt_set_timing(self._h, 1 if enable else 0))

    def set_timing_stages(self, stages):
        """Time only the named stages (an empty list turns timing off)."""
        check(lib().rdt_set_timing_stages(self._h, sum(1 << STAGES.index(s) for s in stages)))

    def read_timing(self):
        """{stage: (total_ms, launches)} since set_timing(True)."""
        ms = (ctypes.c_double * len(STAGES))()
        n = (ctypes.c_int64 * len(STAGES))()
        check(lib().rdt_read_timing(self._h, ms, n))
        return {st: (ms[i], n[i]) for i, st in enumerate(STAGES)}

    def forward(self, e, h0, n_loops, act_threshold, start_pos=0, kv_cache=None, kv_capacity=0,
                workspace=None, h_out=None, halt_counts=None, stream=None):
        B, T, D = e.shape
        if workspace is None:
            workspace = self.new_workspace(B, T)
        if h_out is None:
            h_out = torch.empty_like(e)
        if halt_counts is None:
            halt_counts = torch.empty((B, T), dtype=torch.int32, device=e.device)
        kvb = 0 if kv_cache is None else kv_cache.numel() * kv_cache.element_size()
        check(lib().rdt_recurrent_forward(self._h, _ptr(e), _ptr(h0), B, T, start_pos, n_loops,
                                          float(act_threshold), _ptr(kv_cache), kv_capacity, kvb,
                                          _ptr(workspace), workspace.numel(), _ptr(h_out), _ptr(halt_counts),
                                          _stream(stream)))
        return h_out, halt_counts

    def decode_step(self, e_new, h0_new, start_pos, n_loops, act_threshold, kv_cache, kv_capacity,
                    workspace=None, h_out=None, halt_counts=None, stream=None):
        B = e_new.shape[0]
        if workspace is None:
            workspace = self.new_workspace(B, 1)
        if h_out is None:
            h_out = torch.empty_like(e_new)
        if halt_counts is None:
            halt_counts = torch.empty((B, 1), dtype=torch.int32, device=e_new.device)
        kvb = 0 if kv_cache is None else kv_cache.numel() * kv_cache.element_size()
        check(lib().rdt_decode_step(self._h, _ptr(e_new), _ptr(h0_new), B, start_pos, n_loops,
                                    float(act_threshold), _ptr(kv_cache), kv_capacity, kvb, _ptr(workspace),
                                    workspace.numel(), _ptr(h_out), _ptr(halt_counts), _stream(stream)))
        return h_out, halt_counts


def weights_to_device(W, device="cuda"):
    """numpy arrays (bf16 bit patterns as uint16, or float32) -> device tensors."""
    import numpy as np
    out = {}
    for k, v in W.items():
        if v.dtype == np.uint16:
            out[k] = torch.from_numpy(v.view(np.int16)).to(device).view(torch.bfloat16)
        else:
            out[k] = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(device)
    return out
