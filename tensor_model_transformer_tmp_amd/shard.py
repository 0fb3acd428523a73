"""ctypes binding of liboases_shard (argument marshalling only).

Every step of the TMP-shard path runs in the library's HIP kernels; torch is
used here only to own device memory and to provide HIP streams.  The names of
the three entry points match the C ABI: ``layer_fwd``, ``layer_bwd_recompute``
and ``schedule_step``.  Importing this module fails loudly if the library has
not been built; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboases_shard.so")

OK, E_ARG, E_STATE, E_SHAPE, E_ALIGN, E_HIP, E_UNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
F32, BF16 = 0, 1
ATTN, FFN = 0, 1
MODES = {"overlap_fine": 0, "serial_fine": 1, "serial_default": 2, "serial_norecompute": 3,
         "overlap_fused": 4, "overlap_streams": 5}
OP_KINDS = ("F", "C_F", "R", "C_R", "B_dX", "C_B", "B_dW")
KCLASS = {"gemm_fwd": 0, "gemm_dx": 1, "gemm_dw": 2, "attn_fwd": 3, "attn_bwd": 4, "sum": 5,
          "colsum": 6, "all": 7}  # "all": every class (timeline runs)

EXPORTED = ("oases_create", "oases_workspace_bytes", "oases_bind", "oases_set_streams",
            "layer_fwd", "layer_bwd_recompute", "schedule_step", "oases_schedule_ops",
            "oases_sync", "oases_last_error", "oases_destroy", "oases_profile_begin",
            "oases_profile_end", "oases_profile_timeline", "oases_mfma_probe", "oases_allreduce_point", "oases_gemm", "oases_gemm_tile_variant",
            "oases_attention_variant", "oases_sum_grid_cap", "oases_sum_variant", "oases_attention_fwd",
            "oases_attention_bwd_workspace_bytes", "oases_attention_bwd", "oases_attention_bwd_noalloc",
            "oases_last_call_error")


class OasesError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"liboases_shard error {code}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("blocks", ctypes.POINTER(ctypes.c_int32)),
                ("micro_batch", ctypes.c_int32), ("seq", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("heads_per_shard", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("ffn_shard", ctypes.c_int32),
                ("tmp_width", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("full_block", ctypes.c_int32),
                ("drop_q", ctypes.c_int32), ("drop_seed", ctypes.c_uint64),
                ("ln_eps", ctypes.c_float), ("gelu_tanh", ctypes.c_int32)]


class LayerParams(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_in", "b_in", "w_out", "dw_in", "db_in", "dw_out",
                                                 "ln_w", "ln_b", "dln_w", "dln_b")]


class Buffers(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("x", "y", "dy", "dx", "ckpt", "peers_fwd",
                                                 "peers_bwd", "workspace")] + \
               [("workspace_bytes", ctypes.c_size_t)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m "
                          "tensor_model_transformer_tmp_amd.build` (no fallback exists)")
    lib = ctypes.CDLL(path)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    sig = {
        "oases_create": (ctypes.c_int, [ctypes.POINTER(Config), ctypes.POINTER(P)]),
        "oases_workspace_bytes": (ctypes.c_int, [ctypes.POINTER(Config), I32,
                                                 ctypes.POINTER(ctypes.c_size_t)]),
        "oases_bind": (ctypes.c_int, [P, ctypes.POINTER(Buffers), ctypes.POINTER(LayerParams)]),
        "oases_set_streams": (ctypes.c_int, [P, P, P]),
        "layer_fwd": (ctypes.c_int, [P, I32, I32]),
        "layer_bwd_recompute": (ctypes.c_int, [P, I32, I32]),
        "schedule_step": (ctypes.c_int, [P, I32, I32]),
        "oases_schedule_ops": (ctypes.c_int, [P, I32, ctypes.POINTER(I32), I32, ctypes.POINTER(I32)]),
        "oases_sync": (ctypes.c_int, [P]),
        "oases_last_error": (ctypes.c_char_p, [P]),
        "oases_destroy": (None, [P]),
        "oases_profile_begin": (ctypes.c_int, [P, I32, I32]),
        "oases_profile_end": (ctypes.c_int, [P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]),
        "oases_profile_timeline": (ctypes.c_int, [P, I32, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                                  ctypes.POINTER(ctypes.c_double),
                                                  ctypes.POINTER(ctypes.c_double), ctypes.POINTER(I32)]),
        "oases_mfma_probe": (ctypes.c_int, [I32, I32, P, P]),
        "oases_allreduce_point": (ctypes.c_int, [I32, P, P, I64, I32, P, I64, P]),
        "oases_gemm": (ctypes.c_int, [I32, I32, I32, I32, I32, I32, I32, P, I32, P, I32, P, I32, P, P,
                                      P, I32, I32, P]),
        "oases_gemm_tile_variant": (ctypes.c_int, [I32]),
        "oases_attention_variant": (ctypes.c_int, [I32]),
        "oases_sum_grid_cap": (ctypes.c_int, [I32]),
        "oases_sum_variant": (ctypes.c_int, [I32]),
        "oases_attention_fwd": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, P]),
        "oases_attention_bwd_workspace_bytes": (ctypes.c_int, [I32, I32, I32, ctypes.POINTER(ctypes.c_size_t)]),
        "oases_attention_bwd": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, P, P, P, ctypes.c_size_t, P]),
        "oases_attention_bwd_noalloc": (ctypes.c_int, [I32, I32, I32, I32, I32, P, P, P, P, P, P]),
        "oases_last_call_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


def _ptr(t):
    """Device (or host) address of a torch tensor, or None."""
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    if stream is None:
        return None
    return ctypes.c_void_p(stream.cuda_stream)


def make_config(cfg) -> tuple:
    """ctypes Config from a ShardConfig-like object (keeps the blocks array alive)."""
    blocks = (ctypes.c_int32 * cfg.n_layers)(*cfg.blocks)
    full = bool(getattr(cfg, "full_block", False))
    c = Config(cfg.n_layers, ctypes.cast(blocks, ctypes.POINTER(ctypes.c_int32)), cfg.micro_batch,
               cfg.seq, cfg.hidden, cfg.heads_per_shard, cfg.head_dim, cfg.ffn_shard,
               cfg.tmp_width, cfg.dtype, int(cfg.causal), int(full),
               int(getattr(cfg, "drop_q", 0)) if full else 0, int(getattr(cfg, "drop_seed", 0)),
               float(getattr(cfg, "ln_eps", 1e-5)), int(bool(getattr(cfg, "gelu_tanh", False))))
    return c, blocks


def workspace_bytes(cfg, mode) -> int:
    c, _keep = make_config(cfg)
    out = ctypes.c_size_t(0)
    r = lib().oases_workspace_bytes(ctypes.byref(c), MODES.get(mode, mode), ctypes.byref(out))
    if r != OK:
        raise OasesError(r, "oases_workspace_bytes rejected the configuration")
    return out.value


class ShardContext:
    """One liboases_shard context.  Buffers are torch tensors owned by the caller."""

    def __init__(self, cfg):
        self.cfg = cfg
        c, self._blocks = make_config(cfg)
        h = ctypes.c_void_p()
        r = lib().oases_create(ctypes.byref(c), ctypes.byref(h))
        if r != OK:
            raise OasesError(r, "oases_create rejected the configuration")
        self.h = h
        self._keep = []

    def _check(self, r, what):
        if r != OK:
            raise OasesError(r, f"{what}: {lib().oases_last_error(self.h).decode()}")

    def bind(self, bufs: dict, params: list):
        """bufs: x, y, dy, dx, ckpt, peers_fwd, peers_bwd, workspace (torch tensors or None).
        params: per layer dict w_in, b_in, w_out, dw_in, db_in, dw_out (and ln_w, ln_b,
        dln_w, dln_b for full blocks)."""
        ws = bufs["workspace"]
        b = Buffers(*[_ptr(bufs.get(n)) for n in ("x", "y", "dy", "dx", "ckpt", "peers_fwd",
                                                  "peers_bwd", "workspace")],
                    ws.numel() * ws.element_size())
        arr = (LayerParams * self.cfg.n_layers)()
        for l, p in enumerate(params):
            arr[l] = LayerParams(*[_ptr(p.get(n)) for n in ("w_in", "b_in", "w_out", "dw_in", "db_in",
                                                             "dw_out", "ln_w", "ln_b", "dln_w", "dln_b")])
        self._check(lib().oases_bind(self.h, ctypes.byref(b), arr), "oases_bind")
        self._keep = [bufs, params]

    def bind_raw(self, buffers: Buffers, params) -> int:
        """Bind pre-built ctypes structures; returns the status (no raise)."""
        return lib().oases_bind(self.h, ctypes.byref(buffers), params)

    def set_streams(self, compute, side):
        self._check(lib().oases_set_streams(self.h, _stream_handle(compute), _stream_handle(side)),
                    "oases_set_streams")

    def layer_fwd(self, layer: int, sub_batch: int):
        self._check(lib().layer_fwd(self.h, layer, sub_batch), "layer_fwd")

    def layer_bwd_recompute(self, layer: int, sub_batch: int):
        self._check(lib().layer_bwd_recompute(self.h, layer, sub_batch), "layer_bwd_recompute")

    def schedule_step(self, mode="overlap_fine", use_graph: bool = False):
        self._check(lib().schedule_step(self.h, MODES.get(mode, mode), int(use_graph)),
                    "schedule_step")

    def status(self, fn: str, *args) -> int:
        """Call an entry point by name and return its raw status."""
        return getattr(lib(), fn)(self.h, *args)

    def schedule_ops(self, mode):
        n = ctypes.c_int32(0)
        m = MODES.get(mode, mode)
        self._check(lib().oases_schedule_ops(self.h, m, None, 0, ctypes.byref(n)), "oases_schedule_ops")
        buf = (ctypes.c_int32 * (4 * n.value))()
        self._check(lib().oases_schedule_ops(self.h, m, buf, n.value, ctypes.byref(n)),
                    "oases_schedule_ops")
        a = np.frombuffer(buf, dtype=np.int32).reshape(-1, 4)
        return [(OP_KINDS[k], int(l), int(sb), int(st)) for k, l, sb, st in a]

    def sync(self):
        self._check(lib().oases_sync(self.h), "oases_sync")

    def profile_begin(self, kernel_class: str, max_launches: int = 4096):
        self._check(lib().oases_profile_begin(self.h, KCLASS[kernel_class], max_launches),
                    "oases_profile_begin")

    def profile_end(self):
        ms, n = ctypes.c_double(0), ctypes.c_int32(0)
        self._check(lib().oases_profile_end(self.h, ctypes.byref(ms), ctypes.byref(n)),
                    "oases_profile_end")
        return ms.value, n.value

    def profile_timeline(self, cap: int):
        """End a timing run begun with profile_begin("all", ...): a list of
        (class name, stream 0 compute / 1 side, start ms, end ms) per timed
        launch, times relative to the start of the first timed launch."""
        cls, st = (ctypes.c_int32 * cap)(), (ctypes.c_int32 * cap)()
        t0, t1 = (ctypes.c_double * cap)(), (ctypes.c_double * cap)()
        n = ctypes.c_int32(0)
        self._check(lib().oases_profile_timeline(self.h, cap, cls, st, t0, t1, ctypes.byref(n)),
                    "oases_profile_timeline")
        names = {v: k for k, v in KCLASS.items()}
        return [(names[cls[i]], st[i], t0[i], t1[i]) for i in range(n.value)]

    def last_error(self) -> str:
        return lib().oases_last_error(self.h).decode()

    def close(self):
        if getattr(self, "h", None):
            lib().oases_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---- single-kernel entry points ------------------------------------------------

def _check_free(r, what):
    if r != OK:
        raise OasesError(r, f"{what}: {lib().oases_last_call_error().decode()}")


def mfma_probe(workgroups: int, iters: int, out, stream=None):
    """Dense bf16 MFMA throughput probe; out: float32 device tensor of
    workgroups * 256 elements.  Returns the FLOPs the launch issues."""
    _check_free(lib().oases_mfma_probe(workgroups, iters, _ptr(out), _stream_handle(stream)),
                "oases_mfma_probe")
    return workgroups * 4 * 4 * iters * 32 * 32 * 16 * 2


def allreduce_point(dtype, own, peers, n_peers, out, stream=None):
    n = own.numel()
    stride = n if n_peers > 0 else 0
    _check_free(lib().oases_allreduce_point(dtype, _ptr(own), _ptr(peers), stride, n_peers,
                                            _ptr(out), n, _stream_handle(stream)),
                "oases_allreduce_point")


EPILOGUES = {"store": 0, "bias": 1, "gelu": 2, "gelu_bwd": 3, "f32": 4, "f32_colsum": 5, "gelu_tanh": 6,
             "gelu_tanh_bwd": 7}


def gemm(dtype, a, b, c, a_layout=0, b_layout=0, epilogue="store", m=None, n=None, k=None,
         bias=None, pre=None, aux=None, beta=0, stream=None):
    """C = A B with the operand layouts of the C ABI (0: k contiguous, 1: m/n contiguous)."""
    if m is None:
        m = a.shape[0] if a_layout == 0 else a.shape[1]
        k = a.shape[1] if a_layout == 0 else a.shape[0]
        n = b.shape[0] if b_layout == 0 else b.shape[1]
    _check_free(lib().oases_gemm(dtype, a_layout, b_layout, EPILOGUES[epilogue], m, n, k, _ptr(a),
                                 a.stride(0), _ptr(b), b.stride(0), _ptr(c), c.stride(0), _ptr(bias),
                                 _ptr(pre), _ptr(aux), aux.stride(0) if aux is not None else 0,
                                 int(beta), _stream_handle(stream)), "oases_gemm")


def gemm_fwd(dtype, a, b, c, bias=None, gelu=False, pre=None, stream=None):
    """C[M,N] = A[M,K] B[N,K]^T (+ bias) (GeLU)."""
    epi = "gelu" if gelu else ("bias" if bias is not None else "store")
    gemm(dtype, a, b, c, 0, 0, epi, bias=bias, pre=pre, stream=stream)


def set_gemm_tile_variant(v: int):
    _check_free(lib().oases_gemm_tile_variant(v), "oases_gemm_tile_variant")


def set_sum_grid_cap(workgroups: int):
    _check_free(lib().oases_sum_grid_cap(workgroups), "oases_sum_grid_cap")


def set_sum_variant(v: int):
    _check_free(lib().oases_sum_variant(v), "oases_sum_variant")


def set_attention_variant(v: int):
    _check_free(lib().oases_attention_variant(v), "oases_attention_variant")


def attention_fwd(nb, s, nh, d, causal, qkv, o, lse, stream=None):
    _check_free(lib().oases_attention_fwd(nb, s, nh, d, int(causal), _ptr(qkv), _ptr(o), _ptr(lse),
                                          _stream_handle(stream)), "oases_attention_fwd")


def attention_bwd_workspace_bytes(nb, s, nh) -> int:
    out = ctypes.c_size_t(0)
    _check_free(lib().oases_attention_bwd_workspace_bytes(nb, s, nh, ctypes.byref(out)),
                "oases_attention_bwd_workspace_bytes")
    return out.value


def attention_bwd(nb, s, nh, d, causal, qkv, o, dout, lse, dqkv, workspace, stream=None):
    """dQKV of the attention block; workspace: a device tensor of at least
    attention_bwd_workspace_bytes(nb, s, nh) bytes."""
    _check_free(lib().oases_attention_bwd(nb, s, nh, d, int(causal), _ptr(qkv), _ptr(o), _ptr(dout), _ptr(lse),
                                          _ptr(dqkv), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(),
                                          _stream_handle(stream)), "oases_attention_bwd")


def attention_bwd_noalloc(nb, s, nh, d, causal, qkv, o, dout, lse, dqkv, stream=None):
    """dQKV of the attention block with the library's static scratch (no
    workspace argument; problems up to 48 MiB of scratch)."""
    _check_free(lib().oases_attention_bwd_noalloc(nb, s, nh, d, int(causal), _ptr(qkv), _ptr(o), _ptr(dout),
                                                  _ptr(lse), _ptr(dqkv), _stream_handle(stream)),
                "oases_attention_bwd_noalloc")
