"""Python binding of libdmx, the MI355X (gfx950) action-expert layer library.

Thin ctypes marshalling over the C ABI declared in ``include/dmx.h``: every
function here has the C entry point's name without the ``dmx_`` prefix, takes
torch tensors (device memory) and the current HIP stream, checks shapes and
dtypes, and calls the library.  All arithmetic runs in the HIP kernels.  There
is no fallback: if the library is missing or the call fails, an exception is
raised.
"""
from __future__ import annotations

import ctypes
import os

import torch

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdmx.so")

OK, FALLBACK_EAGER = 0, 1
ERR_INVALID_ARG, ERR_BAD_BUCKETS, ERR_PREFIX_TOO_LONG = -1, -2, -3
ERR_UNSUPPORTED, ERR_MISALIGNED, ERR_WORKSPACE, ERR_HIP, ERR_SYNC = -4, -5, -6, -7, -8

H, I, D, HQ, HK = 1024, 4096, 256, 8, 4

# kernels of the stack, for per-kernel timing (Stack.stage_launch)
STAGE_MODS, STAGE_PACK, STAGE_QKV, STAGE_ATTN, STAGE_COMBINE, STAGE_OPROJ, STAGE_GATEUP, STAGE_DOWN = range(8)
STAGE_NAMES = ("modulation", "input pack", "qkv+norm+rope", "attention", "attention combine", "o-projection",
               "gate-up", "down")
PREFIX_HIDDEN = 2560

EXPORTED = (
    "dmx_select_bucket", "dmx_workspace_bytes", "dmx_stack_workspace_bytes", "dmx_workspace_init", "dmx_pack_weight",
    "dmx_adarms_prenorm",
    "dmx_qkv_qknorm_rope", "dmx_suffix_attention", "dmx_oproj_gated_residual", "dmx_geglu_mlp",
    "dmx_suffix_layer_forward", "dmx_suffix_layer_forward_noalloc", "dmx_stack_forward", "dmx_stack_sync_check",
    "dmx_stack_stage_launch",
    "dmx_stack_mod_table_bytes", "dmx_stack_mod_table_fill",
    "dmx_image_merge", "dmx_prefix_attention", "dmx_prefix_attention_workspace_bytes", "dmx_prefix_workspace_bytes", "dmx_prefix_layer_forward",
    "dmx_sampler_schedule_bytes", "dmx_sampler_schedule_fill", "dmx_sampler_forward", "dmx_sampler_graph_create",
    "dmx_lazy_bucket", "dmx_profile_cache_create", "dmx_profile_cache_destroy", "dmx_profile_cache_plan",
    "dmx_profile_cache_keys", "dmx_profile_cache_run_sampler",
    "dmx_stack_graph_create", "dmx_graph_launch", "dmx_graph_destroy", "dmx_status_string", "dmx_last_error_string",
)


class DmxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"dmx status {status}: {message}")
        self.status = status


class LayerWeights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in
                ("w_mod1", "b_mod1", "w_qkv", "q_norm", "k_norm", "w_o", "w_mod2", "b_mod2", "w_gu", "w_down")]


class PrefixKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("mask", ctypes.c_void_p),
                ("p_bucket", ctypes.c_int32)]


PREFIX_WEIGHTS = ("w_in", "w_qkv", "q_norm", "k_norm", "w_o", "w_post_attn", "w_pre_ffn", "w_gu", "w_down",
                  "w_post_ffn")
PREFIX_MATRICES = ("w_qkv", "w_o", "w_gu", "w_down")
PREFIX_INTER = 10240


class PrefixLayerWeights(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in PREFIX_WEIGHTS]


class StackDesc(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("n_steps", ctypes.c_int32), ("batch", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("p_bucket", ctypes.c_int32),
                ("layers", ctypes.POINTER(LayerWeights)),
                ("k_pre", ctypes.POINTER(ctypes.c_void_p)), ("v_pre", ctypes.POINTER(ctypes.c_void_p)),
                ("mask", ctypes.c_void_p), ("cond", ctypes.c_void_p), ("pos0", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
                ("mod_table", ctypes.c_void_p), ("persistent", ctypes.c_int32), ("layer_trace", ctypes.c_void_p)]


SAMPLER_WEIGHTS = ("w_in", "b_in", "w_t1", "b_t1", "w_t2", "b_t2", "w_fmod", "b_fmod", "w_out", "b_out")
SAMPLER_MATRICES = ("w_t1", "w_t2", "w_fmod")  # tiled; w_in / w_out stay row-major


class SamplerWeights(ctypes.Structure):
    _fields_ = [("action_dim", ctypes.c_int32)] + [(k, ctypes.c_void_p) for k in SAMPLER_WEIGHTS]


class SamplerDesc(ctypes.Structure):
    _fields_ = [("stack", ctypes.POINTER(StackDesc)), ("w", ctypes.POINTER(SamplerWeights)),
                ("sched", ctypes.c_void_p), ("sched_bytes", ctypes.c_size_t), ("actions", ctypes.c_void_p),
                ("trajectory", ctypes.c_void_p)]


_lib = None


def lib():
    """Load libdmx.so (building it first only if no build exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            _build.build_library()
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        sig = {
            "dmx_select_bucket": ([i32, P, i32, i32, i32, P], ctypes.c_int),
            "dmx_workspace_bytes": ([i32, i32, i32], sz),
            "dmx_stack_workspace_bytes": ([i32, i32, i32, i32], sz),
            "dmx_workspace_init": ([P, sz, P], ctypes.c_int),
            "dmx_pack_weight": ([P, i32, i32, P, P], ctypes.c_int),
            "dmx_adarms_prenorm": ([P, P, P, P, i32, i32, P, P, P], ctypes.c_int),
            "dmx_qkv_qknorm_rope": ([P, P, P, P, i32, i32, i32, P, ctypes.c_float, P, P, P, i32, i32, P, sz, P],
                                    ctypes.c_int),
            "dmx_suffix_attention": ([P, P, P, P, P, P, i32, i32, i32, P, P, sz, P], ctypes.c_int),
            "dmx_oproj_gated_residual": ([P, P, P, P, i32, i32, P, P, sz, P], ctypes.c_int),
            "dmx_geglu_mlp": ([P, P, P, P, P, i32, i32, P, P, sz, P], ctypes.c_int),
            "dmx_suffix_layer_forward": ([ctypes.POINTER(LayerWeights), ctypes.POINTER(PrefixKV), P, P, P, i32, i32,
                                          P, P, sz, P], ctypes.c_int),
            "dmx_suffix_layer_forward_noalloc": ([ctypes.POINTER(LayerWeights), ctypes.POINTER(PrefixKV), P, P, P, i32,
                                                  i32, P, P], ctypes.c_int),
            "dmx_stack_forward": ([ctypes.POINTER(StackDesc), P], ctypes.c_int),
            "dmx_stack_sync_check": ([ctypes.POINTER(StackDesc), P], ctypes.c_int),
            "dmx_stack_stage_launch": ([ctypes.POINTER(StackDesc), i32, i32, i32, P], ctypes.c_int),
            "dmx_stack_mod_table_bytes": ([i32, i32, i32], sz),
            "dmx_stack_mod_table_fill": ([ctypes.POINTER(StackDesc), P, P], ctypes.c_int),
            "dmx_image_merge": ([P, P, P, i32, i32, i32, P, P], ctypes.c_int),
            "dmx_prefix_attention": ([P, P, P, P, i32, i32, P, P, sz, P], ctypes.c_int),
            "dmx_prefix_attention_workspace_bytes": ([i32], sz),
            "dmx_prefix_workspace_bytes": ([i32], sz),
            "dmx_prefix_layer_forward": ([ctypes.POINTER(PrefixLayerWeights), P, P, i32, P, P, i32, P, P, sz, P],
                                         ctypes.c_int),
            "dmx_stack_graph_create": ([ctypes.POINTER(StackDesc), P, ctypes.POINTER(P)], ctypes.c_int),
            "dmx_sampler_schedule_bytes": ([i32], sz),
            "dmx_sampler_schedule_fill": ([ctypes.POINTER(SamplerWeights), i32, i32, P, P, sz, P], ctypes.c_int),
            "dmx_sampler_forward": ([ctypes.POINTER(SamplerDesc), P], ctypes.c_int),
            "dmx_sampler_graph_create": ([ctypes.POINTER(SamplerDesc), P, ctypes.POINTER(P)], ctypes.c_int),
            "dmx_lazy_bucket": ([i32, i32], i32),
            "dmx_profile_cache_create": ([i32, i32, ctypes.POINTER(P)], ctypes.c_int),
            "dmx_profile_cache_destroy": ([P], None),
            "dmx_profile_cache_plan": ([P, ctypes.c_int64, ctypes.c_uint64, ctypes.POINTER(i32),
                                        ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
            "dmx_profile_cache_keys": ([P, ctypes.POINTER(ctypes.c_int64)], ctypes.c_int),
            "dmx_profile_cache_run_sampler": ([P, ctypes.POINTER(SamplerDesc), P, ctypes.POINTER(i32)], ctypes.c_int),
            "dmx_graph_launch": ([P, P], ctypes.c_int),
            "dmx_graph_destroy": ([P], None),
            "dmx_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "dmx_last_error_string": ([], ctypes.c_char_p),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(status: int) -> int:
    if status < 0:
        raise DmxError(status, lib().dmx_last_error_string().decode())
    return status


def _p(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _want(t, shape, dtype, name, device=True):
    """Raise ValueError naming `name` unless t is a contiguous tensor of this
    dtype and shape (and on a GPU, unless device=False)."""
    if (t.dtype != dtype or tuple(t.shape) != tuple(shape) or not t.is_contiguous()
            or (device and not t.is_cuda)):
        raise ValueError(f"{name}: expected contiguous cuda {dtype} {tuple(shape)}, got "
                         f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} device={t.device}")


# --------------------------------------------------------------------------- host logic
def select_bucket(prefix_len: int, buckets, fast_prefix_len: int = 1024, min_tokens: int = 0):
    """Returns (status, index); status is OK, FALLBACK_EAGER or a negative error."""
    arr = (ctypes.c_int32 * max(1, len(buckets)))(*[int(b) for b in buckets])
    idx = ctypes.c_int32(-7)
    st = lib().dmx_select_bucket(int(prefix_len), arr, len(buckets), int(fast_prefix_len), int(min_tokens),
                                 ctypes.byref(idx))
    return int(st), int(idx.value)


def workspace_bytes(batch: int, tokens: int, p_bucket: int) -> int:
    return int(lib().dmx_workspace_bytes(batch, tokens, p_bucket))


def new_workspace(batch: int, tokens: int, p_bucket: int, device="cuda"):
    n = workspace_bytes(batch, tokens, p_bucket)
    if n == 0:
        raise DmxError(ERR_UNSUPPORTED, f"no workspace size for batch={batch} tokens={tokens} p={p_bucket}")
    return torch.empty(n, dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- stages
def pack_weight(w, stream=None):
    """Tiled copy of a row-major bf16 weight matrix [rows][cols] (the layout
    every weight argument takes).  The result keeps w's shape for bookkeeping;
    its memory holds the tiles, not rows."""
    if w.dim() != 2:
        raise ValueError(f"pack_weight: expected a 2-D matrix, got shape {tuple(w.shape)}")
    _want(w, w.shape, torch.bfloat16, "w")
    out = torch.empty_like(w)
    _check(lib().dmx_pack_weight(_p(w), w.shape[0], w.shape[1], _p(out), _stream(stream)))
    return out


WEIGHT_MATRICES = ("w_mod1", "w_qkv", "w_o", "w_mod2", "w_gu", "w_down")


def pack_layer_weights(w: dict, stream=None) -> dict:
    """A layer's weights as the library takes them: the matrices tiled by
    pack_weight, the bias and norm vectors unchanged."""
    return {k: pack_weight(v, stream) if k in WEIGHT_MATRICES else v for k, v in w.items()}


def adarms_prenorm(x, cond, w_mod, b_mod, x_norm=None, mod=None, stream=None):
    B, T, _ = x.shape
    _want(x, (B, T, H), torch.bfloat16, "x")
    _want(cond, (B, H), torch.bfloat16, "cond")
    _want(w_mod, (3 * H, H), torch.bfloat16, "w_mod")
    _want(b_mod, (3 * H,), torch.bfloat16, "b_mod")
    x_norm = torch.empty_like(x) if x_norm is None else x_norm
    mod = torch.empty(B, 3 * H, dtype=torch.float32, device=x.device) if mod is None else mod
    _check(lib().dmx_adarms_prenorm(_p(x), _p(cond), _p(w_mod), _p(b_mod), B, T, _p(x_norm), _p(mod),
                                    _stream(stream)))
    return x_norm, mod


def qkv_qknorm_rope(x_norm, w_qkv, q_norm, k_norm, pos0, ws, rope_base=10000.0, k=None, v=None, kv_rows=None,
                    kv_row0=0, stream=None):
    B, T, hidden = x_norm.shape
    _want(x_norm, (B, T, hidden), torch.bfloat16, "x_norm")
    _want(w_qkv, ((HQ + 2 * HK) * D, hidden), torch.bfloat16, "w_qkv")
    _want(pos0, (B,), torch.int32, "pos0")
    kv_rows = T if kv_rows is None else kv_rows
    q = torch.empty(B, T, HQ, D, dtype=torch.bfloat16, device=x_norm.device)
    if k is None:
        k = torch.empty(B, HK, kv_rows, D, dtype=torch.bfloat16, device=x_norm.device)
    if v is None:
        v = torch.empty(B, HK, kv_rows, D, dtype=torch.bfloat16, device=x_norm.device)
    _want(k, (B, HK, kv_rows, D), torch.bfloat16, "k")
    _want(v, (B, HK, kv_rows, D), torch.bfloat16, "v")
    _check(lib().dmx_qkv_qknorm_rope(_p(x_norm), _p(w_qkv), _p(q_norm), _p(k_norm), B, T, hidden, _p(pos0),
                                     float(rope_base), _p(q), _p(k), _p(v), kv_rows, kv_row0, _p(ws), ws.numel(),
                                     _stream(stream)))
    return q, k, v


def suffix_attention(q, k_suf, v_suf, k_pre, v_pre, mask, ws, ctx=None, stream=None):
    B, C = q.shape[:2]
    P = k_pre.shape[2]
    _want(q, (B, C, HQ, D), torch.bfloat16, "q")
    _want(k_suf, (B, HK, C, D), torch.bfloat16, "k_suf")
    _want(v_suf, (B, HK, C, D), torch.bfloat16, "v_suf")
    _want(k_pre, (B, HK, P, D), torch.bfloat16, "k_pre")
    _want(v_pre, (B, HK, P, D), torch.bfloat16, "v_pre")
    _want(mask, (B, P), torch.uint8, "mask")
    ctx = torch.empty_like(q) if ctx is None else ctx
    _check(lib().dmx_suffix_attention(_p(q), _p(k_suf), _p(v_suf), _p(k_pre), _p(v_pre), _p(mask), B, C, P, _p(ctx),
                                      _p(ws), ws.numel(), _stream(stream)))
    return ctx


def oproj_gated_residual(ctx, w_o, mod, residual, ws, out=None, stream=None):
    B, T = residual.shape[:2]
    _want(ctx, (B, T, HQ, D), torch.bfloat16, "ctx")
    _want(w_o, (H, HQ * D), torch.bfloat16, "w_o")
    _want(mod, (B, 3 * H), torch.float32, "mod")
    _want(residual, (B, T, H), torch.bfloat16, "residual")
    out = torch.empty_like(residual) if out is None else out
    _check(lib().dmx_oproj_gated_residual(_p(ctx), _p(w_o), _p(mod), _p(residual), B, T, _p(out), _p(ws),
                                          ws.numel(), _stream(stream)))
    return out


def geglu_mlp(x_norm2, w_gu, w_down, mod2, residual, ws, out=None, stream=None):
    B, T = residual.shape[:2]
    _want(x_norm2, (B, T, H), torch.bfloat16, "x_norm2")
    _want(w_gu, (2 * I, H), torch.bfloat16, "w_gu")
    _want(w_down, (H, I), torch.bfloat16, "w_down")
    _want(mod2, (B, 3 * H), torch.float32, "mod2")
    _want(residual, (B, T, H), torch.bfloat16, "residual")
    out = torch.empty_like(residual) if out is None else out
    _check(lib().dmx_geglu_mlp(_p(x_norm2), _p(w_gu), _p(w_down), _p(mod2), _p(residual), B, T, _p(out), _p(ws),
                               ws.numel(), _stream(stream)))
    return out


WEIGHT_SHAPES = {
    "w_mod1": (3 * H, H), "b_mod1": (3 * H,), "w_qkv": ((HQ + 2 * HK) * D, H), "q_norm": (D,), "k_norm": (D,),
    "w_o": (H, HQ * D), "w_mod2": (3 * H, H), "b_mod2": (3 * H,), "w_gu": (2 * I, H), "w_down": (H, I),
}


def layer_weights_struct(w: dict) -> LayerWeights:
    for k, s in WEIGHT_SHAPES.items():
        _want(w[k], s, torch.bfloat16, k)
    return LayerWeights(**{k: w[k].data_ptr() for k in WEIGHT_SHAPES})


def suffix_layer_forward(w: dict, k_pre, v_pre, mask, x, cond, pos0, ws, out=None, stream=None):
    B, C, _ = x.shape
    P = k_pre.shape[2]
    _want(x, (B, C, H), torch.bfloat16, "x")
    _want(cond, (B, H), torch.bfloat16, "cond")
    _want(pos0, (B,), torch.int32, "pos0")
    _want(k_pre, (B, HK, P, D), torch.bfloat16, "k_pre")
    _want(v_pre, (B, HK, P, D), torch.bfloat16, "v_pre")
    _want(mask, (B, P), torch.uint8, "mask")
    out = torch.empty_like(x) if out is None else out
    lw = layer_weights_struct(w)
    kv = PrefixKV(k_pre.data_ptr(), v_pre.data_ptr(), mask.data_ptr(), P)
    _check(lib().dmx_suffix_layer_forward(ctypes.byref(lw), ctypes.byref(kv), _p(x), _p(cond), _p(pos0), B, C,
                                          _p(out), _p(ws), ws.numel(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 12 * 1024 * 1024  # DMX_NOALLOC_SCRATCH_BYTES


def suffix_layer_forward_noalloc(w: dict, k_pre, v_pre, mask, x, cond, pos0, out, stream=None):
    """dmx_suffix_layer_forward_noalloc: the layer with the library's fixed
    per-GPU scratch instead of a workspace (the caller passes only inputs and
    the output, so nothing is allocated here either)."""
    B, C, _ = x.shape
    P = k_pre.shape[2]
    _want(x, (B, C, H), torch.bfloat16, "x")
    _want(out, (B, C, H), torch.bfloat16, "out")
    _want(cond, (B, H), torch.bfloat16, "cond")
    _want(pos0, (B,), torch.int32, "pos0")
    _want(k_pre, (B, HK, P, D), torch.bfloat16, "k_pre")
    _want(v_pre, (B, HK, P, D), torch.bfloat16, "v_pre")
    _want(mask, (B, P), torch.uint8, "mask")
    lw = layer_weights_struct(w)
    kv = PrefixKV(k_pre.data_ptr(), v_pre.data_ptr(), mask.data_ptr(), P)
    _check(lib().dmx_suffix_layer_forward_noalloc(ctypes.byref(lw), ctypes.byref(kv), _p(x), _p(cond), _p(pos0), B,
                                                  C, _p(out), _stream(stream)))
    return out


# --------------------------------------------------------------------------- stack / graphs
class Stack:
    """The action-expert stack bound to fixed buffers.

    layers: list of weight dicts; k_pre / v_pre: per-layer [B][4][P][256]
    tensors; mask [B][P] uint8; cond [n_steps][B][1024]; pos0 [B] int32;
    x [B][C][1024] (updated in place by run / replay).

    mod_table=True computes the modulation vectors of every step and layer
    once, from cond as it is at construction (or at the last
    fill_mod_table()), and the runs read them instead of recomputing them in
    every step.

    persistent=True runs the whole stack as one persistent kernel (batch 1);
    trace, an optional [n_steps][n_layers][B][C][1024] bf16 tensor, then
    receives every layer's output.  sync_check() reports a persistent run
    that gave up waiting."""

    def __init__(self, layers, k_pre, v_pre, mask, cond, pos0, x, ws=None, mod_table=False, stream=None,
                 persistent=False, trace=None):
        self.n_layers = len(layers)
        self.n_steps, B, _ = cond.shape
        _, C, _ = x.shape
        P = mask.shape[1]
        # the layers write x in place and read pos0 per request: both must
        # match the batch that cond gives
        _want(x, (B, C, H), torch.bfloat16, "x", device=False)
        _want(pos0, (B,), torch.int32, "pos0", device=False)
        _want(x, (B, C, H), torch.bfloat16, "x")
        _want(pos0, (B,), torch.int32, "pos0")
        self._keep = (layers, k_pre, v_pre, mask, cond, pos0, x)
        if ws is None:
            n = int(lib().dmx_stack_workspace_bytes(self.n_layers, B, C, P))
            if n == 0:
                raise DmxError(ERR_UNSUPPORTED, f"no stack workspace for {self.n_layers} layers B={B} C={C} P={P}")
            ws = torch.empty(n, dtype=torch.uint8, device=x.device)
        self.ws = ws
        self._lw = (LayerWeights * self.n_layers)(*[layer_weights_struct(w) for w in layers])
        for t in k_pre + v_pre:
            _want(t, (B, HK, P, D), torch.bfloat16, "k_pre/v_pre")
        self._kp = (ctypes.c_void_p * self.n_layers)(*[t.data_ptr() for t in k_pre])
        self._vp = (ctypes.c_void_p * self.n_layers)(*[t.data_ptr() for t in v_pre])
        _want(cond, (self.n_steps, B, H), torch.bfloat16, "cond")
        _want(mask, (B, P), torch.uint8, "mask")
        if trace is not None:
            _want(trace, (self.n_steps, self.n_layers, B, C, H), torch.bfloat16, "trace")
        self.trace = trace
        self.desc = StackDesc(self.n_layers, self.n_steps, B, C, P, self._lw, self._kp, self._vp,
                              mask.data_ptr(), cond.data_ptr(), pos0.data_ptr(), x.data_ptr(),
                              self.ws.data_ptr(), self.ws.numel(), None, int(bool(persistent)),
                              None if trace is None else trace.data_ptr())
        self._graph = None
        self.mod_table = None
        if mod_table:
            n = int(lib().dmx_stack_mod_table_bytes(self.n_layers, self.n_steps, B))
            if n == 0:
                raise DmxError(ERR_UNSUPPORTED, f"no modulation table for {self.n_layers} layers {self.n_steps} steps")
            self.mod_table = torch.empty(n // 4, dtype=torch.float32, device=x.device)
            self.fill_mod_table(stream)
            self.desc.mod_table = self.mod_table.data_ptr()

    def fill_mod_table(self, stream=None):
        """(Re)compute the cached modulation vectors from the current cond."""
        _check(lib().dmx_stack_mod_table_fill(ctypes.byref(self.desc), _p(self.mod_table), _stream(stream)))

    def run(self, stream=None):
        _check(lib().dmx_stack_forward(ctypes.byref(self.desc), _stream(stream)))

    def sync_check(self, stream=None):
        """Persistent mode: wait for the stream and raise if a run gave up
        waiting (its hand-off counters are reset for the next run)."""
        _check(lib().dmx_stack_sync_check(ctypes.byref(self.desc), _stream(stream)))

    def stage_launch(self, layer, stage, reps=1, stream=None):
        """reps back-to-back launches of one kernel of the stack (per-kernel timing)."""
        _check(lib().dmx_stack_stage_launch(ctypes.byref(self.desc), int(layer), int(stage), int(reps),
                                            _stream(stream)))

    def capture(self, stream):
        """Capture the stack into a hipGraph on a non-default stream."""
        g = ctypes.c_void_p()
        _check(lib().dmx_stack_graph_create(ctypes.byref(self.desc), _stream(stream), ctypes.byref(g)))
        self._graph = g
        return self

    def replay(self, stream=None):
        if self._graph is None:
            raise DmxError(ERR_INVALID_ARG, "replay() before capture()")
        _check(lib().dmx_graph_launch(self._graph, _stream(stream)))

    def close(self):
        if self._graph is not None:
            lib().dmx_graph_destroy(self._graph)
            self._graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --------------------------------------------------------------------------- prefix (prefill) layer
def image_merge(tok, img, idx, out=None, stream=None):
    """tok [T][H] bf16, img [NI][H] bf16, idx [T] int32 -> [T][H] (image row idx[t], or tok[t] for -1)."""
    T, Hd = tok.shape
    _want(idx, (T,), torch.int32, "idx")
    out = torch.empty_like(tok) if out is None else out
    _check(lib().dmx_image_merge(_p(tok), _p(img) if img.numel() else None, _p(idx), T, img.shape[0], Hd, _p(out),
                                 _stream(stream)))
    return out


def prefix_attention(q, k, v, valid, ctx=None, ws=None, stream=None):
    """q [T][8][256]; k, v [4][kv_rows][256]; valid [T] uint8 -> ctx [T][8][256].
    ws: optional workspace of dmx_prefix_attention_workspace_bytes(T) bytes."""
    T = q.shape[0]
    kv_rows = k.shape[1]
    _want(q, (T, HQ, D), torch.bfloat16, "q")
    _want(k, (HK, kv_rows, D), torch.bfloat16, "k")
    _want(v, (HK, kv_rows, D), torch.bfloat16, "v")
    _want(valid, (T,), torch.uint8, "valid")
    ctx = torch.empty_like(q) if ctx is None else ctx
    if ws is None:
        n = int(lib().dmx_prefix_attention_workspace_bytes(T))
        if n == 0:
            raise DmxError(ERR_UNSUPPORTED, f"no prefix attention workspace for {T} tokens")
        ws = torch.empty(n, dtype=torch.uint8, device=q.device)
    _check(lib().dmx_prefix_attention(_p(q), _p(k), _p(v), _p(valid), T, kv_rows, _p(ctx), _p(ws), ws.numel(),
                                      _stream(stream)))
    return ctx


def pack_prefix_weights(w: dict, stream=None) -> dict:
    """Tile the matrices of a prefix-layer weight dict (vectors are kept)."""
    return {k: pack_weight(v, stream) if k in PREFIX_MATRICES else v for k, v in w.items()}


def new_prefix_workspace(tokens: int, device="cuda"):
    n = int(lib().dmx_prefix_workspace_bytes(int(tokens)))
    if n == 0:
        raise DmxError(ERR_UNSUPPORTED, f"no prefix workspace for {tokens} tokens")
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefix_layer_forward(w: dict, x, valid, k_cache, v_cache, ws=None, out=None, stream=None):
    """One prefix decoder layer.  w: tiled weights keyed by PREFIX_WEIGHTS; x [T][2560];
    valid [T] uint8; k_cache / v_cache [4][kv_rows][256] (rows 0 .. T-1 written)."""
    T = x.shape[0]
    kv_rows = k_cache.shape[1]
    _want(x, (T, PREFIX_HIDDEN), torch.bfloat16, "x")
    _want(valid, (T,), torch.uint8, "valid")
    _want(k_cache, (HK, kv_rows, D), torch.bfloat16, "k_cache")
    _want(v_cache, (HK, kv_rows, D), torch.bfloat16, "v_cache")
    _want(w["w_qkv"], ((HQ + 2 * HK) * D, PREFIX_HIDDEN), torch.bfloat16, "w_qkv")
    _want(w["w_o"], (PREFIX_HIDDEN, HQ * D), torch.bfloat16, "w_o")
    _want(w["w_gu"], (2 * PREFIX_INTER, PREFIX_HIDDEN), torch.bfloat16, "w_gu")
    _want(w["w_down"], (PREFIX_HIDDEN, PREFIX_INTER), torch.bfloat16, "w_down")
    ws = new_prefix_workspace(T, x.device) if ws is None else ws
    out = torch.empty_like(x) if out is None else out
    pw = PrefixLayerWeights(*[w[k].data_ptr() for k in PREFIX_WEIGHTS])
    _check(lib().dmx_prefix_layer_forward(ctypes.byref(pw), _p(x), _p(valid), T, _p(k_cache), _p(v_cache), kv_rows,
                                          _p(out), _p(ws), ws.numel(), _stream(stream)))
    return out


# --------------------------------------------------------------------------- denoise sampler
def pack_sampler_weights(w: dict, stream=None) -> dict:
    """Tile the sampler's square / modulation matrices (w_in, w_out and the
    biases are kept row-major)."""
    return {k: pack_weight(v, stream) if k in SAMPLER_MATRICES else v for k, v in w.items()}


class Sampler:
    """Denoising runs over a Stack's buffers: per step the action
    in-projection writes the stack's x, the layers run with the step's
    conditioning, and the final norm + out-projection + Euler update advance
    `actions` [B][C][A] (fp32, the noise on entry).  Building the sampler
    writes the schedule's conditioning into the stack's cond buffer (and
    refreshes its modulation table, if it has one).

    sw: sampler weights from pack_sampler_weights; trajectory: optional
    [n_steps][B][C][A] fp32 receiving the actions after every step."""

    def __init__(self, stack: Stack, sw: dict, actions, trajectory=None, stream=None):
        d = stack.desc
        B, C, n = d.batch, d.chunk, d.n_steps
        A = sw["w_out"].shape[0]
        _want(sw["w_in"], (H, A), torch.bfloat16, "w_in")
        _want(sw["w_t1"], (H, H), torch.bfloat16, "w_t1")
        _want(sw["w_t2"], (H, H), torch.bfloat16, "w_t2")
        _want(sw["w_fmod"], (2 * H, H), torch.bfloat16, "w_fmod")
        _want(sw["w_out"], (A, H), torch.bfloat16, "w_out")
        _want(actions, (B, C, A), torch.float32, "actions")
        if trajectory is not None:
            _want(trajectory, (n, B, C, A), torch.float32, "trajectory")
        nb = int(lib().dmx_sampler_schedule_bytes(n))
        if nb == 0:
            raise DmxError(ERR_UNSUPPORTED, f"no sampler schedule for {n} steps")
        self.stack = stack
        self.sched = torch.empty(nb, dtype=torch.uint8, device=actions.device)
        self._keep = (sw, actions, trajectory)
        self._sw = SamplerWeights(A, *[sw[k].data_ptr() for k in SAMPLER_WEIGHTS])
        self.desc = SamplerDesc(ctypes.pointer(stack.desc), ctypes.pointer(self._sw), self.sched.data_ptr(), nb,
                                actions.data_ptr(), None if trajectory is None else trajectory.data_ptr())
        self._graph = None
        self.fill_schedule(stream)

    def fill_schedule(self, stream=None):
        """(Re)compute the step conditioning (into the stack's cond) and the
        final norm's modulation from the sampler weights."""
        d = self.stack.desc
        _check(lib().dmx_sampler_schedule_fill(ctypes.byref(self._sw), d.n_steps, d.batch, ctypes.c_void_p(d.cond),
                                               _p(self.sched), self.sched.numel(), _stream(stream)))
        if self.stack.mod_table is not None:
            self.stack.fill_mod_table(stream)

    def run(self, stream=None):
        _check(lib().dmx_sampler_forward(ctypes.byref(self.desc), _stream(stream)))

    def capture(self, stream):
        """Capture a whole denoising run into a hipGraph on a non-default stream."""
        g = ctypes.c_void_p()
        _check(lib().dmx_sampler_graph_create(ctypes.byref(self.desc), _stream(stream), ctypes.byref(g)))
        self._graph = g
        return self

    def replay(self, stream=None):
        if self._graph is None:
            raise DmxError(ERR_INVALID_ARG, "replay() before capture()")
        _check(lib().dmx_graph_launch(self._graph, _stream(stream)))

    def close(self):
        if self._graph is not None:
            lib().dmx_graph_destroy(self._graph)
            self._graph = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# --------------------------------------------------------------------------- lazy graph profiles
ACTION_EAGER, ACTION_CAPTURE, ACTION_REPLAY = 0, 1, 2
LAZY_GRANULE, LAZY_MAX_PROFILES = 16, 8


def lazy_bucket(prefix_len: int, max_len: int = 2048) -> int:
    """16 * ceil(prefix_len / 16); raises for lengths outside [1, max_len]."""
    return _check(int(lib().dmx_lazy_bucket(int(prefix_len), int(max_len))))


class ProfileCache:
    """At most `capacity` lazily captured graph profiles: a profile's first
    call runs eager, its second is captured and run, later calls replay.
    evict=True replaces the least recently used profile with a new one;
    evict=False runs new profiles beyond capacity eager without keeping them."""

    def __init__(self, capacity: int = LAZY_MAX_PROFILES, evict: bool = True):
        h = ctypes.c_void_p()
        _check(lib().dmx_profile_cache_create(int(capacity), int(bool(evict)), ctypes.byref(h)))
        self._h = h

    def plan(self, key: int, fingerprint: int = 0):
        """The policy step alone: (action, evicted key or -1)."""
        act, ev = ctypes.c_int32(-1), ctypes.c_int64(-2)
        _check(lib().dmx_profile_cache_plan(self._h, int(key), int(fingerprint), ctypes.byref(act), ctypes.byref(ev)))
        return int(act.value), int(ev.value)

    def keys(self):
        """Profile keys from least to most recently used."""
        buf = (ctypes.c_int64 * LAZY_MAX_PROFILES)()
        n = _check(lib().dmx_profile_cache_keys(self._h, buf))
        return [int(buf[i]) for i in range(n)]

    def run(self, sampler: "Sampler", stream) -> int:
        """One denoising run of `sampler` through the cache on `stream` (not
        the null stream); returns the action taken."""
        act = ctypes.c_int32(-1)
        _check(lib().dmx_profile_cache_run_sampler(self._h, ctypes.byref(sampler.desc), _stream(stream),
                                                   ctypes.byref(act)))
        return int(act.value)

    def close(self):
        if self._h:
            lib().dmx_profile_cache_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
