"""dmx oracle -- TEST INFRASTRUCTURE ONLY.

Python access (ctypes + numpy float64) to the plain C oracle in
``dmx_oracle.c``.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this package.  It never imports, loads or calls the
HIP library, and the HIP library never uses it.

Every function computes in float64 from the exact values it is given (bf16
inputs are upcast exactly by the caller).  Citations of the pages are in the C
source next to each step.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dmx_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, FALLBACK_EAGER = 0, 1
ERR_INVALID_ARG, ERR_BAD_BUCKETS, ERR_PREFIX_TOO_LONG = -1, -2, -3

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C99, OpenMP over independent loops)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        # DMX_ORACLE_LIB names another build of the same source (the
        # sanitizer build of the CPU tests); it is loaded as it is
        path = os.environ.get("DMX_ORACLE_LIB") or build()
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i32 = ctypes.c_int32
        dbl = ctypes.c_double
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = ctypes.c_int
        lib.orc_select_bucket.argtypes = [i32, P, i32, i32, i32, P]
        lib.orc_select_bucket.restype = ctypes.c_int
        lib.orc_linear.argtypes = [P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        lib.orc_linear.restype = None
        lib.orc_adarms.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, dbl, P, P]
        lib.orc_adarms.restype = None
        lib.orc_qkv_qknorm_rope.argtypes = [P, P, P, P] + [ctypes.c_int] * 5 + [P, dbl, dbl, P, P, P]
        lib.orc_qkv_qknorm_rope.restype = None
        lib.orc_attention.argtypes = [P] * 6 + [ctypes.c_int] * 5 + [dbl, P, P]
        lib.orc_attention.restype = None
        lib.orc_oproj_gated_residual.argtypes = [P, P, P, P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
        lib.orc_oproj_gated_residual.restype = None
        lib.orc_gelu_tanh.argtypes = [dbl]
        lib.orc_gelu_tanh.restype = dbl
        lib.orc_geglu_mlp.argtypes = [P] * 5 + [ctypes.c_int] * 3 + [P, P]
        lib.orc_geglu_mlp.restype = None
        lib.orc_layer.argtypes = [P] * 15 + [ctypes.c_int] * 7 + [i32, dbl, dbl] + [P] * 10
        lib.orc_layer.restype = None
        lib.orc_rmsnorm.argtypes = [P, P, ctypes.c_int, ctypes.c_int, dbl, P]
        lib.orc_rmsnorm.restype = None
        lib.orc_image_merge.argtypes = [P, P, P, ctypes.c_int, ctypes.c_int, P]
        lib.orc_image_merge.restype = None
        lib.orc_prefix_attention.argtypes = [P] * 4 + [ctypes.c_int] * 4 + [dbl, P]
        lib.orc_prefix_attention.restype = None
        lib.orc_prefix_layer.argtypes = [P] * 12 + [ctypes.c_int] * 6 + [dbl, dbl, P, P, P]
        lib.orc_prefix_layer.restype = None
        lib.orc_time_embedding.argtypes = [dbl, ctypes.c_int, P]
        lib.orc_time_embedding.restype = None
        lib.orc_swish.argtypes = [dbl]
        lib.orc_swish.restype = dbl
        lib.orc_time_mlp.argtypes = [P] * 5 + [ctypes.c_int, P]
        lib.orc_time_mlp.restype = None
        lib.orc_action_in.argtypes = [P, P, P] + [ctypes.c_int] * 3 + [P]
        lib.orc_action_in.restype = None
        lib.orc_final_velocity.argtypes = [P] * 6 + [ctypes.c_int] * 3 + [dbl, P]
        lib.orc_final_velocity.restype = None
        lib.orc_euler.argtypes = [P, P, ctypes.c_long, dbl]
        lib.orc_euler.restype = None
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def set_threads(n: int) -> int:
    """Set the OpenMP thread count; returns the count now in effect."""
    return int(_load().orc_set_threads(int(n)))


def select_bucket(prefix_len: int, buckets, cap: int, min_tokens: int = 0):
    """Bucket rule; returns (status, index)."""
    b = np.ascontiguousarray(np.asarray(buckets, dtype=np.int32))
    idx = np.full(1, -7, dtype=np.int32)
    st = _load().orc_select_bucket(int(prefix_len), _ptr(b), int(b.size), int(cap), int(min_tokens), _ptr(idx))
    return int(st), int(idx[0])


def linear(a, w):
    a, w = _f64(a), _f64(w)
    T, K = a.shape
    N = w.shape[0]
    y = np.empty((T, N))
    _load().orc_linear(_ptr(a), _ptr(w), T, K, N, _ptr(y))
    return y


def adarms(x, cond, w_mod, b_mod, eps=1e-6):
    """Returns (xn [T][H], mod [3H] = scale|shift|gate)."""
    x, cond, w_mod, b_mod = _f64(x), _f64(cond), _f64(w_mod), _f64(b_mod)
    T, H = x.shape
    xn = np.empty((T, H))
    mod = np.empty(3 * H)
    _load().orc_adarms(_ptr(x), _ptr(cond), _ptr(w_mod), _ptr(b_mod), T, H, float(eps), _ptr(xn), _ptr(mod))
    return xn, mod


def qkv_qknorm_rope(xn, w_qkv, q_norm, k_norm, pos, hq, hk, d, base=10000.0, eps=1e-6):
    """Returns q [T][hq][d], k [hk][T][d], v [hk][T][d]."""
    xn, w_qkv, q_norm, k_norm = _f64(xn), _f64(w_qkv), _f64(q_norm), _f64(k_norm)
    T, H = xn.shape
    pos = np.ascontiguousarray(np.asarray(pos, dtype=np.int32).reshape(T))
    q = np.empty((T, hq, d))
    k = np.empty((hk, T, d))
    v = np.empty((hk, T, d))
    _load().orc_qkv_qknorm_rope(_ptr(xn), _ptr(w_qkv), _ptr(q_norm), _ptr(k_norm), T, H, hq, hk, d,
                                _ptr(pos), float(base), float(eps), _ptr(q), _ptr(k), _ptr(v))
    return q, k, v


def attention(q, ks, vs, kp, vp, mask, scale=None, return_prob_sums=False):
    """q [C][HQ][D]; ks, vs [HK][C][D]; kp, vp [HK][P][D]; mask [P] -> ctx [C][HQ][D]."""
    q, ks, vs, kp, vp = _f64(q), _f64(ks), _f64(vs), _f64(kp), _f64(vp)
    C, HQ_, D_ = q.shape
    HK_, P, _ = kp.shape
    mask = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(P))
    if scale is None:
        scale = 1.0 / np.sqrt(D_)
    ctx = np.empty((C, HQ_, D_))
    ps = np.empty((C, HQ_))
    _load().orc_attention(_ptr(q), _ptr(ks), _ptr(vs), _ptr(kp), _ptr(vp), _ptr(mask), C, P, HQ_, HK_, D_,
                          float(scale), _ptr(ctx), _ptr(ps))
    return (ctx, ps) if return_prob_sums else ctx


def oproj_gated_residual(ctx, w_o, gate, resid):
    ctx, w_o, gate, resid = _f64(ctx), _f64(w_o), _f64(gate), _f64(resid)
    T = resid.shape[0]
    H = w_o.shape[0]
    K = w_o.shape[1]
    out = np.empty((T, H))
    _load().orc_oproj_gated_residual(_ptr(ctx.reshape(T, K)), _ptr(w_o), _ptr(gate), _ptr(resid), T, K, H, _ptr(out))
    return out


def gelu_tanh(z: float) -> float:
    return float(_load().orc_gelu_tanh(float(z)))


def geglu_mlp(xn2, w_gu, w_down, gate2, resid):
    """Returns (out [T][H], h [T][I])."""
    xn2, w_gu, w_down, gate2, resid = _f64(xn2), _f64(w_gu), _f64(w_down), _f64(gate2), _f64(resid)
    T, H = xn2.shape
    I_ = w_down.shape[1]
    out = np.empty((T, H))
    h = np.empty((T, I_))
    _load().orc_geglu_mlp(_ptr(xn2), _ptr(w_gu), _ptr(w_down), _ptr(gate2), _ptr(resid), T, H, I_, _ptr(out), _ptr(h))
    return out, h


PROBE_KEYS = ("xn1", "mod1", "q", "ks", "vs", "ctx", "x1", "xn2", "mod2")


def layer(x, cond, w: dict, kp, vp, mask, pos0: int, hq=8, hk=4, d=256,
          base=10000.0, eps=1e-6, probes=False):
    """One action-expert layer for one request.  x [C][H]; cond [H]; w: float
    arrays keyed like the weight dict; kp, vp [HK][P][D]; mask [P].
    Returns out [C][H], or (out, probes dict) when probes=True."""
    x, cond = _f64(x), _f64(cond)
    C, H = x.shape
    I_ = w["w_down"].shape[1]
    P = kp.shape[1]
    ww = {k: _f64(v) for k, v in w.items()}
    kp, vp = _f64(kp), _f64(vp)
    mask = np.ascontiguousarray(np.asarray(mask, dtype=np.uint8).reshape(P))
    out = np.empty((C, H))
    pr = None
    if probes:
        pr = {"xn1": np.empty((C, H)), "mod1": np.empty(3 * H), "q": np.empty((C, hq, d)),
              "ks": np.empty((hk, C, d)), "vs": np.empty((hk, C, d)), "ctx": np.empty((C, hq, d)),
              "x1": np.empty((C, H)), "xn2": np.empty((C, H)), "mod2": np.empty(3 * H)}
    pp = [None] * 9 if pr is None else [pr[k] for k in PROBE_KEYS]
    _load().orc_layer(_ptr(x), _ptr(cond), _ptr(ww["w_mod1"]), _ptr(ww["b_mod1"]), _ptr(ww["w_qkv"]),
                      _ptr(ww["q_norm"]), _ptr(ww["k_norm"]), _ptr(ww["w_o"]), _ptr(ww["w_mod2"]),
                      _ptr(ww["b_mod2"]), _ptr(ww["w_gu"]), _ptr(ww["w_down"]), _ptr(kp), _ptr(vp),
                      _ptr(mask), C, P, H, I_, hq, hk, d, int(pos0), float(base), float(eps),
                      _ptr(out), *[_ptr(a) for a in pp])
    return (out, pr) if probes else out


# ----------------------------------------------------------------------------- prefix side
def rmsnorm(x, w, eps=1e-6):
    """Rows of x [T][H] RMS-normalised with the (1 + w) weight."""
    x, w = _f64(x), _f64(w)
    T, H = x.shape
    y = np.empty((T, H))
    _load().orc_rmsnorm(_ptr(x), _ptr(w), T, H, float(eps), _ptr(y))
    return y


def image_merge(tok, img, idx):
    """tok [T][H], img [NI][H], idx [T] (row of img, or -1 for the text embedding)."""
    tok, img = _f64(tok), _f64(img)
    T, H = tok.shape
    idx = np.ascontiguousarray(np.asarray(idx, dtype=np.int32).reshape(T))
    out = np.empty((T, H))
    _load().orc_image_merge(_ptr(tok), _ptr(img), _ptr(idx), T, H, _ptr(out))
    return out


def prefix_attention(q, k, v, valid, scale=None):
    """q [T][HQ][D]; k, v [HK][T][D]; valid [T] -> ctx [T][HQ][D] (prefix-causal mask)."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, HQ_, D_ = q.shape
    HK_ = k.shape[0]
    valid = np.ascontiguousarray(np.asarray(valid, dtype=np.uint8).reshape(T))
    if scale is None:
        scale = 1.0 / np.sqrt(D_)
    ctx = np.empty((T, HQ_, D_))
    _load().orc_prefix_attention(_ptr(q), _ptr(k), _ptr(v), _ptr(valid), T, HQ_, HK_, D_, float(scale), _ptr(ctx))
    return ctx


PREFIX_WEIGHTS = ("w_in", "w_qkv", "q_norm", "k_norm", "w_o", "w_post_attn", "w_pre_ffn", "w_gu", "w_down",
                  "w_post_ffn")


def prefix_layer(x, w: dict, valid, hq=8, hk=4, d=256, base=10000.0, eps=1e-6):
    """One prefix decoder layer.  x [T][H]; w keyed by PREFIX_WEIGHTS; valid [T].
    Returns (out [T][H], k [hk][T][d], v [hk][T][d])."""
    x = _f64(x)
    T, H = x.shape
    ww = {k: _f64(w[k]) for k in PREFIX_WEIGHTS}
    I_ = ww["w_down"].shape[1]
    valid = np.ascontiguousarray(np.asarray(valid, dtype=np.uint8).reshape(T))
    out = np.empty((T, H))
    k = np.empty((hk, T, d))
    v = np.empty((hk, T, d))
    _load().orc_prefix_layer(_ptr(x), *[_ptr(ww[n]) for n in PREFIX_WEIGHTS], _ptr(valid), T, H, I_, hq, hk, d,
                             float(base), float(eps), _ptr(out), _ptr(k), _ptr(v))
    return out, k, v


# ----------------------------------------------------------------------------- denoise sampler
SAMPLER_WEIGHTS = ("w_in", "b_in", "w_t1", "b_t1", "w_t2", "b_t2", "w_fmod", "b_fmod", "w_out", "b_out")


def step_time(k: int, n_steps: int) -> float:
    """t_k = 1 - k / n: step 0 starts from noise at t = 1."""
    return 1.0 - k / n_steps


def time_embedding(t: float, h: int = 1024):
    out = np.empty(h)
    _load().orc_time_embedding(float(t), int(h), _ptr(out))
    return out


def swish(z: float) -> float:
    return float(_load().orc_swish(float(z)))


def time_mlp(temb, w1, b1, w2, b2):
    """cond = swish(W2 swish(W1 temb + b1) + b2)."""
    temb, w1, b1, w2, b2 = (_f64(a) for a in (temb, w1, b1, w2, b2))
    H = temb.size
    cond = np.empty(H)
    _load().orc_time_mlp(_ptr(temb), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), H, _ptr(cond))
    return cond


def time_condition(t: float, sw: dict):
    """Conditioning vector of diffusion time t from the sampler weights."""
    H = sw["b_t1"].size
    return time_mlp(time_embedding(t, H), sw["w_t1"], sw["b_t1"], sw["w_t2"], sw["b_t2"])


def action_in(a, w_in, b_in):
    """a [C][A] -> x [C][H] = a W_in^T + b_in."""
    a, w_in, b_in = _f64(a), _f64(w_in), _f64(b_in)
    C, A = a.shape
    H = w_in.shape[0]
    x = np.empty((C, H))
    _load().orc_action_in(_ptr(a), _ptr(w_in), _ptr(b_in), C, A, H, _ptr(x))
    return x


def final_velocity(x, cond, w_f, b_f, w_out, b_out, eps=1e-6):
    """Final AdaRMS norm of x [C][H] with [scale | shift] = W_f cond + b_f, then
    v = xf W_out^T + b_out -> [C][A]."""
    x, cond, w_f, b_f, w_out, b_out = (_f64(a) for a in (x, cond, w_f, b_f, w_out, b_out))
    C, H = x.shape
    A = w_out.shape[0]
    v = np.empty((C, A))
    _load().orc_final_velocity(_ptr(x), _ptr(cond), _ptr(w_f), _ptr(b_f), _ptr(w_out), _ptr(b_out), C, H, A,
                               float(eps), _ptr(v))
    return v


def euler(a, v, dt: float):
    a = _f64(a).copy()
    v = _f64(v)
    _load().orc_euler(_ptr(a), _ptr(v), a.size, float(dt))
    return a


def sampler_step(a, k: int, n_steps: int, sw: dict, layers, kps, vps, mask, pos0: int, **dims):
    """One denoising step k of n for one request: a [C][A] -> (next a, v).
    layers: per-layer weight dicts; kps / vps: per-layer [HK][P][D] caches;
    dims: head counts / size passed to layer()."""
    cond = time_condition(step_time(k, n_steps), sw)
    x = action_in(a, sw["w_in"], sw["b_in"])
    for w, kp, vp in zip(layers, kps, vps):
        x = layer(x, cond, w, kp, vp, mask, pos0, **dims)
    v = final_velocity(x, cond, sw["w_fmod"], sw["b_fmod"], sw["w_out"], sw["b_out"])
    return euler(a, v, -1.0 / n_steps), v


def sampler(noise, n_steps: int, sw: dict, layers, kps, vps, mask, pos0: int, **dims):
    """The whole denoising run for one request from noise [C][A]; returns the
    actions after every step, [n_steps][C][A]."""
    a = _f64(noise)
    traj = []
    for k in range(n_steps):
        a, _ = sampler_step(a, k, n_steps, sw, layers, kps, vps, mask, pos0, **dims)
        traj.append(a)
    return np.stack(traj)


# ----------------------------------------------------------------------------- lazy graph profiles
# The default backend's row of [Art §5]'s comparison table: prefix lengths
# bucketed by 16 tokens, at most 8 profiles, a shape's first call eager and
# its second captured.  A plain model of that policy in Python (host logic,
# nothing numeric): a list of profiles ordered from least to most recently
# used.
EAGER, CAPTURE, REPLAY = 0, 1, 2


def lazy_bucket(prefix_len: int, max_len: int):
    """The 16-token bucket of a prefix length, or None outside [1, max_len]."""
    if prefix_len < 1 or prefix_len > max_len:
        return None
    return -(-prefix_len // 16) * 16


def lazy_profile_actions(calls, capacity: int = 8, evict: bool = True):
    """calls: sequence of (key, fingerprint).  Returns the (action, evicted
    key or -1) of every call and the final keys, least recently used first.
    A profile counts its calls: the first runs eager, the second is captured,
    the rest replay; other buffers (fingerprint) start the count again.  A new
    key when `capacity` profiles exist replaces the least recently used one
    (evict) or runs eager without being kept."""
    order = []   # [key, fingerprint, calls], least recently used first
    out = []
    for key, fp in calls:
        hit = [p for p in order if p[0] == key]
        if hit:
            p = hit[0]
            order.remove(p)
            order.append(p)
            if p[1] != fp:
                p[1], p[2] = fp, 0
            p[2] += 1
            out.append(((EAGER, CAPTURE)[p[2] - 1] if p[2] <= 2 else REPLAY, -1))
            continue
        evicted = -1
        if len(order) == capacity:
            if not evict:
                out.append((EAGER, -1))
                continue
            evicted = order.pop(0)[0]
        order.append([key, fp, 1])
        out.append((EAGER, evicted))
    return out, [p[0] for p in order]


def prefix_layer_rows(x, w: dict, valid, rows, hq=8, hk=4, d=256, base=10000.0, eps=1e-6):
    """prefix_layer's output at the token rows `rows` only, plus the whole K/V
    cache: every row's K and V (and the attention of the chosen rows over all
    earlier rows) is still computed; the projections and MLP after the
    attention run for the chosen rows only.  The same steps in the same
    order as orc_prefix_layer, for token counts where the full layer is too
    slow.  Returns (out [len(rows)][H], k [hk][T][d], v [hk][T][d])."""
    x = _f64(x)
    T, H = x.shape
    ww = {kk: _f64(w[kk]) for kk in PREFIX_WEIGHTS}
    rows = np.asarray(rows, dtype=np.int64)
    xn = rmsnorm(x, ww["w_in"], eps)
    q, k, v = qkv_qknorm_rope(xn, ww["w_qkv"], ww["q_norm"], ww["k_norm"], np.arange(T, dtype=np.int32), hq, hk, d,
                              base, eps)
    ctx = prefix_attention(q, k, v, valid)[rows].reshape(len(rows), hq * d)
    x1 = x[rows] + rmsnorm(linear(ctx, ww["w_o"]), ww["w_post_attn"], eps)
    gu = linear(rmsnorm(x1, ww["w_pre_ffn"], eps), ww["w_gu"])
    I_ = gu.shape[1] // 2
    hdn = np.vectorize(gelu_tanh)(gu[:, :I_]) * gu[:, I_:]
    out = x1 + rmsnorm(linear(hdn, ww["w_down"]), ww["w_post_ffn"], eps)
    return out, k, v
