"""Pins of the oracle against facts that do not come from the oracle itself:
the pages' stated rules (golden bucket cases), library routines (numpy /
torch float64 matmul, RMS norm, SDPA attention, tanh-GELU, complex rotation),
brute force on tiny shapes, closed forms and invariants.

Each test is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, a mask that leaks) fails it.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bucket_cases.txt")
STATUS = {"OK": orc.OK, "FALLBACK_EAGER": orc.FALLBACK_EAGER, "INVALID_ARG": orc.ERR_INVALID_ARG,
          "BAD_BUCKETS": orc.ERR_BAD_BUCKETS, "PREFIX_TOO_LONG": orc.ERR_PREFIX_TOO_LONG}


def read_golden():
    cases = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        b, cap, mt, ln, st, ch = [f.strip() for f in line.split("|")]
        buckets = [] if b == "-" else [int(v) for v in b.split(",")]
        cases.append((buckets, int(cap), int(mt), int(ln), STATUS[st], None if ch == "-" else int(ch)))
    return cases


# ---------------------------------------------------------------- bucket rule
@pytest.mark.parametrize("case", read_golden())
def test_bucket_golden(case):
    buckets, cap, mt, ln, st, chosen = case
    s, idx = orc.select_bucket(ln, buckets, cap, mt)
    assert s == st
    if chosen is None:
        assert idx == -1
    else:
        assert buckets[idx] == chosen


def test_bucket_properties_exhaustive():
    """Defining properties over every length: the chosen bucket holds the
    prefix and no smaller eligible bucket does."""
    for buckets, cap in [((576, 704, 768, 896, 1024), 1024), ((2048,), 2048), ((576, 704), 1024),
                         ((576, 704, 768, 896, 1024), 2048), ((100, 200, 300), 300)]:
        for mt in (0, 650):
            for ln in range(-2, cap + 80):
                s, idx = orc.select_bucket(ln, buckets, cap, mt)
                eligible = [b for b in buckets if b >= mt]
                if ln <= 0:
                    assert s == orc.ERR_INVALID_ARG
                elif ln > cap:
                    assert s == orc.ERR_PREFIX_TOO_LONG
                elif any(b >= ln for b in eligible):
                    assert s == orc.OK
                    b = buckets[idx]
                    assert b >= ln and b >= mt
                    assert all(not (e >= ln and e < b) for e in eligible)
                else:
                    assert s == orc.FALLBACK_EAGER and idx == -1


# ---------------------------------------------------------------- helpers
def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def t64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def rope_complex(u, pos, base):
    """Rotation as complex multiplication: the pair (u_j, u_{j+D/2}) is the
    complex number u_j + i u_{j+D/2}, multiplied by exp(i pos base^(-2j/D))."""
    D = u.shape[-1]
    half = D // 2
    z = torch.complex(u[..., :half], u[..., half:])
    j = torch.arange(half, dtype=torch.float64)
    theta = pos * base ** (-2.0 * j / D)
    z = z * torch.polar(torch.ones_like(theta), theta)
    return torch.cat([z.real, z.imag], dim=-1)


# ---------------------------------------------------------------- linear
def test_linear_matches_numpy_matmul():
    r = rng(1)
    a = r.standard_normal((7, 33))
    w = r.standard_normal((19, 33))
    np.testing.assert_allclose(orc.linear(a, w), a @ w.T, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- AdaRMS
def test_adarms_zero_modulation_is_plain_rmsnorm():
    r = rng(2)
    T, H = 5, 64
    x = r.standard_normal((T, H)) * 3.0
    cond = r.standard_normal(H)
    xn, mod = orc.adarms(x, cond, np.zeros((3 * H, H)), np.zeros(3 * H), eps=1e-6)
    ref = F.rms_norm(t64(x), (H,), eps=1e-6).numpy()
    np.testing.assert_allclose(xn, ref, rtol=1e-12, atol=1e-12)
    assert np.all(mod == 0.0)


def test_adarms_scale_shift_gate_chunks():
    """With W_mod = 0 the modulation is the bias; its thirds are scale, shift
    and gate in that order."""
    r = rng(3)
    T, H = 4, 32
    x = r.standard_normal((T, H))
    s, sh, g = r.standard_normal(H), r.standard_normal(H), r.standard_normal(H)
    xn, mod = orc.adarms(x, r.standard_normal(H), np.zeros((3 * H, H)), np.concatenate([s, sh, g]))
    ref = F.rms_norm(t64(x), (H,), weight=t64(1.0 + s), eps=1e-6).numpy() + sh
    np.testing.assert_allclose(xn, ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(mod[2 * H:], g)


def test_adarms_modulation_is_affine_in_cond():
    r = rng(4)
    H = 16
    w = r.standard_normal((3 * H, H))
    b = r.standard_normal(3 * H)
    cond = r.standard_normal(H)
    _, mod = orc.adarms(r.standard_normal((2, H)), cond, w, b)
    np.testing.assert_allclose(mod, w @ cond + b, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- QKV + QK-norm + RoPE
def _qkv_case(seed, T=3, H=24, hq=4, hk=2, d=8):
    r = rng(seed)
    return (r.standard_normal((T, H)), r.standard_normal(((hq + 2 * hk) * d, H)),
            0.1 * r.standard_normal(d), 0.1 * r.standard_normal(d), hq, hk, d)


def test_qkv_matches_library_composition():
    xn, w, qn, kn, hq, hk, d = _qkv_case(5)
    T = xn.shape[0]
    pos = np.array([7, 100, 2049])
    q, k, v = orc.qkv_qknorm_rope(xn, w, qn, kn, pos, hq, hk, d, base=10000.0, eps=1e-6)
    qkv = t64(xn) @ t64(w).T
    qr = qkv[:, :hq * d].reshape(T, hq, d)
    kr = qkv[:, hq * d:(hq + hk) * d].reshape(T, hk, d)
    vr = qkv[:, (hq + hk) * d:].reshape(T, hk, d)
    qr = F.rms_norm(qr, (d,), weight=1.0 + t64(qn), eps=1e-6)
    kr = F.rms_norm(kr, (d,), weight=1.0 + t64(kn), eps=1e-6)
    p = t64(pos).reshape(T, 1, 1)
    qr = rope_complex(qr, p, 10000.0)
    kr = rope_complex(kr, p, 10000.0)
    np.testing.assert_allclose(q, qr.numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(k, kr.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(v, vr.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-12)


def test_rope_position_zero_is_identity():
    xn, w, qn, kn, hq, hk, d = _qkv_case(6, T=1)
    q, k, _ = orc.qkv_qknorm_rope(xn, w, qn, kn, [0], hq, hk, d)
    qkv = t64(xn) @ t64(w).T
    qr = F.rms_norm(qkv[:, :hq * d].reshape(1, hq, d), (d,), weight=1.0 + t64(qn), eps=1e-6)
    np.testing.assert_allclose(q, qr.numpy(), rtol=1e-12, atol=1e-12)


def test_rope_preserves_pair_norms():
    xn, w, qn, kn, hq, hk, d = _qkv_case(7, T=1)
    q0, k0, _ = orc.qkv_qknorm_rope(xn, w, qn, kn, [0], hq, hk, d)
    q1, k1, _ = orc.qkv_qknorm_rope(xn, w, qn, kn, [1234], hq, hk, d)
    half = d // 2
    for a, b in ((q0, q1), (k0, k1)):
        n0 = a[..., :half] ** 2 + a[..., half:] ** 2
        n1 = b[..., :half] ** 2 + b[..., half:] ** 2
        np.testing.assert_allclose(n0, n1, rtol=1e-12)
        assert not np.allclose(a, b)


def test_rope_dot_depends_on_relative_position_only():
    """For one token's query head 0 and key head 0, RoPE(q, a) . RoPE(k, b)
    must depend on a - b only."""
    xn, w, qn, kn, hq, hk, d = _qkv_case(8, T=1)

    def dot(a, b):
        qa, _, _ = orc.qkv_qknorm_rope(xn, w, qn, kn, [a], hq, hk, d)
        _, kb, _ = orc.qkv_qknorm_rope(xn, w, qn, kn, [b], hq, hk, d)
        return float(qa[0, 0] @ kb[0, 0])

    ref = dot(5, 2)
    for a, b in ((13, 10), (1003, 1000), (3, 0)):
        assert abs(dot(a, b) - ref) < 1e-9
    assert abs(dot(2, 5) - ref) > 1e-6  # not symmetric in general


# ---------------------------------------------------------------- attention
def _attn_case(seed, C=3, P=9, hq=4, hk=2, d=8, frac_visible=0.6):
    r = rng(seed)
    q = r.standard_normal((C, hq, d))
    ks, vs = r.standard_normal((hk, C, d)), r.standard_normal((hk, C, d))
    kp, vp = r.standard_normal((hk, P, d)), r.standard_normal((hk, P, d))
    mask = (r.random(P) < frac_visible).astype(np.uint8)
    return q, ks, vs, kp, vp, mask


def bruteforce_attention(q, ks, vs, kp, vp, mask, scale):
    """Full logits matrix over [prefix ; suffix] with -inf where masked, KV heads
    repeated to the query heads."""
    C, hq, d = q.shape
    hk = kp.shape[0]
    K = np.concatenate([kp, ks], axis=1).repeat(hq // hk, axis=0)   # [hq][P+C][d]
    V = np.concatenate([vp, vs], axis=1).repeat(hq // hk, axis=0)
    allow = np.concatenate([mask != 0, np.ones(C, dtype=bool)])
    out = np.empty_like(q)
    for h in range(hq):
        s = scale * (q[:, h, :] @ K[h].T)                         # [C][P+C]
        s = np.where(allow[None, :], s, -np.inf)
        s = s - s.max(axis=1, keepdims=True)
        p = np.exp(s)
        p /= p.sum(axis=1, keepdims=True)
        out[:, h, :] = p @ V[h]
    return out


@pytest.mark.parametrize("seed", [10, 11, 12, 13])
def test_attention_bruteforce(seed):
    q, ks, vs, kp, vp, mask = _attn_case(seed)
    ctx = orc.attention(q, ks, vs, kp, vp, mask)
    ref = bruteforce_attention(q, ks, vs, kp, vp, mask, 1 / math.sqrt(q.shape[2]))
    np.testing.assert_allclose(ctx, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("seed", [20, 21])
def test_attention_matches_torch_sdpa_gqa(seed):
    q, ks, vs, kp, vp, mask = _attn_case(seed, C=5, P=17, hq=8, hk=4, d=16)
    C = q.shape[0]
    ctx = orc.attention(q, ks, vs, kp, vp, mask)
    Q = t64(q).permute(1, 0, 2).unsqueeze(0)                    # [1][hq][C][d]
    K = torch.cat([t64(kp), t64(ks)], dim=1).unsqueeze(0)       # [1][hk][P+C][d]
    V = torch.cat([t64(vp), t64(vs)], dim=1).unsqueeze(0)
    allow = torch.cat([torch.from_numpy(mask != 0), torch.ones(C, dtype=torch.bool)])
    ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=allow.expand(C, -1), enable_gqa=True)
    np.testing.assert_allclose(ctx, ref[0].permute(1, 0, 2).numpy(), rtol=1e-10, atol=1e-12)


def test_attention_softmax_rows_sum_to_one():
    q, ks, vs, kp, vp, mask = _attn_case(30, C=4, P=40, hq=8, hk=4, d=32)
    q = q * 5.0  # sharp distributions
    _, ps = orc.attention(q, ks, vs, kp, vp, mask, return_prob_sums=True)
    assert np.max(np.abs(ps - 1.0)) <= 1e-12


def test_attention_constant_values_give_constant_output():
    q, ks, vs, kp, vp, mask = _attn_case(31)
    ctx = orc.attention(q, ks, np.ones_like(vs), kp, np.ones_like(vp), mask)
    np.testing.assert_allclose(ctx, 1.0, rtol=0, atol=1e-14)


@pytest.mark.parametrize("poison", [np.nan, np.inf, -np.inf, 3e4, -3e4])
def test_attention_masked_rows_never_read(poison):
    q, ks, vs, kp, vp, mask = _attn_case(32, P=13)
    assert (mask == 0).any() and (mask != 0).any()
    clean = orc.attention(q, ks, vs, np.where(mask[None, :, None] != 0, kp, 0.0),
                          np.where(mask[None, :, None] != 0, vp, 0.0), mask)
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[:, mask == 0, :] = poison
    vp2[:, mask == 0, :] = poison
    dirty = orc.attention(q, ks, vs, kp2, vp2, mask)
    assert np.array_equal(clean, dirty)  # bit-identical


def test_attention_gqa_equals_duplicated_kv_heads():
    q, ks, vs, kp, vp, mask = _attn_case(33, C=3, P=11, hq=8, hk=4, d=8)
    a = orc.attention(q, ks, vs, kp, vp, mask)
    b = orc.attention(q, ks.repeat(2, axis=0), vs.repeat(2, axis=0), kp.repeat(2, axis=0),
                      vp.repeat(2, axis=0), mask)
    assert np.array_equal(a, b)


def test_attention_zero_query_is_mean_of_visible_values():
    q, ks, vs, kp, vp, mask = _attn_case(34, P=15)
    q = np.zeros_like(q)
    ctx = orc.attention(q, ks, vs, kp, vp, mask)
    hq, hk = q.shape[1], kp.shape[0]
    for h in range(hq):
        g = h // (hq // hk)
        rows = np.concatenate([vp[g][mask != 0], vs[g]], axis=0)
        np.testing.assert_allclose(ctx[:, h, :], np.broadcast_to(rows.mean(axis=0), ctx[:, h, :].shape),
                                   rtol=1e-12, atol=1e-14)


def test_attention_all_prefix_masked_reads_suffix_only():
    q, ks, vs, kp, vp, mask = _attn_case(35)
    ctx = orc.attention(q, ks, vs, kp * np.nan, vp * np.nan, np.zeros_like(mask))
    assert np.isfinite(ctx).all()
    ref = bruteforce_attention(q, ks, vs, kp[:, :0], vp[:, :0], mask[:0], 1 / math.sqrt(q.shape[2]))
    np.testing.assert_allclose(ctx, ref, rtol=1e-10, atol=1e-12)


def test_attention_group_mapping_is_consecutive_pairs():
    """Query head h reads KV head h // 2: changing KV head 1 changes only
    query heads 2 and 3."""
    q, ks, vs, kp, vp, mask = _attn_case(36, hq=8, hk=4)
    a = orc.attention(q, ks, vs, kp, vp, mask)
    vs2 = vs.copy()
    vs2[1] += 1.0
    b = orc.attention(q, ks, vs2, kp, vp, mask)
    changed = [h for h in range(8) if not np.array_equal(a[:, h], b[:, h])]
    assert changed == [2, 3]


# ---------------------------------------------------------------- GEGLU / MLP
def test_gelu_tanh_matches_torch():
    for z in (-6.0, -1.0, -0.3, 0.0, 0.5, 1.0, 2.5, 7.0):
        ref = F.gelu(torch.tensor(z, dtype=torch.float64), approximate="tanh").item()
        assert abs(orc.gelu_tanh(z) - ref) <= 1e-15 * max(1.0, abs(ref))


def test_geglu_matches_library_composition():
    r = rng(40)
    T, H, I_ = 3, 16, 24
    xn2 = r.standard_normal((T, H))
    w_gu = r.standard_normal((2 * I_, H)) * 0.3
    w_d = r.standard_normal((H, I_)) * 0.3
    g2, resid = r.standard_normal(H), r.standard_normal((T, H))
    out, h = orc.geglu_mlp(xn2, w_gu, w_d, g2, resid)
    a = F.linear(t64(xn2), t64(w_gu[:I_]))
    u = F.linear(t64(xn2), t64(w_gu[I_:]))
    hr = F.gelu(a, approximate="tanh") * u
    ref = t64(resid) + t64(g2) * F.linear(hr, t64(w_d))
    np.testing.assert_allclose(h, hr.numpy(), rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_geglu_zero_gate_weights_add_nothing():
    r = rng(41)
    T, H, I_ = 2, 8, 12
    w_gu = r.standard_normal((2 * I_, H))
    w_gu[:I_] = 0.0
    resid = r.standard_normal((T, H))
    out, h = orc.geglu_mlp(r.standard_normal((T, H)), w_gu, r.standard_normal((H, I_)),
                           r.standard_normal(H), resid)
    assert np.all(h == 0.0)
    assert np.array_equal(out, resid)


def test_oproj_gated_residual_matches_matmul():
    r = rng(42)
    T, K, H = 3, 32, 8
    ctx, w_o = r.standard_normal((T, K)), r.standard_normal((H, K))
    gate, resid = r.standard_normal(H), r.standard_normal((T, H))
    out = orc.oproj_gated_residual(ctx, w_o, gate, resid)
    np.testing.assert_allclose(out, resid + gate * (ctx @ w_o.T), rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------- whole layer
def _tiny_layer(seed, H=16, I_=24, hq=4, hk=2, d=8, C=3, P=9, std=0.3):
    r = rng(seed)
    w = {"w_mod1": std * r.standard_normal((3 * H, H)), "b_mod1": std * r.standard_normal(3 * H),
         "w_qkv": std * r.standard_normal(((hq + 2 * hk) * d, H)),
         "q_norm": std * r.standard_normal(d), "k_norm": std * r.standard_normal(d),
         "w_o": std * r.standard_normal((H, hq * d)),
         "w_mod2": std * r.standard_normal((3 * H, H)), "b_mod2": std * r.standard_normal(3 * H),
         "w_gu": std * r.standard_normal((2 * I_, H)), "w_down": std * r.standard_normal((H, I_))}
    x, cond = r.standard_normal((C, H)), r.standard_normal(H)
    kp, vp = r.standard_normal((hk, P, d)), r.standard_normal((hk, P, d))
    mask = (r.random(P) < 0.6).astype(np.uint8)
    return w, x, cond, kp, vp, mask, dict(hq=hq, hk=hk, d=d)


def torch_layer(w, x, cond, kp, vp, mask, pos0, hq, hk, d, base=10000.0, eps=1e-6):
    """The layer assembled from torch float64 library routines."""
    W = {k: t64(v) for k, v in w.items()}
    X, cnd = t64(x), t64(cond)
    C, H = X.shape
    m1 = F.linear(cnd, W["w_mod1"], W["b_mod1"])
    sc1, sh1, g1 = m1[:H], m1[H:2 * H], m1[2 * H:]
    xn = F.rms_norm(X, (H,), weight=1.0 + sc1, eps=eps) + sh1
    qkv = F.linear(xn, W["w_qkv"])
    q = qkv[:, :hq * d].reshape(C, hq, d)
    k = qkv[:, hq * d:(hq + hk) * d].reshape(C, hk, d)
    v = qkv[:, (hq + hk) * d:].reshape(C, hk, d)
    q = F.rms_norm(q, (d,), weight=1.0 + W["q_norm"], eps=eps)
    k = F.rms_norm(k, (d,), weight=1.0 + W["k_norm"], eps=eps)
    pos = (pos0 + torch.arange(C, dtype=torch.float64)).reshape(C, 1, 1)
    q, k = rope_complex(q, pos, base), rope_complex(k, pos, base)
    K = torch.cat([t64(kp), k.permute(1, 0, 2)], dim=1).unsqueeze(0)
    V = torch.cat([t64(vp), v.permute(1, 0, 2)], dim=1).unsqueeze(0)
    allow = torch.cat([torch.from_numpy(mask != 0), torch.ones(C, dtype=torch.bool)])
    att = F.scaled_dot_product_attention(q.permute(1, 0, 2).unsqueeze(0), K, V,
                                         attn_mask=allow.expand(C, -1), enable_gqa=True)
    ctx = att[0].permute(1, 0, 2).reshape(C, hq * d)
    x1 = X + g1 * F.linear(ctx, W["w_o"])
    m2 = F.linear(cnd, W["w_mod2"], W["b_mod2"])
    sc2, sh2, g2 = m2[:H], m2[H:2 * H], m2[2 * H:]
    xn2 = F.rms_norm(x1, (H,), weight=1.0 + sc2, eps=eps) + sh2
    I_ = W["w_down"].shape[1]
    hdn = F.gelu(F.linear(xn2, W["w_gu"][:I_]), approximate="tanh") * F.linear(xn2, W["w_gu"][I_:])
    return (x1 + g2 * F.linear(hdn, W["w_down"])).numpy()


@pytest.mark.parametrize("seed,pos0", [(50, 9), (51, 1024), (52, 0)])
def test_layer_matches_library_composition(seed, pos0):
    w, x, cond, kp, vp, mask, dims = _tiny_layer(seed)
    out = orc.layer(x, cond, w, kp, vp, mask, pos0, **dims)
    ref = torch_layer(w, x, cond, kp, vp, mask, pos0, **dims)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-11)


def test_layer_zero_gates_is_identity():
    w, x, cond, kp, vp, mask, dims = _tiny_layer(53)
    H = x.shape[1]
    for k in ("w_mod1", "w_mod2"):
        w[k][2 * H:] = 0.0
    for k in ("b_mod1", "b_mod2"):
        w[k][2 * H:] = 0.0
    out = orc.layer(x, cond, w, kp, vp, mask, 5, **dims)
    assert np.array_equal(out, x)


def test_layer_probes_are_consistent_with_stages():
    w, x, cond, kp, vp, mask, dims = _tiny_layer(54)
    out, p = orc.layer(x, cond, w, kp, vp, mask, 7, probes=True, **dims)
    xn1, mod1 = orc.adarms(x, cond, w["w_mod1"], w["b_mod1"])
    np.testing.assert_array_equal(xn1, p["xn1"])
    np.testing.assert_array_equal(mod1, p["mod1"])
    ctx = orc.attention(p["q"], p["ks"], p["vs"], kp, vp, mask)
    np.testing.assert_array_equal(ctx, p["ctx"])


# ---------------------------------------------------------------- prefix side
def test_rmsnorm_matches_torch_and_closed_form():
    r = rng(60)
    x, w = r.standard_normal((5, 24)), 0.3 * r.standard_normal(24)
    ref = F.rms_norm(t64(x), (24,), weight=1.0 + t64(w), eps=1e-6).numpy()
    np.testing.assert_allclose(orc.rmsnorm(x, w), ref, rtol=1e-13, atol=1e-14)
    # a constant row c: every element becomes c / sqrt(c^2 + eps) * (1 + w_j)
    c = -2.5
    y = orc.rmsnorm(np.full((1, 8), c), np.arange(8) / 10.0)
    np.testing.assert_allclose(y[0], c / np.sqrt(c * c + 1e-6) * (1.0 + np.arange(8) / 10.0), rtol=1e-14)


def test_image_merge_takes_image_rows_where_indexed():
    r = rng(61)
    tok, img = r.standard_normal((7, 5)), r.standard_normal((3, 5))
    idx = np.array([-1, 0, 1, -1, 2, 2, -1], np.int32)
    out = orc.image_merge(tok, img, idx)
    for t in range(7):
        np.testing.assert_array_equal(out[t], img[idx[t]] if idx[t] >= 0 else tok[t])
    np.testing.assert_array_equal(orc.image_merge(tok, img, np.full(7, -1, np.int32)), tok)


def _prefix_qkv(seed, T=11, hq=4, hk=2, d=8):
    r = rng(seed)
    return r.standard_normal((T, hq, d)), r.standard_normal((hk, T, d)), r.standard_normal((hk, T, d))


def test_prefix_attention_all_valid_is_causal_sdpa():
    q, k, v = _prefix_qkv(62)
    T = q.shape[0]
    ctx = orc.prefix_attention(q, k, v, np.ones(T, np.uint8))
    ref = F.scaled_dot_product_attention(t64(q).permute(1, 0, 2).unsqueeze(0), t64(k).unsqueeze(0),
                                         t64(v).unsqueeze(0), is_causal=True, enable_gqa=True)
    np.testing.assert_allclose(ctx, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_prefix_attention_masked_keys_match_sdpa_and_edge_rows():
    q, k, v = _prefix_qkv(63, T=13)
    T, hq = q.shape[0], q.shape[1]
    valid = np.ones(T, np.uint8)
    valid[[0, 4, 5, 12]] = 0
    ctx = orc.prefix_attention(q, k, v, valid)
    allow = torch.tril(torch.ones(T, T, dtype=torch.bool)) & torch.from_numpy(valid != 0).unsqueeze(0)
    rows = [i for i in range(T) if allow[i].any()]
    ref = F.scaled_dot_product_attention(t64(q).permute(1, 0, 2).unsqueeze(0), t64(k).unsqueeze(0),
                                         t64(v).unsqueeze(0), attn_mask=allow, enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    np.testing.assert_allclose(ctx[rows], ref[rows], rtol=1e-12, atol=1e-13)
    # token 0 is invalid and sees no key: zero output; token 1 sees only key 1: its value row
    assert np.all(ctx[0] == 0.0)
    for h in range(hq):
        np.testing.assert_allclose(ctx[1, h], v[h // (hq // k.shape[0]), 1], rtol=1e-14)
    # poisoned invisible keys change nothing
    k2, v2 = k.copy(), v.copy()
    k2[:, valid == 0] = np.nan
    v2[:, valid == 0] = np.inf
    np.testing.assert_array_equal(orc.prefix_attention(q, k2, v2, valid), ctx)


def _tiny_prefix(seed, T=9, H=16, I_=24, hq=4, hk=2, d=8, std=0.3):
    r = rng(seed)
    w = {"w_in": std * r.standard_normal(H), "w_qkv": std * r.standard_normal(((hq + 2 * hk) * d, H)),
         "q_norm": std * r.standard_normal(d), "k_norm": std * r.standard_normal(d),
         "w_o": std * r.standard_normal((H, hq * d)), "w_post_attn": std * r.standard_normal(H),
         "w_pre_ffn": std * r.standard_normal(H), "w_gu": std * r.standard_normal((2 * I_, H)),
         "w_down": std * r.standard_normal((H, I_)), "w_post_ffn": std * r.standard_normal(H)}
    x = r.standard_normal((T, H))
    valid = np.ones(T, np.uint8)
    valid[T - 2:] = 0
    return w, x, valid, dict(hq=hq, hk=hk, d=d)


def torch_prefix_layer(w, x, valid, hq, hk, d, base=10000.0, eps=1e-6):
    """The prefix layer assembled from torch float64 library routines."""
    W = {k: t64(v) for k, v in w.items()}
    X = t64(x)
    T, H = X.shape
    xn = F.rms_norm(X, (H,), weight=1.0 + W["w_in"], eps=eps)
    qkv = F.linear(xn, W["w_qkv"])
    q = F.rms_norm(qkv[:, :hq * d].reshape(T, hq, d), (d,), weight=1.0 + W["q_norm"], eps=eps)
    k = F.rms_norm(qkv[:, hq * d:(hq + hk) * d].reshape(T, hk, d), (d,), weight=1.0 + W["k_norm"], eps=eps)
    v = qkv[:, (hq + hk) * d:].reshape(T, hk, d)
    pos = torch.arange(T, dtype=torch.float64).reshape(T, 1, 1)
    q, k = rope_complex(q, pos, base), rope_complex(k, pos, base)
    allow = torch.tril(torch.ones(T, T, dtype=torch.bool)) & torch.from_numpy(valid != 0).unsqueeze(0)
    att = F.scaled_dot_product_attention(q.permute(1, 0, 2).unsqueeze(0), k.permute(1, 0, 2).unsqueeze(0),
                                         v.permute(1, 0, 2).unsqueeze(0), attn_mask=allow, enable_gqa=True)
    ctx = att[0].permute(1, 0, 2).reshape(T, hq * d)
    x1 = X + F.rms_norm(F.linear(ctx, W["w_o"]), (H,), weight=1.0 + W["w_post_attn"], eps=eps)
    xn2 = F.rms_norm(x1, (H,), weight=1.0 + W["w_pre_ffn"], eps=eps)
    I_ = W["w_down"].shape[1]
    hdn = F.gelu(F.linear(xn2, W["w_gu"][:I_]), approximate="tanh") * F.linear(xn2, W["w_gu"][I_:])
    out = x1 + F.rms_norm(F.linear(hdn, W["w_down"]), (H,), weight=1.0 + W["w_post_ffn"], eps=eps)
    return out.numpy(), k.permute(1, 0, 2).numpy(), v.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("seed", [64, 65])
def test_prefix_layer_matches_library_composition(seed):
    w, x, valid, dims = _tiny_prefix(seed)
    out, k, v = orc.prefix_layer(x, w, valid, **dims)
    ref, rk, rv = torch_prefix_layer(w, x, valid, **dims)
    rows = [0] + list(range(1, x.shape[0]))  # every row sees at least itself or key 0
    np.testing.assert_allclose(out[rows], ref[rows], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(k, rk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(v, rv, rtol=1e-12, atol=1e-13)


def test_prefix_layer_zero_projections_is_identity():
    w, x, valid, dims = _tiny_prefix(66)
    w["w_o"][:] = 0.0
    w["w_down"][:] = 0.0
    out, _, _ = orc.prefix_layer(x, w, valid, **dims)
    np.testing.assert_array_equal(out, x)


# ---------------------------------------------------------------- denoise sampler
def test_time_embedding_closed_forms():
    H = 16
    assert np.array_equal(orc.time_embedding(0.0, H), np.r_[np.zeros(8), np.ones(8)])
    for t in (0.1, 0.37, 1.0):
        e = orc.time_embedding(t, H)
        np.testing.assert_allclose(e[:8] ** 2 + e[8:] ** 2, 1.0, rtol=1e-15)
        # frequency 1 at i = 0, 10000^(-1/2) at i = H/4: angles 1000 t and 10 t
        assert e[0] == pytest.approx(math.sin(1000.0 * t), abs=1e-12)
        assert e[4] == pytest.approx(math.sin(10.0 * t), abs=1e-13)
        assert e[12] == pytest.approx(math.cos(10.0 * t), abs=1e-13)
        # frequencies fall geometrically: angle(i) / angle(i + 1) = 10000^(1/8)
        assert e[8 + 7] == pytest.approx(math.cos(1000.0 * t * 10000.0 ** (-7 / 8)), abs=1e-13)


def test_swish_matches_silu_and_identities():
    z = np.linspace(-30.0, 30.0, 61) + 0.123
    ref = F.silu(t64(z)).numpy()
    np.testing.assert_allclose([orc.swish(v) for v in z], ref, rtol=1e-14, atol=1e-300)
    for v in (0.3, 1.7, 5.0, 12.0):
        assert orc.swish(v) - orc.swish(-v) == pytest.approx(v, rel=1e-14)  # z (s(z) + s(-z)) = z
    assert orc.swish(0.0) == 0.0
    assert orc.swish(math.log(3.0)) == pytest.approx(0.75 * math.log(3.0), rel=1e-15)  # sigmoid(ln 3) = 3/4


def test_time_mlp_against_torch_and_permutation():
    r = rng(70)
    H = 12
    w1, w2 = r.standard_normal((H, H)), r.standard_normal((H, H))
    b1, b2 = r.standard_normal(H), r.standard_normal(H)
    temb = r.standard_normal(H)
    ref = F.silu(F.linear(F.silu(F.linear(t64(temb), t64(w1), t64(b1))), t64(w2), t64(b2))).numpy()
    np.testing.assert_allclose(orc.time_mlp(temb, w1, b1, w2, b2), ref, rtol=1e-13, atol=1e-14)
    # permutation weights (a 12-cycle, not an involution): row j picks temb[j + 1];
    # a transposed operand would pick temb[j - 1]
    P = np.zeros((H, H))
    P[np.arange(H), (np.arange(H) + 1) % H] = 1.0
    z = np.zeros(H)
    cond = orc.time_mlp(temb, P, z, np.eye(H), z)
    want = [orc.swish(orc.swish(temb[(j + 1) % H])) for j in range(H)]
    np.testing.assert_allclose(cond, want, rtol=1e-15)
    # zero second layer: the conditioning is swish of its bias, whatever the time
    np.testing.assert_allclose(orc.time_mlp(temb, w1, b1, np.zeros((H, H)), b2), [orc.swish(v) for v in b2],
                               rtol=1e-15)


def test_action_in_one_hot_picks_a_column():
    r = rng(71)
    C, A, H = 3, 5, 7
    w_in, b_in = r.standard_normal((H, A)), r.standard_normal(H)
    a = np.zeros((C, A))
    a[0, 2], a[1, 4] = 1.0, -2.0
    x = orc.action_in(a, w_in, b_in)
    np.testing.assert_allclose(x[0], w_in[:, 2] + b_in, rtol=1e-15)
    np.testing.assert_allclose(x[1], -2.0 * w_in[:, 4] + b_in, rtol=1e-15)
    assert np.array_equal(x[2], b_in)


def test_final_velocity_against_torch_and_closed_forms():
    r = rng(72)
    C, H, A = 4, 8, 3
    x, cond = r.standard_normal((C, H)), r.standard_normal(H)
    w_f, b_f = r.standard_normal((2 * H, H)), r.standard_normal(2 * H)
    w_out, b_out = r.standard_normal((A, H)), r.standard_normal(A)
    m = F.linear(t64(cond), t64(w_f), t64(b_f))
    xf = F.rms_norm(t64(x), (H,), eps=1e-6) * (1.0 + m[:H]) + m[H:]
    ref = F.linear(xf, t64(w_out), t64(b_out)).numpy()
    np.testing.assert_allclose(orc.final_velocity(x, cond, w_f, b_f, w_out, b_out), ref, rtol=1e-12, atol=1e-13)
    # zero output weights: the bias on every token
    v = orc.final_velocity(x, cond, w_f, b_f, np.zeros((A, H)), b_out)
    assert np.array_equal(v, np.tile(b_out, (C, 1)))
    # zero rows normalise to zero, so they carry the shift half only (the second H values)
    zf = np.zeros((2 * H, H))
    v = orc.final_velocity(np.zeros((2, H)), cond, zf, b_f, w_out, b_out)
    np.testing.assert_allclose(v, np.tile(w_out @ b_f[H:] + b_out, (2, 1)), rtol=1e-14)
    # a constant row c with the scale half only: c / sqrt(c^2 + eps) (1 + scale)
    c, bs = -1.5, np.r_[b_f[:H], np.zeros(H)]
    v = orc.final_velocity(np.full((1, H), c), cond, zf, bs, w_out, b_out)
    np.testing.assert_allclose(v[0], w_out @ (c / math.sqrt(c * c + 1e-6) * (1.0 + b_f[:H])) + b_out, rtol=1e-13)
    # with eps = 0 the velocity does not see the row's scale
    v1 = orc.final_velocity(x, cond, w_f, b_f, w_out, b_out, eps=0.0)
    v2 = orc.final_velocity(3.7 * x, cond, w_f, b_f, w_out, b_out, eps=0.0)
    np.testing.assert_allclose(v1, v2, rtol=1e-13, atol=1e-13)


def _tiny_sampler(seed, H=16, A=4):
    r = rng(seed)
    return {"w_in": r.standard_normal((H, A)), "b_in": 0.1 * r.standard_normal(H),
            "w_t1": 0.3 * r.standard_normal((H, H)), "b_t1": 0.1 * r.standard_normal(H),
            "w_t2": 0.3 * r.standard_normal((H, H)), "b_t2": 0.1 * r.standard_normal(H),
            "w_fmod": 0.3 * r.standard_normal((2 * H, H)), "b_fmod": 0.1 * r.standard_normal(2 * H),
            "w_out": r.standard_normal((A, H)), "b_out": r.standard_normal(A)}


def _identity_layers(n, seed):
    out = []
    for i in range(n):
        w, _, _, kp, vp, mask, dims = _tiny_layer(seed + i)
        H = w["w_mod1"].shape[1]
        for k in ("w_mod1", "w_mod2", "b_mod1", "b_mod2"):
            w[k][2 * H:] = 0.0
        out.append((w, kp, vp))
    return out, mask, dims


def test_sampler_constant_velocity_ends_at_noise_minus_bias():
    """Zero output weights make v = b_out at every step; the n Euler steps of
    dt = -1/n then move the noise by exactly -b_out, in equal steps."""
    sw = _tiny_sampler(73)
    sw["w_out"][:] = 0.0
    lay, mask, dims = _identity_layers(2, 74)
    noise = rng(75).standard_normal((3, 4))
    n = 5
    traj = orc.sampler(noise, n, sw, [w for w, _, _ in lay], [k for _, k, _ in lay], [v for _, _, v in lay],
                       mask, 9, **dims)
    for k in range(n):
        np.testing.assert_allclose(traj[k], noise - (k + 1) / n * sw["b_out"], rtol=1e-14, atol=1e-14)


def test_sampler_schedule_runs_from_time_one():
    """With zero input weights and bias the expert sees zero rows, which the
    final norm maps to its shift: v_k = W_out (W_f[H:] cond(t_k) + b_f[H:]) +
    b_out.  Two steps must use t = 1 and t = 1/2, each with dt = -1/2."""
    H = 16
    sw = _tiny_sampler(76, H=H)
    sw["w_in"][:] = 0.0
    sw["b_in"][:] = 0.0
    lay, mask, dims = _identity_layers(1, 77)
    noise = rng(78).standard_normal((2, 4))
    traj = orc.sampler(noise, 2, sw, [lay[0][0]], [lay[0][1]], [lay[0][2]], mask, 0, **dims)
    prev = noise
    for k, t in enumerate((1.0, 0.5)):
        cond = orc.time_condition(t, sw)
        v = sw["w_out"] @ (sw["w_fmod"][H:] @ cond + sw["b_fmod"][H:]) + sw["b_out"]
        np.testing.assert_allclose(traj[k], prev - 0.5 * v, rtol=1e-12, atol=1e-12)
        prev = traj[k]


def test_prefix_layer_rows_equals_full_layer():
    """The row-sampled prefix layer (used at 2048 tokens) is the full layer's
    output at those rows, K/V cache included."""
    r = rng(80)
    T, H, I_, hq, hk, d = 21, 16, 24, 4, 2, 8
    w = {"w_in": 0.3 * r.standard_normal(H), "w_qkv": 0.3 * r.standard_normal(((hq + 2 * hk) * d, H)),
         "q_norm": 0.3 * r.standard_normal(d), "k_norm": 0.3 * r.standard_normal(d),
         "w_o": 0.3 * r.standard_normal((H, hq * d)), "w_post_attn": 0.3 * r.standard_normal(H),
         "w_pre_ffn": 0.3 * r.standard_normal(H), "w_gu": 0.3 * r.standard_normal((2 * I_, H)),
         "w_down": 0.3 * r.standard_normal((H, I_)), "w_post_ffn": 0.3 * r.standard_normal(H)}
    x = r.standard_normal((T, H))
    valid = (r.random(T) < 0.8).astype(np.uint8)
    valid[0] = 1
    full, k, v = orc.prefix_layer(x, w, valid, hq=hq, hk=hk, d=d)
    rows = [0, 3, 7, 20]
    out, k2, v2 = orc.prefix_layer_rows(x, w, valid, rows, hq=hq, hk=hk, d=d)
    np.testing.assert_allclose(out, full[rows], rtol=1e-12, atol=1e-12)
    assert np.array_equal(k2, k) and np.array_equal(v2, v)
