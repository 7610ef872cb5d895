"""GPU parity: every stage and the whole layer through the C ABI against the
float64 oracle on the same seeded bf16 inputs, at the workloads' sizes.

Gate (floating point): max |err| <= 2e-2 * RMS(oracle) and cosine >= 0.9995.
Integer / selection work (which prefix rows are visible) is checked bit-exactly
through poisoning: masked rows filled with NaN / Inf / huge values must leave
the GPU output bit-identical to its clean run.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
from masked_gqa_attention_action_amd import synth
from tests.helpers import (LAYER_BRANCH_REL, delta_gate, device_weights, f64, from_dev, gate, oracle_weights, stage_gate,
                           to_dev, to_dev_w)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

dmx = None


@pytest.fixture(scope="module", autouse=True)
def _lib():
    global dmx
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_gqa_attention_action_amd as m
    m.lib()
    dmx = m
    yield


def rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def rand_bf16(r, shape, std=1.0):
    return synth.bf16_bits(r.standard_normal(shape, dtype=np.float32) * np.float32(std))


# ---------------------------------------------------------------- weight tiling
@pytest.mark.parametrize("rows,cols", [(16, 32), (48, 96), (4096, 1024), (1024, 4096)])
def test_pack_weight_layout(rows, cols):
    """Bit-exact: tile (rt, ct) at (rt * cols/32 + ct) * 512, inside it the
    8 columns 8q..8q+7 of tile row i at (i + 16 q) * 8."""
    r = rng(rows + cols)
    w = rand_bf16(r, (rows, cols))
    got = dmx.pack_weight(to_dev(w))
    torch.cuda.synchronize()
    got_bits = got.view(torch.int16).cpu().numpy().view(np.uint16).ravel()
    want = w.reshape(rows // 16, 16, cols // 32, 4, 8).transpose(0, 2, 3, 1, 4).ravel()
    assert np.array_equal(got_bits, want)


# ---------------------------------------------------------------- AdaRMS
@pytest.mark.parametrize("B,T", [(1, 10), (1, 50), (16, 50), (3, 1)])
def test_adarms_prenorm(B, T):
    r = rng(100 + B * 7 + T)
    x, cond = rand_bf16(r, (B, T, synth.H)), rand_bf16(r, (B, synth.H))
    w, bias = rand_bf16(r, (3 * synth.H, synth.H), 0.02), rand_bf16(r, (3 * synth.H,), 0.02)
    xn, mod = dmx.adarms_prenorm(to_dev(x), to_dev(cond), to_dev_w(w), to_dev(bias))
    torch.cuda.synchronize()
    for b in range(B):
        xr, mr = orc.adarms(f64(x[b]), f64(cond[b]), f64(w), f64(bias))
        stage_gate(f"mod[b={b}]", from_dev(mod[b]), mr)
        stage_gate(f"x_norm[b={b}]", from_dev(xn[b]), xr)


# ---------------------------------------------------------------- QKV + QK-norm + RoPE
@pytest.mark.parametrize("B,T,pos0", [(1, 50, 1024), (1, 10, 576), (2, 50, 2048), (16, 50, 700)])
def test_qkv_qknorm_rope_suffix(B, T, pos0):
    r = rng(200 + B + T)
    xn = rand_bf16(r, (B, T, synth.H))
    w = rand_bf16(r, (4096, synth.H), 0.02)
    qn, kn = rand_bf16(r, (256,), 0.02), rand_bf16(r, (256,), 0.02)
    pos = np.array([pos0 + 13 * b for b in range(B)], dtype=np.int32)
    ws = dmx.new_workspace(B, T, 0)
    q, k, v = dmx.qkv_qknorm_rope(to_dev(xn), to_dev_w(w), to_dev(qn), to_dev(kn), to_dev(pos, "raw"), ws)
    torch.cuda.synchronize()
    for b in range(B):
        qr, kr, vr = orc.qkv_qknorm_rope(f64(xn[b]), f64(w), f64(qn), f64(kn), pos[b] + np.arange(T), 8, 4, 256)
        stage_gate(f"q[b={b}]", from_dev(q[b]), qr)
        stage_gate(f"k[b={b}]", from_dev(k[b]), kr)
        stage_gate(f"v[b={b}]", from_dev(v[b]), vr)


def test_qkv_prefix_hidden2560_into_cache():
    """Prefix-side variant: hidden 2560, 2048 tokens at positions 0..2047,
    K/V written straight into the [4][P_b][256] cache layout.  The oracle runs
    on a sample of tokens (each token's output depends only on its own row)."""
    inp = synth.prefix_qkv_inputs(synth.BASE_SEED + 4000 + 77)
    T, P = 2048, 2048
    ws = dmx.new_workspace(1, T, 0)
    kc = torch.full((1, 4, P, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full((1, 4, P, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    pos = to_dev(np.zeros(1, dtype=np.int32), "raw")
    q, k, v = dmx.qkv_qknorm_rope(to_dev(inp["x"]).view(1, T, 2560), to_dev_w(inp["w_qkv"]), to_dev(inp["q_norm"]),
                                  to_dev(inp["k_norm"]), pos, ws, k=kc, v=vc, kv_rows=P)
    torch.cuda.synchronize()
    assert torch.isfinite(k).all() and torch.isfinite(v).all()
    sample = np.array(sorted(set([0, 1, 2, 127, 128, 1000, 2046, 2047] +
                                 list(rng(5).integers(0, T, 24)))))
    qr, kr, vr = orc.qkv_qknorm_rope(f64(inp["x"][sample]), f64(inp["w_qkv"]), f64(inp["q_norm"]),
                                     f64(inp["k_norm"]), sample, 8, 4, 256)
    stage_gate("prefix q", from_dev(q[0, sample]), qr)
    stage_gate("prefix k", from_dev(k[0][:, sample]), kr)
    stage_gate("prefix v", from_dev(v[0][:, sample]), vr)


def test_qkv_prefix_large_m_schedule_is_bit_identical():
    """The 2048-token prefix QKV runs on the large-M GEMM schedule; 32 calls of
    64 tokens (positions and cache rows offset) run on the skinny one.  Both
    schedules add the same products in the same order, so every output bit
    agrees."""
    inp = synth.prefix_qkv_inputs(synth.BASE_SEED + 4000 + 78)
    T, P, S = 2048, 2048, 64
    x = to_dev(inp["x"]).view(1, T, 2560)
    w, qn, kn = to_dev_w(inp["w_qkv"]), to_dev(inp["q_norm"]), to_dev(inp["k_norm"])
    ws = dmx.new_workspace(1, T, 0)
    pos = to_dev(np.zeros(1, dtype=np.int32), "raw")
    q, k, v = dmx.qkv_qknorm_rope(x, w, qn, kn, pos, ws, kv_rows=P)
    k2 = torch.empty_like(k)
    v2 = torch.empty_like(v)
    ws2 = dmx.new_workspace(1, S, 0)
    qs = []
    for c in range(T // S):
        pc = to_dev(np.array([c * S], dtype=np.int32), "raw")
        qc, _, _ = dmx.qkv_qknorm_rope(x[:, c * S:(c + 1) * S].contiguous(), w, qn, kn, pc, ws2, k=k2, v=v2,
                                       kv_rows=P, kv_row0=c * S)
        qs.append(qc)
    torch.cuda.synchronize()
    assert torch.equal(q, torch.cat(qs, dim=1))
    assert torch.equal(k, k2) and torch.equal(v, v2)


def test_qkv_writes_only_its_cache_rows():
    r = rng(210)
    T, P, row0 = 50, 1024, 1024 - 50 - 7
    xn = rand_bf16(r, (1, T, synth.H))
    w = rand_bf16(r, (4096, synth.H), 0.02)
    qn, kn = rand_bf16(r, (256,), 0.02), rand_bf16(r, (256,), 0.02)
    ws = dmx.new_workspace(1, T, 0)
    kc = torch.full((1, 4, P, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full((1, 4, P, 256), 7.0, dtype=torch.bfloat16, device="cuda")
    dmx.qkv_qknorm_rope(to_dev(xn), to_dev_w(w), to_dev(qn), to_dev(kn), to_dev(np.array([5], np.int32), "raw"), ws,
                        k=kc, v=vc, kv_rows=P, kv_row0=row0)
    torch.cuda.synchronize()
    untouched = torch.ones(P, dtype=torch.bool)
    untouched[row0:row0 + T] = False
    assert (kc[0][:, untouched] == 7.0).all() and (vc[0][:, untouched] == 7.0).all()
    assert not (kc[0][:, row0:row0 + T] == 7.0).all()


# ---------------------------------------------------------------- attention
def attn_inputs(seed, B, C, P, masks):
    r = rng(seed)
    q = rand_bf16(r, (B, C, 8, 256))
    ks, vs = rand_bf16(r, (B, 4, C, 256)), rand_bf16(r, (B, 4, C, 256))
    kp, vp = rand_bf16(r, (B, 4, P, 256)), rand_bf16(r, (B, 4, P, 256))
    mask = np.stack(masks).astype(np.uint8) if P > 0 else np.zeros((B, 0), np.uint8)
    return q, ks, vs, kp, vp, mask


def run_attention(q, ks, vs, kp, vp, mask):
    B, C = q.shape[:2]
    P = kp.shape[2]
    ws = dmx.new_workspace(B, C, P)
    mask_d = to_dev(mask, "raw") if P > 0 else torch.zeros((B, 0), dtype=torch.uint8, device="cuda")
    kp_d = to_dev(kp) if P > 0 else torch.zeros((B, 4, 0, 256), dtype=torch.bfloat16, device="cuda")
    vp_d = to_dev(vp) if P > 0 else torch.zeros((B, 4, 0, 256), dtype=torch.bfloat16, device="cuda")
    ctx = dmx.suffix_attention(to_dev(q), to_dev(ks), to_dev(vs), kp_d, vp_d, mask_d, ws)
    torch.cuda.synchronize()
    return ctx


def check_attention(name, ctx, q, ks, vs, kp, vp, mask):
    for b in range(q.shape[0]):
        P = kp.shape[2]
        ref = orc.attention(f64(q[b]), f64(ks[b]), f64(vs[b]), f64(kp[b]) if P else np.zeros((4, 0, 256)),
                            f64(vp[b]) if P else np.zeros((4, 0, 256)), mask[b])
        stage_gate(f"{name}[b={b}]", from_dev(ctx[b]), ref)


def wl_masks(wl, B):
    out = []
    for b in range(B):
        m, _ = synth.make_mask(rng(wl.request_seed(b)), wl.p_bucket, wl.len_lo, wl.len_hi, wl.hole_p)
        out.append(m)
    return out


@pytest.mark.parametrize("wname", ["c1", "c2", "c4", "c5"])
def test_attention_workload_shapes(wname):
    wl = synth.WORKLOADS[wname]
    B = wl.batch
    inp = attn_inputs(wl.seed + 11, B, wl.chunk, wl.p_bucket, wl_masks(wl, B))
    ctx = run_attention(*inp)
    check_attention(wname, ctx, *inp)


@pytest.mark.parametrize("B,C,P,kind", [
    (1, 50, 1024, "all_masked"), (1, 50, 0, "no_prefix"), (1, 1, 576, "ragged"), (1, 64, 704, "ragged"),
    (2, 7, 100, "ragged"), (1, 50, 1024, "one_visible"), (1, 10, 33, "ragged"), (1, 50, 2048, "first_and_last"),
])
def test_attention_edge_cases(B, C, P, kind):
    r = rng(300 + C + P)
    masks = []
    for b in range(B):
        m = np.zeros(P, np.uint8)
        if kind == "ragged":
            m[: max(1, P - 5 - 3 * b)] = 1
            m[r.integers(0, P, P // 7)] = 0
        elif kind == "one_visible":
            m[P // 3] = 1
        elif kind == "first_and_last":
            m[0] = 1
            m[P - 1] = 1
        masks.append(m)
    inp = attn_inputs(400 + C + P, B, C, P, masks)
    ctx = run_attention(*inp)
    check_attention(kind, ctx, *inp)


def test_attention_batched_edge_cases_equal_single_requests():
    """Eight requests (the launch pairs the two query heads of a KV group in
    one work-group at this grid size) mixing the degenerate masks: all
    masked, one visible key, first and last only, ragged, full.  Each
    request gets the bits it gets alone (one head per work-group) and passes
    the oracle gate."""
    B, C, P = 8, 50, 1024
    r = rng(777)
    masks = []
    for b in range(B):
        m = np.zeros(P, np.uint8)
        kind = b % 5
        if kind == 1:
            m[P // 3 + b] = 1
        elif kind == 2:
            m[0] = 1
            m[P - 1] = 1
        elif kind == 3:
            m[: P - 5 - 3 * b] = 1
            m[r.integers(0, P, P // 7)] = 0
        elif kind == 4:
            m[:] = 1
        masks.append(m)
    inp = attn_inputs(778, B, C, P, masks)
    ctx = run_attention(*inp)
    check_attention("batched edge cases", ctx, *inp)
    for b in range(B):
        single = run_attention(*(x[b:b + 1] for x in inp))
        assert torch.equal(ctx[b], single[0]), f"request {b} differs from its single-request run"


@pytest.mark.parametrize("poison", [float("nan"), float("inf"), -float("inf"), 3e4, -3e4])
def test_attention_masked_rows_never_read(poison):
    wl = synth.WORKLOADS["c4"]  # holes inside the valid range plus a masked tail
    q, ks, vs, kp, vp, mask = attn_inputs(wl.seed + 12, 1, wl.chunk, wl.p_bucket, wl_masks(wl, 1))
    assert (mask == 0).any()
    clean = run_attention(q, ks, vs, kp, vp, mask)
    pk = synth.bf16_bits(np.full(1, poison, np.float32))[0]
    kp2, vp2 = kp.copy(), vp.copy()
    kp2[0][:, mask[0] == 0, :] = pk
    vp2[0][:, mask[0] == 0, :] = pk
    dirty = run_attention(q, ks, vs, kp2, vp2, mask)
    assert torch.equal(clean, dirty)


def test_attention_is_deterministic():
    wl = synth.WORKLOADS["c2"]
    inp = attn_inputs(wl.seed + 13, 1, wl.chunk, wl.p_bucket, wl_masks(wl, 1))
    a = run_attention(*inp)
    b = run_attention(*inp)
    assert torch.equal(a, b)


# ---------------------------------------------------------------- projections
@pytest.mark.parametrize("B,T", [(1, 50), (1, 10), (16, 50)])
def test_oproj_gated_residual(B, T):
    r = rng(500 + B + T)
    ctx = rand_bf16(r, (B, T, 8, 256))
    w_o = rand_bf16(r, (1024, 2048), 0.02)
    mod = r.standard_normal((B, 3072)).astype(np.float32)
    resid = rand_bf16(r, (B, T, 1024))
    ws = dmx.new_workspace(B, T, 0)
    out = dmx.oproj_gated_residual(to_dev(ctx), to_dev_w(w_o), to_dev(mod, "raw"), to_dev(resid), ws)
    out2 = dmx.oproj_gated_residual(to_dev(ctx), to_dev_w(w_o), to_dev(mod, "raw"), to_dev(resid), ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    for b in range(B):
        ref = orc.oproj_gated_residual(f64(ctx[b]).reshape(T, 2048), f64(w_o), mod[b, 2048:].astype(np.float64),
                                       f64(resid[b]))
        stage_gate(f"oproj[b={b}]", from_dev(out[b]), ref)
        # the projection alone, without the residual that dominates the sum
        delta_gate(f"oproj-branch[b={b}]", from_dev(out[b]), ref, f64(resid[b]))


@pytest.mark.parametrize("B,T", [(1, 50), (1, 10), (16, 50)])
def test_geglu_mlp(B, T):
    r = rng(600 + B + T)
    xn2 = rand_bf16(r, (B, T, 1024))
    w_gu = rand_bf16(r, (8192, 1024), 0.02)
    w_d = rand_bf16(r, (1024, 4096), 0.02)
    mod2 = r.standard_normal((B, 3072)).astype(np.float32)
    resid = rand_bf16(r, (B, T, 1024))
    ws = dmx.new_workspace(B, T, 0)
    out = dmx.geglu_mlp(to_dev(xn2), to_dev_w(w_gu), to_dev_w(w_d), to_dev(mod2, "raw"), to_dev(resid), ws)
    torch.cuda.synchronize()
    for b in range(B):
        ref, _ = orc.geglu_mlp(f64(xn2[b]), f64(w_gu), f64(w_d), mod2[b, 2048:].astype(np.float64), f64(resid[b]))
        stage_gate(f"geglu[b={b}]", from_dev(out[b]), ref)
        delta_gate(f"geglu-branch[b={b}]", from_dev(out[b]), ref, f64(resid[b]))


# ---------------------------------------------------------------- whole layer
def layer_case(wname):
    wl = synth.WORKLOADS[wname]
    wbits = synth.layer_weights(wl.weight_seed(0))
    reqs = [synth.make_request(wl.request_seed(b), wl.chunk, wl.p_bucket, wl.len_lo, wl.len_hi, 1, wl.hole_p)
            for b in range(wl.batch)]
    return wl, wbits, reqs


def run_layer(wbits, reqs, wd=None):
    B = len(reqs)
    C, P = reqs[0].x.shape[0], reqs[0].mask.shape[0]
    wd = device_weights(wbits) if wd is None else wd
    x = to_dev(np.stack([r.x for r in reqs]))
    cond = to_dev(np.stack([r.cond for r in reqs]))
    kp = to_dev(np.stack([r.k_pre[0] for r in reqs]))
    vp = to_dev(np.stack([r.v_pre[0] for r in reqs]))
    mask = to_dev(np.stack([r.mask for r in reqs]), "raw")
    pos0 = to_dev(np.array([r.pos0 for r in reqs], np.int32), "raw")
    ws = dmx.new_workspace(B, C, P)
    out = dmx.suffix_layer_forward(wd, kp, vp, mask, x, cond, pos0, ws)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("wname", ["c1", "c2", "c4", "c5"])
def test_layer_forward(wname):
    wl, wbits, reqs = layer_case(wname)
    out = run_layer(wbits, reqs)
    ow = oracle_weights(wbits)
    for b in range(len(reqs)):
        rq = reqs[b]
        ref = orc.layer(f64(rq.x), f64(rq.cond), ow, f64(rq.k_pre[0]), f64(rq.v_pre[0]), rq.mask, rq.pos0)
        gate(f"{wname} layer[b={b}]", from_dev(out[b]), ref)
        delta_gate(f"{wname} layer-branch[b={b}]", from_dev(out[b]), ref, f64(rq.x), rel=LAYER_BRANCH_REL)


def test_layer_batched_equals_single_requests():
    """A request's output does not depend on the other requests in the batch
    (four requests run the attention with both heads of a KV group per
    work-group, one request with one head per work-group)."""
    wl, wbits, reqs = layer_case("c5")
    wd = device_weights(wbits)
    batched = run_layer(wbits, reqs[:4], wd)
    for b in range(4):
        single = run_layer(wbits, [reqs[b]], wd)
        assert torch.equal(batched[b], single[0])


@pytest.mark.parametrize("B,C,P", [(20, 10, 576), (9, 40, 704), (5, 64, 768)])
def test_layer_large_m_batches_equal_single_requests(B, C, P):
    """Batches of 256+ padded rows run on the large-M GEMM schedules, whose
    blocks hold several requests (padded to 16, 48 or 64 rows, so requests
    straddle 128-row blocks) with one AdaRMS shift row each, and grids whose
    blocks do not split evenly over the XCDs.  Every request still gets the
    bits it gets alone on the skinny schedule, and the batch passes the
    oracle gate on a sample of requests."""
    wbits = synth.layer_weights(synth.BASE_SEED + 7000 + C)
    reqs = [synth.make_request(synth.BASE_SEED + 7100 + 31 * C + b, C, P, P // 2, P, 1) for b in range(B)]
    wd = device_weights(wbits)
    batched = run_layer(wbits, reqs, wd)
    for b in range(B):
        single = run_layer(wbits, [reqs[b]], wd)
        assert torch.equal(batched[b], single[0]), f"request {b} of {B} (C={C})"
    ow = oracle_weights(wbits)
    rq = reqs[B - 1]
    ref = orc.layer(f64(rq.x), f64(rq.cond), ow, f64(rq.k_pre[0]), f64(rq.v_pre[0]), rq.mask, rq.pos0)
    gate(f"large-M batch B={B} C={C} request {B - 1}", from_dev(batched[B - 1]), ref)


def test_layer_largest_shapes():
    """16 requests at the 2048 bucket (the largest batch and prefix of the
    workloads at once: large-M projections, the paired-head attention over
    34 splits), the c4 mask rule with holes; requests 0, 7 and 15 against the
    oracle, and request 15 bit-equal to its single-request run."""
    wbits = synth.layer_weights(synth.BASE_SEED + 7700)
    reqs = [synth.make_request(synth.BASE_SEED + 7800 + b, 50, 2048, 1900, 2048, 1, 0.05) for b in range(16)]
    wd = device_weights(wbits)
    out = run_layer(wbits, reqs, wd)
    ow = oracle_weights(wbits)
    for b in (0, 7, 15):
        rq = reqs[b]
        ref = orc.layer(f64(rq.x), f64(rq.cond), ow, f64(rq.k_pre[0]), f64(rq.v_pre[0]), rq.mask, rq.pos0)
        gate(f"B=16 P_b=2048 layer[b={b}]", from_dev(out[b]), ref)
    single = run_layer(wbits, [reqs[15]], wd)
    assert torch.equal(out[15], single[0])


def test_layer_maximum_shapes():
    """The library's limits at once: 64 requests of 64 tokens at the 4096
    bucket (4096 rows through the large-M projections, 66 splits per request
    and KV head in the attention), valid lengths 3800..4096 with holes (16
    seeded requests, each in four batch slots, to keep the host draws short);
    requests 0, 40 and 63 against the oracle, and request 63 bit-equal to
    its single-request run."""
    B, C, P = 64, 64, 4096
    wbits = synth.layer_weights(synth.BASE_SEED + 7900)
    base = [synth.make_request(synth.BASE_SEED + 8000 + b, C, P, 3800, P, 1, 0.05) for b in range(16)]
    reqs = [base[b % 16] for b in range(B)]
    wd = device_weights(wbits)
    out = run_layer(wbits, reqs, wd)
    ow = oracle_weights(wbits)
    for b in (0, 40, 63):
        rq = reqs[b]
        ref = orc.layer(f64(rq.x), f64(rq.cond), ow, f64(rq.k_pre[0]), f64(rq.v_pre[0]), rq.mask, rq.pos0)
        gate(f"B={B} C={C} P_b={P} layer[b={b}]", from_dev(out[b]), ref)
    single = run_layer(wbits, [reqs[63]], wd)
    assert torch.equal(out[63], single[0])


def test_layer_masked_rows_never_read():
    wl, wbits, reqs = layer_case("c4")
    wd = device_weights(wbits)
    clean = run_layer(wbits, reqs, wd)
    rq = reqs[0]
    nanb = synth.bf16_bits(np.full(1, np.nan, np.float32))[0]
    rq.k_pre[0][:, rq.mask == 0, :] = nanb
    rq.v_pre[0][:, rq.mask == 0, :] = nanb
    dirty = run_layer(wbits, reqs, wd)
    assert torch.equal(clean, dirty)
