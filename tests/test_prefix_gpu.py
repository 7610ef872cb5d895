"""GPU: the prefix (prefill) decoder layer of the Gemma3-4B prefix path and its
pieces, through the C ABI, against the float64 oracle.

- image-feature merge: bit-exact against the definition;
- prefix attention (prefix-causal mask with invalid tokens) at ragged sizes,
  with poisoned invisible rows, against the oracle;
- the whole layer (norms, QKV + QK-norm + RoPE into the cache, attention,
  O-projection with post-norm and residual, GEGLU MLP with post-norm and
  residual) at two token counts, output and KV cache against the oracle.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
from masked_gqa_attention_action_amd import synth
from tests.helpers import LAYER_BRANCH_REL, delta_gate, dev_bits, f64, from_dev, gate, stage_gate, to_dev, untile

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_gqa_attention_action_amd as dmx


# output gate of the whole prefix layer (see test_prefix_layer_against_oracle)
PREFIX_OUT_REL = 3e-2


def rng(seed):
    return np.random.Generator(np.random.PCG64(synth.BASE_SEED + 9000 + seed))


def rand_bf16(r, shape, std=1.0):
    return synth.bf16_bits((std * r.standard_normal(shape)).astype(np.float32))


def test_image_merge_bit_exact():
    r = rng(1)
    T, NI, Hd = 300, 40, 2560
    tok, img = rand_bf16(r, (T, Hd)), rand_bf16(r, (NI, Hd))
    idx = r.integers(-1, NI + 3, T).astype(np.int32)  # includes rows past the image rows
    out = dmx.image_merge(to_dev(tok), to_dev(img), to_dev(idx, "raw"))
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy().view(np.uint16)
    want = np.where(idx[:, None] < 0, tok, 0).astype(np.uint16)
    ok = (idx >= 0) & (idx < NI)
    want[ok] = img[idx[ok]]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("T,kv_rows,hole_p", [(65, 80, 0.0), (200, 256, 0.1), (1024, 1024, 0.05), (2048, 2048, 0.05),
                                              (4096, 4096, 0.03)])
def test_prefix_attention_against_oracle(T, kv_rows, hole_p):
    """Every output row against the oracle, up to the largest prefix (4096
    tokens: the split size the launch picks there leaves up to 11 splits per
    query block for the merge)."""
    r = rng(2 + T)
    q, k, v = rand_bf16(r, (T, 8, 256)), rand_bf16(r, (4, kv_rows, 256)), rand_bf16(r, (4, kv_rows, 256))
    valid = (np.arange(T) < T - T // 9).astype(np.uint8)
    holes = r.random(T) < hole_p
    holes[0] = False
    valid[holes] = 0
    # invisible and unused cache rows hold NaN: they must never reach a valid output
    nan = synth.bf16_bits(np.full(1, np.nan, np.float32))[0]
    k[:, T:] = nan
    v[:, T:] = nan
    k[:, :T][:, valid == 0] = nan
    v[:, :T][:, valid == 0] = nan
    ctx = dmx.prefix_attention(to_dev(q), to_dev(k), to_dev(v), to_dev(valid, "raw"))
    torch.cuda.synchronize()
    ref = orc.prefix_attention(f64(q), f64(k)[:, :T], f64(v)[:, :T], valid)
    got = from_dev(ctx)
    assert np.isfinite(got).all()
    if T <= 1024:
        stage_gate(f"prefix attention T={T}", got, ref)
        return
    # Under the prefix-causal mask row i averages over its i + 1 visible keys,
    # so the output's scale falls along the rows (the first rows near the
    # RMS of V, the last ~1/sqrt(T) of it): each block of 64 query rows is
    # held to the gate against its own RMS, and the whole to the cosine.  At
    # these lengths a query block's keys span several splits, whose outputs
    # are stored in bf16 before the merge rounds the context to bf16 again:
    # two roundings per element.
    for r0 in range(0, T, 64):
        stage_gate(f"prefix attention T={T} rows {r0}..{r0 + 63}", got[r0:r0 + 64], ref[r0:r0 + 64], roundings=2)
    g, w = got.ravel(), ref.ravel().astype(np.float64)
    assert float(g @ w / (np.linalg.norm(g) * np.linalg.norm(w))) >= 0.9995


@pytest.fixture(scope="module")
def prefix_weights():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wbits = synth.prefix_layer_weights(synth.BASE_SEED + 9500)
    wd = dmx.pack_prefix_weights({k: to_dev(v) for k, v in wbits.items()})
    return wbits, wd


@pytest.mark.parametrize("T,valid_len,hole_p", [(96, 90, 0.0), (300, 280, 0.05)])
def test_prefix_layer_against_oracle(prefix_weights, T, valid_len, hole_p):
    wbits, wd = prefix_weights
    x, valid = synth.prefix_inputs(synth.BASE_SEED + 9600 + T, T, valid_len, hole_p)
    kv_rows = T + 16
    kc = torch.full((4, kv_rows, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full((4, kv_rows, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = dmx.prefix_layer_forward(wd, to_dev(x), to_dev(valid, "raw"), kc, vc)
    torch.cuda.synchronize()
    ref, rk, rv = orc.prefix_layer(f64(x), {k: f64(v) for k, v in wbits.items()}, valid)
    got = from_dev(out)
    # Both branches enter the residual ungated at unit scale (post-norm
    # output), so the layer's five bf16 stores (xn, q/k/v, ctx, xn2, h) reach
    # the output undamped: rounding the float64 reference at those same five
    # points alone gives 1.75-1.85e-2 of the output RMS on these inputs.  The
    # output gate is therefore PREFIX_OUT_REL (1.5x that) plus the stored
    # output's own rounding (2^-8 of the element); the branch gate below holds
    # the branches to the layer bound.
    stage_gate(f"prefix layer T={T}", got, ref, rel=PREFIX_OUT_REL)
    delta_gate(f"prefix layer T={T} branch", got, ref, f64(x), rel=LAYER_BRANCH_REL)
    stage_gate(f"prefix k cache T={T}", from_dev(kc)[:, :T], rk)
    stage_gate(f"prefix v cache T={T}", from_dev(vc)[:, :T], rv)
    assert torch.isnan(kc[:, T:].float()).all(), "rows past the tokens were written"


def prefix_ws_pieces(T):
    """(TP, {name: (byte offset, bytes)}) of the pieces a prefix layer leaves in
    its workspace, in the library's order, each 256-byte aligned: tiled
    rmsnorm(x; w_in); the fp32 QKV projection [TP][4096]; row-major q
    [T][8][256]; the tiled context [TP][2048]; the fp32 projection output
    [TP][2560] (last written by the down projection); fp32 x1 [TP][2560];
    tiled rmsnorm(x1; w_pre_ffn); the tiled GEGLU output [TP][10240]."""
    TP = (T + 15) // 16 * 16
    sizes = [("xn", TP * 2560 * 2), ("raw", TP * 4096 * 4), ("q", T * 8 * 256 * 2), ("ctx", TP * 2048 * 2),
             ("y", TP * 2560 * 4), ("x1", TP * 2560 * 4), ("xn2", TP * 2560 * 2), ("h", TP * 10240 * 2)]
    off, out = 0, {}
    for name, n in sizes:
        out[name] = (off, n)
        off += (n + 255) // 256 * 256
    return TP, out


@pytest.mark.parametrize("T,valid_len,hole_p", [(96, 90, 0.0), (300, 280, 0.05)])
def test_prefix_layer_each_stage_strict(prefix_weights, T, valid_len, hole_p):
    """Every stage of the prefix layer at the strict gate, teacher forced: each
    stage's oracle gets the GPU's own input to that stage (read from the
    layer's workspace), so one stage's error cannot hide behind the whole
    layer's looser output gate.  Stages: input norm; QKV projection; QK-norm +
    RoPE (q, and k / v into the cache); prefix-causal attention; O-projection +
    post-attention norm + residual (x1) and the pre-MLP norm; GEGLU; down
    projection + post-MLP norm + residual (the output)."""
    wbits, wd = prefix_weights
    w = {k: f64(v) for k, v in wbits.items()}
    x, valid = synth.prefix_inputs(synth.BASE_SEED + 9600 + T, T, valid_len, hole_p)
    kv_rows = T + 16
    kc = torch.full((4, kv_rows, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full((4, kv_rows, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = torch.full((int(dmx.lib().dmx_prefix_workspace_bytes(T)),), 0xFF, dtype=torch.uint8, device="cuda")
    out = dmx.prefix_layer_forward(wd, to_dev(x), to_dev(valid, "raw"), kc, vc, ws=ws)
    torch.cuda.synchronize()
    TP, pieces = prefix_ws_pieces(T)
    assert ws.numel() >= pieces["h"][0] + pieces["h"][1]
    wsb = ws.cpu().numpy()

    def piece(name, dt):
        o, n = pieces[name]
        return wsb[o:o + n].view(dt)

    xf = f64(x)
    xn = untile(piece("xn", np.uint16), TP, 2560)[:T]
    stage_gate(f"T={T} input norm", xn, orc.rmsnorm(xf, w["w_in"]))
    raw = piece("raw", np.float32).reshape(TP, 4096)[:T].astype(np.float64)
    gate(f"T={T} QKV projection", raw, orc.linear(xn, w["w_qkv"]))
    rq, rk, rv = orc.qkv_qknorm_rope(xn, w["w_qkv"], w["q_norm"], w["k_norm"], np.arange(T), 8, 4, 256)
    q = f64(piece("q", np.uint16).reshape(T, 8, 256))
    stage_gate(f"T={T} QK-norm + RoPE q", q, rq)
    k_gpu = f64(dev_bits(kc).reshape(4, kv_rows, 256))[:, :T]
    v_gpu = f64(dev_bits(vc).reshape(4, kv_rows, 256))[:, :T]
    stage_gate(f"T={T} QK-norm + RoPE k", k_gpu, rk)
    stage_gate(f"T={T} v", v_gpu, rv)
    ctx = untile(piece("ctx", np.uint16), TP, 2048)[:T]
    stage_gate(f"T={T} attention", ctx, orc.prefix_attention(q, k_gpu, v_gpu, valid).reshape(T, 2048))
    x1 = piece("x1", np.float32).reshape(TP, 2560)[:T].astype(np.float64)
    gate(f"T={T} O-projection + post-norm + residual",
         x1, xf + orc.rmsnorm(orc.linear(ctx, w["w_o"]), w["w_post_attn"]))
    xn2 = untile(piece("xn2", np.uint16), TP, 2560)[:T]
    stage_gate(f"T={T} pre-MLP norm", xn2, orc.rmsnorm(x1, w["w_pre_ffn"]))
    _, rh = orc.geglu_mlp(xn2, w["w_gu"], w["w_down"], np.zeros(2560), np.zeros((T, 2560)))
    h = untile(piece("h", np.uint16), TP, 10240)[:T]
    stage_gate(f"T={T} GEGLU", h, rh)
    ref_out = x1 + orc.rmsnorm(orc.linear(h, w["w_down"]), w["w_post_ffn"])
    stage_gate(f"T={T} down + post-norm + residual", from_dev(out), ref_out)
    delta_gate(f"T={T} down branch", from_dev(out), ref_out, x1, rel=LAYER_BRANCH_REL)


def test_prefix_layer_is_deterministic(prefix_weights):
    _, wd = prefix_weights
    x, valid = synth.prefix_inputs(synth.BASE_SEED + 9700, 257, 250, 0.02)
    outs = []
    for _ in range(2):
        kc = torch.empty((4, 257, 256), dtype=torch.bfloat16, device="cuda")
        vc = torch.empty_like(kc)
        outs.append((dmx.prefix_layer_forward(wd, to_dev(x), to_dev(valid, "raw"), kc, vc), kc, vc))
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a, b)


def test_prefix_layer_2048_tokens_sampled_rows(prefix_weights):
    """The benchmarked size: 2048 tokens (1936 valid, 2 % holes), the launch
    the benchmark times.  Against the oracle on sampled rows (first, last,
    holes, padding, spread, and one in every 128 rows, so that every row
    block of every projection's grid is checked over all its columns) and on
    the whole K/V cache."""
    wbits, wd = prefix_weights
    T = 2048
    x, valid = synth.prefix_inputs(synth.BASE_SEED + 9900, T, 1936, 0.02)
    kc = torch.full((4, T, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    vc = torch.full((4, T, 256), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = dmx.prefix_layer_forward(wd, to_dev(x), to_dev(valid, "raw"), kc, vc)
    torch.cuda.synchronize()
    r = rng(11)
    holes = np.flatnonzero(valid[:1936] == 0)
    rows = sorted(set([0, 1, 63, 64, 1935, 1936, 2047] + [int(i) for i in holes[:3]] +
                      [int(i) for i in r.integers(0, T, 14)] + [128 * i + 77 for i in range(T // 128)]))
    print(f"prefix layer T=2048: {int(valid.sum())} valid, rows {rows}", flush=True)
    ref, rk, rv = orc.prefix_layer_rows(f64(x), {k: f64(v) for k, v in wbits.items()}, valid, rows)
    got = from_dev(out)[rows]
    stage_gate("prefix layer T=2048 rows", got, ref, rel=PREFIX_OUT_REL)
    delta_gate("prefix layer T=2048 rows branch", got, ref, f64(x)[rows], rel=LAYER_BRANCH_REL)
    stage_gate("prefix k cache T=2048", from_dev(kc), rk)
    stage_gate("prefix v cache T=2048", from_dev(vc), rv)
