"""Benchmark: ms per denoise step of the 18-layer action-expert stack at the
P_b=1024 prefix bucket, chunk 50, batch 1, and the HBM roofline fraction of
its dominant kernel.

One step = the whole hot path once: 18 action-expert layers (AdaRMS, QKV +
QK-norm + RoPE, masked GQA attention over prefix + suffix KV, gated residuals,
GEGLU MLP) for one denoising step, replayed from a hipGraph captured for the
1024 bucket.  Inputs (seeded synthetic weights, KV cache, mask, time
embedding) are resident in HBM before timing starts.

Per-kernel timing: every kernel of the step is also launched on its own,
through dmx_stack_stage_launch, in a captured graph that runs it once for
each of the 64 layers of a timing stack (the step's 18 layers and copies of
them at other addresses), timed with events on the same stream.  The 64
layers' weights and KV exceed the 256 MB memory-side cache, so every launch
streams its operands from HBM as in the step.  The kernel with the largest
share of the step is the "dominant" one whose roofline fraction is reported.
The single-layer and prefix timings rotate over copies of their operands for
the same reason.

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
H, I, HQ, HK, D = 1024, 4096, 8, 4, 256
W_QKV, W_O, W_GU, W_DOWN = 4096 * H * 2, H * 2048 * 2, 8192 * H * 2, H * I * 2
W_MOD = 3072 * H * 2 + 3072 * 2  # one modulation matrix + bias
LAYER_WEIGHT_BYTES = W_QKV + W_O + W_GU + W_DOWN + 2 * W_MOD + 2 * D * 2  # 50,344,960


def algorithmic_bytes_per_layer(batch, chunk, p_bucket, visible_rows_total):
    """Bytes one layer must move: its weights, the visible prefix K/V rows, and
    its own inputs and outputs (x in and out, cond, mask, pos0)."""
    kv = 2 * HK * D * 2 * visible_rows_total
    io = batch * (2 * chunk * H * 2 + H * 2 + p_bucket + 4)
    return LAYER_WEIGHT_BYTES + kv + io


def stage_bytes(stage, batch, chunk, p_bucket, visible, n_layers):
    """Algorithmic bytes of one launch of a stack kernel: the weights, KV rows
    and layer inputs / outputs that its operation must read or write (bf16
    activations).  Intermediates another fused design keeps on chip are not
    counted; the attention combine therefore has none of its own.  The step's
    modulation launch computes layer 0's two vectors; every other layer's come
    with the attention launch of the layer before it (averaged over the
    layers here)."""
    import masked_gqa_attention_action_amd as dmx
    M = batch * chunk
    act = lambda n: M * n * 2
    mods = 2 * W_MOD + batch * H * 2 + 2 * batch * 3072 * 4  # one layer's two vectors
    return {
        dmx.STAGE_MODS: mods,
        dmx.STAGE_PACK: act(H) * 2,
        dmx.STAGE_QKV: W_QKV + act(H) + act(4096) + 2 * D * 2,
        dmx.STAGE_ATTN: 2 * HK * D * 2 * visible + act(4096) + act(2048) + batch * p_bucket
        + mods * (n_layers - 1) // n_layers,
        dmx.STAGE_COMBINE: 0,
        dmx.STAGE_OPROJ: W_O + act(2048) + 2 * act(H),
        dmx.STAGE_GATEUP: W_GU + act(H) + act(I),
        dmx.STAGE_DOWN: W_DOWN + act(I) + 2 * act(H),
    }[stage]


def layer_flops(batch, chunk, visible_rows_total):
    proj = 2 * batch * chunk * (H * 4096 + 2048 * H + H * 8192 + I * H)
    mod = 2 * batch * 2 * H * 3072
    attn = 4 * HQ * D * chunk * (visible_rows_total + batch * chunk)
    return proj + mod + attn


def dev(bits, raw=False):
    import torch
    a = np.ascontiguousarray(bits)
    t = torch.from_numpy(a) if raw else torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def source_digest(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "masked_gqa_attention_action_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# every kernel source and header of the library (device code included from any
# header changes a kernel, so all of them decide whether a counter summary
# still applies)
KERNEL_SOURCES = tuple(sorted(n for n in os.listdir(os.path.join(ROOT, "masked_gqa_attention_action_amd", "csrc"))
                              if n.endswith((".hip", ".hpp"))))


def recorded_traffic(kernel_tag):
    """HBM bytes per launch of a kernel from the committed counter summary
    (profiles/traffic_<tag>.txt: 'bytes_per_launch' and the digest of the
    kernel sources it was taken with); None if absent or taken with other
    sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_digest") != source_digest(*KERNEL_SOURCES):
        return None
    try:
        return int(float(vals["bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


TIMING_LAYERS = 64  # layers of the per-kernel timing stack (DMX_MAX_LAYERS)


def timing_stack(dmx, wd, kp, vp, mask, cond, pos0, x0, mod_table=False):
    """A TIMING_LAYERS-layer stack over the step's layers and copies of them
    (weights and KV at other addresses), run once so its workspace holds the
    intermediates of a real pass."""
    import torch
    n = len(wd)
    wdt = [wd[l] if l < n else {k: v.clone() for k, v in wd[l % n].items()} for l in range(TIMING_LAYERS)]
    kpt = [kp[l] if l < n else kp[l % n].clone() for l in range(TIMING_LAYERS)]
    vpt = [vp[l] if l < n else vp[l % n].clone() for l in range(TIMING_LAYERS)]
    xt = x0.clone()
    st = dmx.Stack(wdt, kpt, vpt, mask, cond, pos0, xt, mod_table=mod_table)
    st.run()
    torch.cuda.synchronize()
    return st


def time_stage(st, stage, n_layers, stream, reps):
    """Average launch duration (us) of one stack kernel: a captured graph runs
    it once per layer of the timing stack in stack order (each launch streams
    another layer's weights and KV from HBM, as in the step); replays are
    timed with events on the same stream."""
    import torch
    import masked_gqa_attention_action_amd as dmx
    g = torch.cuda.CUDAGraph()
    per_graph = n_layers  # per-step kernels (modulation, input pack) repeat n_layers times too
    with torch.cuda.stream(stream):
        for l in range(per_graph):  # eager warm-up of the same launches
            st.stage_launch(l, stage, 1, stream)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for l in range(per_graph):
                st.stage_launch(l, stage, 1, stream)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):  # replay() launches on the current stream
        for _ in range(3):
            g.replay()
        stream.synchronize()
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    e1.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * per_graph)


def time_replays(st, stream, warmup, reps):
    """ms per replay of a captured stack graph, events on its stream."""
    import torch
    for _ in range(warmup):
        st.replay(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        st.replay(stream)
    e1.record(stream)
    e1.synchronize()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


PEAK_BF16_TFLOPS = 2500.0
ROTATE, ROTATE_BYTES = 8, 512 << 20  # operand copies the single-call timings rotate over (at least)


def time_calls(fn, stream, reps=20, rounds=5):
    """us per call of fn(stream, i), from graph replays of reps back-to-back
    calls (i = 0 .. reps - 1: the call's copy of its operands is i modulo the
    number of copies) timed with events on the capture stream."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        fn(stream, 0)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(reps):
                fn(stream, i)
        g.replay()
        stream.synchronize()
        best = []
        for _ in range(rounds):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            g.replay()
            e1.record(stream)
            e1.synchronize()
            best.append(e0.elapsed_time(e1) * 1e3 / reps)
    del g
    return float(np.median(best))


def layer_case(name):
    """One action-expert layer of a parity workload (eager path: modulation,
    input pack and the six kernels), its us per layer and roofline fractions."""
    import torch
    import masked_gqa_attention_action_amd as dmx
    from masked_gqa_attention_action_amd import synth
    wl = synth.WORKLOADS[name]
    B, C, P = wl.batch, wl.chunk, wl.p_bucket
    w = dmx.pack_layer_weights({k: dev(v) for k, v in synth.layer_weights(wl.weight_seed(0)).items()})
    rqs = [synth.make_request(wl.request_seed(b), C, P, wl.len_lo, wl.len_hi, 1, wl.hole_p) for b in range(B)]
    x = dev(np.stack([r.x for r in rqs]))
    cond = dev(np.stack([r.cond for r in rqs]))
    kp = dev(np.stack([r.k_pre[0] for r in rqs]))
    vp = dev(np.stack([r.v_pre[0] for r in rqs]))
    mask = dev(np.stack([r.mask for r in rqs]), raw=True)
    pos0 = dev(np.array([r.pos0 for r in rqs], np.int32), raw=True)
    ws = dmx.new_workspace(B, C, P)
    out = torch.empty_like(x)
    # ROTATE copies of the weights and KV (>= 8, and >= 512 MB in all), so
    # that no call finds its operands in the memory-side cache
    per_copy = LAYER_WEIGHT_BYTES + kp.numel() * 4
    n_copies = max(ROTATE, -(-ROTATE_BYTES // per_copy))
    ops = [(w, kp, vp)] + [({k: v.clone() for k, v in w.items()}, kp.clone(), vp.clone()) for _ in range(n_copies - 1)]
    us = time_calls(lambda s, i: dmx.suffix_layer_forward(ops[i % n_copies][0], ops[i % n_copies][1],
                                                          ops[i % n_copies][2], mask, x, cond, pos0, ws, out=out,
                                                          stream=s),
                    torch.cuda.Stream(), reps=2 * n_copies)
    assert torch.isfinite(out.float()).all(), "non-finite layer output"
    visible = int(sum(int(r.mask.sum()) for r in rqs))
    nbytes = algorithmic_bytes_per_layer(B, C, P, visible)
    flops = layer_flops(B, C, visible)
    del ops
    return {"workload": wl.note, "us_per_layer": round(us, 2), "operand_copies": n_copies, "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4), "flops": flops,
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4)}


def prefix_qkv_case():
    """Prefix-side QKV + QK-norm + RoPE at hidden 2560 over 2048 tokens, K/V
    into a 2048-row cache: us per call against the bf16 MFMA peak."""
    import torch
    import masked_gqa_attention_action_amd as dmx
    from masked_gqa_attention_action_amd import synth
    T, hid = 2048, 2560
    inp = synth.prefix_qkv_inputs(synth.BASE_SEED + 4000 + 77)
    x = dev(inp["x"]).view(1, T, hid)
    w = dmx.pack_weight(dev(inp["w_qkv"]))
    qn, kn = dev(inp["q_norm"]), dev(inp["k_norm"])
    pos = dev(np.zeros(1, np.int32), raw=True)
    ws = dmx.new_workspace(1, T, 0)
    kc = torch.empty((1, HK, T, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    per_copy = (x.numel() + w.numel() + 2 * kc.numel()) * 2
    n = max(ROTATE, -(-ROTATE_BYTES // per_copy))
    ops = [(x, w, kc, vc)] + [(x.clone(), w.clone(), torch.empty_like(kc), torch.empty_like(vc)) for _ in range(n - 1)]
    us = time_calls(lambda s, i: dmx.qkv_qknorm_rope(ops[i % n][0], ops[i % n][1], qn, kn, pos, ws, k=ops[i % n][2],
                                                     v=ops[i % n][3], kv_rows=T, stream=s),
                    torch.cuda.Stream(), reps=2 * n)
    del ops
    flops = 2 * T * hid * (HQ + 2 * HK) * D
    nbytes = T * hid * 2 + (HQ + 2 * HK) * D * hid * 2 + T * (HQ + 2 * HK) * D * 2 + 2 * D * 2
    return {"workload": "prefix QKV + QK-norm + RoPE, hidden 2560, 2048 tokens, K/V into the cache",
            "us": round(us, 2), "operand_copies": n, "flops": flops, "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4), "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}


def prefix_layer_case(T=2048, valid_len=1936, hole_p=0.02):
    """One prefix (prefill) decoder layer, hidden 2560 / intermediate 10240,
    at the 2048-token bucket with padding and invisible tokens; and its
    prefix-causal attention alone.  us per call against the bf16 MFMA peak
    (the GEMMs dominate) and the HBM peak (weights, activations, K/V)."""
    import torch
    import masked_gqa_attention_action_amd as dmx
    from masked_gqa_attention_action_amd import synth
    PH, PI = 2560, 10240
    wd = dmx.pack_prefix_weights({k: dev(v) for k, v in synth.prefix_layer_weights(synth.BASE_SEED + 9500).items()})
    xb, valid_np = synth.prefix_inputs(synth.BASE_SEED + 9800, T, valid_len, hole_p)
    x, valid = dev(xb), dev(valid_np, raw=True)
    kc = torch.empty((HK, T, D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    ws = dmx.new_prefix_workspace(T)
    out = torch.empty_like(x)
    per_copy = sum(v.numel() for v in wd.values()) * 2 + (x.numel() + 2 * kc.numel()) * 2
    n = max(2, -(-ROTATE_BYTES // per_copy))
    ops = [(wd, x, kc, vc)] + [({k: v.clone() for k, v in wd.items()}, x.clone(), torch.empty_like(kc),
                                torch.empty_like(vc)) for _ in range(n - 1)]
    us = time_calls(lambda s, i: dmx.prefix_layer_forward(ops[i % n][0], ops[i % n][1], valid, ops[i % n][2],
                                                          ops[i % n][3], ws=ws, out=out, stream=s),
                    torch.cuda.Stream(), reps=2 * n)
    assert torch.isfinite(out.float()).all(), "non-finite prefix layer output"
    # key j is visible to query i when j <= i and j is valid
    pairs = int(np.cumsum(valid_np.astype(np.int64)).sum())
    attn_flops = 4 * HQ * D * pairs
    w_elems = (HQ + 2 * HK) * D * PH + PH * HQ * D + 2 * PI * PH + PH * PI
    flops = 2 * T * w_elems + attn_flops
    nbytes = w_elems * 2 + 5 * PH * 2 + 2 * T * PH * 2 + 2 * HK * T * D * 2
    q = torch.randn((T, HQ, D), device="cuda").to(torch.bfloat16)
    ctx = torch.empty_like(q)
    qs = [q] + [q.clone() for _ in range(n - 1)]
    us_attn = time_calls(lambda s, i: dmx.prefix_attention(qs[i % n], ops[i % n][2], ops[i % n][3], valid, ctx=ctx,
                                                           stream=s),
                         torch.cuda.Stream(), reps=2 * n)
    del ops, qs
    attn_bytes = 2 * T * HQ * D * 2 + 2 * HK * T * D * 2 + T
    return {"workload": f"prefix decoder layer, hidden 2560, {T} tokens ({int(valid_np.sum())} valid)",
            "us": round(us, 2), "operand_copies": n, "flops": flops, "tflops": round(flops / (us * 1e-6) / 1e12, 1),
            "mfma_frac": round(flops / (us * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4), "algorithmic_bytes": nbytes,
            "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "attention": {"us": round(us_attn, 2), "flops": attn_flops,
                          "tflops": round(attn_flops / (us_attn * 1e-6) / 1e12, 1),
                          "mfma_frac": round(attn_flops / (us_attn * 1e-6) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "algorithmic_bytes": attn_bytes}}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, wbits, rq, conds, n_steps_sample, n_layers_single):
    """Time the float64 C oracle on the host: whole denoise steps (all layers)
    of the same workload on every core, and a few layers on one thread
    (scaled to a step); report ms per step."""
    import oracle as orc
    from masked_gqa_attention_action_amd import synth
    f = synth.bf16_to_f64
    ow = [{k: f(v) for k, v in w.items()} for w in wbits]
    kp = [f(rq.k_pre[l]) for l in range(wl.n_layers)]
    vp = [f(rq.v_pre[l]) for l in range(wl.n_layers)]
    cond = f(conds[0])

    def run(n_layers):
        x = f(rq.x)
        t0 = time.perf_counter()
        for i in range(n_layers):
            l = i % wl.n_layers
            x = orc.layer(x, cond, ow[l], kp[l], vp[l], rq.mask, rq.pos0)
        return time.perf_counter() - t0

    threads = orc.set_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    dt = run(n_steps_sample * wl.n_layers)
    out = {"value": round(dt / n_steps_sample * 1e3, 2), "unit": "ms/step", "cores": threads, "kind": "oracle",
           "cpu_model": cpu_model(),
           "sample": f"{n_steps_sample} whole denoise steps ({n_steps_sample * wl.n_layers} layer evaluations) of "
                     f"the same workload by the float64 C oracle on {threads} threads, {dt:.1f} s wall"}
    if n_layers_single > 0:
        orc.set_threads(1)
        dt1 = run(n_layers_single)
        orc.set_threads(threads)
        out["single_thread"] = {
            "value": round(dt1 / n_layers_single * wl.n_layers * 1e3, 1), "unit": "ms/step", "cores": 1,
            "sample": f"{n_layers_single} layer evaluations on one thread, {dt1:.1f} s wall, scaled to "
                      f"{wl.n_layers} layers"}
    return out


def copy_bandwidth(nbytes=1 << 30, reps=10):
    """GB/s of a plain device-to-device copy (bytes read + bytes written)."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    e1.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return round(gbs, 1)


def stack_c3(dmx, reps=3):
    """The 18-layer x 10-step stack at the P_b=896 bucket, chunk 50, captured
    as one graph (the whole denoise loop per replay): ms per step."""
    import torch
    from masked_gqa_attention_action_amd import synth
    wl = synth.WORKLOADS["c3"]
    L = wl.n_layers
    wbits = [synth.layer_weights(wl.weight_seed(l)) for l in range(L)]
    rq = synth.make_request(wl.request_seed(0), wl.chunk, wl.p_bucket, wl.len_lo, wl.len_hi, L, wl.hole_p)
    conds = np.stack([synth.time_embedding(t) for t in synth.step_times(wl.n_steps)])
    wd = [dmx.pack_layer_weights({k: dev(v) for k, v in w.items()}) for w in wbits]
    kp = [dev(rq.k_pre[l][None]) for l in range(L)]
    vp = [dev(rq.v_pre[l][None]) for l in range(L)]
    x0 = dev(rq.x[None])
    x = x0.clone()
    st = dmx.Stack(wd, kp, vp, dev(rq.mask[None], raw=True), dev(conds[:, None, :]),
                   dev(np.array([rq.pos0], np.int32), raw=True), x)
    stream = torch.cuda.Stream()
    st.capture(stream)
    ms = time_replays(st, stream, 1, reps) / wl.n_steps
    assert torch.isfinite(x.float()).all(), "non-finite activations (c3)"
    st.close()
    visible = int(rq.mask.sum())
    nbytes = L * algorithmic_bytes_per_layer(1, wl.chunk, wl.p_bucket, visible)
    return {"workload": wl.note, "ms_per_step": round(ms, 4), "steps_per_replay": wl.n_steps,
            "visible_prefix_rows": visible, "algorithmic_bytes_per_step": nbytes,
            "frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}


def progress(msg):
    """A line per finished phase, on stderr (stdout carries only the result)."""
    print(f"bench.py: {msg}", file=sys.stderr, flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="step1024")
    ap.add_argument("--cpu-steps", type=int, default=8, help="denoise steps the oracle runs for the CPU baseline "
                                                            "on every core (0: skip the CPU baseline)")
    ap.add_argument("--cpu-single-layers", type=int, default=4, help="layer evaluations the oracle runs on one "
                                                                     "thread for the CPU baseline (0: skip)")
    ap.add_argument("--kernel-reps", type=int, default=20, help="replays per kernel for per-kernel timing (0: skip)")
    ap.add_argument("--variants", type=int, default=1, help="also time the cached-modulation variants (0: skip)")
    ap.add_argument("--extras", type=int, default=1, help="also time single layers of the batched and long-prefix "
                                                          "workloads and the prefix QKV (0: skip)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU; --gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import masked_gqa_attention_action_amd as dmx
    from masked_gqa_attention_action_amd import synth

    wl = synth.WORKLOADS[args.workload]
    B, C, P, L = wl.batch, wl.chunk, wl.p_bucket, wl.n_layers
    wbits = [synth.layer_weights(wl.weight_seed(l)) for l in range(L)]
    rq = synth.make_request(wl.request_seed(0), C, P, wl.len_lo, wl.len_hi, L, wl.hole_p)
    conds = np.stack([synth.time_embedding(t) for t in synth.step_times(wl.n_steps)])
    visible = int(rq.mask.sum())

    torch.cuda.set_device(0)
    wd = [dmx.pack_layer_weights({k: dev(v) for k, v in w.items()}) for w in wbits]
    kp = [dev(rq.k_pre[l][None]) for l in range(L)]
    vp = [dev(rq.v_pre[l][None]) for l in range(L)]
    mask = dev(rq.mask[None], raw=True)
    cond = dev(conds[:1, None, :])          # one denoise step per replay
    pos0 = dev(np.array([rq.pos0], np.int32), raw=True)
    x = dev(rq.x[None])
    st = dmx.Stack(wd, kp, vp, mask, cond, pos0, x)
    stream = torch.cuda.Stream()
    st.capture(stream)
    ms_step = time_replays(st, stream, args.warmup, args.steps)
    assert torch.isfinite(x.float()).all(), "non-finite activations"
    progress(f"headline step timed: {ms_step:.4f} ms")

    # Reported beside the headline, never as it: the same step with the
    # modulation vectors read from a table filled once per timestep schedule,
    # and the whole denoise loop captured as one graph with that table.
    variants = {}
    if args.variants:
        x.copy_(dev(rq.x[None]))
        with torch.cuda.stream(stream):
            tb = dmx.Stack(wd, kp, vp, mask, cond, pos0, x, mod_table=True, stream=stream)
        tb.capture(stream)
        # no double credit: the modulation weights are not read in these steps
        # (the table's two vectors per layer and request are)
        tb_bytes = L * (algorithmic_bytes_per_layer(B, C, P, visible) - 2 * W_MOD + 2 * B * 3072 * 4)
        ms_tb = time_replays(tb, stream, args.warmup, args.steps)
        variants["mod_table_step"] = {"ms_per_step": round(ms_tb, 4), "algorithmic_bytes": tb_bytes,
                                      "frac_of_hbm_peak": round(tb_bytes / (ms_tb * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                      "note": "one step per replay, modulation vectors precomputed per schedule"}
        tb.close()
        # the same step as one persistent kernel (batch 1: the whole stack in
        # one launch, weights prefetched across its stage hand-offs)
        x.copy_(dev(rq.x[None]))
        ps = dmx.Stack(wd, kp, vp, mask, cond, pos0, x, persistent=True)
        ps.capture(stream)
        ms_ps = time_replays(ps, stream, args.warmup, args.steps)
        ps.sync_check(stream)
        assert torch.isfinite(x.float()).all(), "non-finite activations (persistent)"
        step_b = L * algorithmic_bytes_per_layer(B, C, P, visible)
        variants["persistent_step"] = {"ms_per_step": round(ms_ps, 4), "algorithmic_bytes": step_b,
                                       "frac_of_hbm_peak": round(step_b / (ms_ps * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                       "note": "one step per replay as a single persistent kernel (k_step)"}
        ps.close()
        # the whole denoise loop as one graph, the same work per step as the
        # headline (modulation vectors computed in every step, no table)
        x.copy_(dev(rq.x[None]))
        cond_all = dev(conds[:, None, :])
        lpn = dmx.Stack(wd, kp, vp, mask, cond_all, pos0, x)
        lpn.capture(stream)
        n = max(1, args.steps // wl.n_steps)
        ms_lpn = time_replays(lpn, stream, max(1, args.warmup // wl.n_steps), n) / wl.n_steps
        variants["step_loop"] = {"ms_per_step": round(ms_lpn, 4), "algorithmic_bytes": L * algorithmic_bytes_per_layer(
            B, C, P, visible), "frac_of_hbm_peak": round(L * algorithmic_bytes_per_layer(B, C, P, visible) /
                                                          (ms_lpn * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                 "note": f"whole {wl.n_steps}-step denoise loop per replay, the headline's work per step "
                                         "(modulation computed in every step)"}
        lpn.close()
        x.copy_(dev(rq.x[None]))
        with torch.cuda.stream(stream):
            lp = dmx.Stack(wd, kp, vp, mask, cond_all, pos0, x, mod_table=True, stream=stream)
        lp.capture(stream)
        ms_loop = time_replays(lp, stream, max(1, args.warmup // wl.n_steps), n)
        ms_lp = ms_loop / wl.n_steps
        variants["mod_table_loop"] = {"ms_per_step": round(ms_lp, 4), "algorithmic_bytes": tb_bytes,
                                      "frac_of_hbm_peak": round(tb_bytes / (ms_lp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                      "note": f"whole {wl.n_steps}-step denoise loop per replay, modulation "
                                              "vectors precomputed per schedule"}
        lp.close()
        # the full sampler: per step the action in-projection, the stack (with
        # the table) and the final norm + out-projection + Euler update
        x.copy_(dev(rq.x[None]))
        swd = dmx.pack_sampler_weights({k: dev(v) for k, v in synth.sampler_weights(wl.seed + 50).items()})
        A = synth.ACTION_DIM
        acts = torch.from_numpy(synth.sampler_noise(wl.seed + 60, B, C)).cuda()
        cond_s = torch.empty_like(cond_all)
        with torch.cuda.stream(stream):
            sp_stack = dmx.Stack(wd, kp, vp, mask, cond_s, pos0, x, mod_table=True, stream=stream)
            sp = dmx.Sampler(sp_stack, swd, acts, stream=stream)
        sp.capture(stream)
        ms_sp = time_replays(sp, stream, max(1, args.warmup // wl.n_steps), n) / wl.n_steps
        assert torch.isfinite(acts).all(), "non-finite actions"
        sp_bytes = tb_bytes + 2 * A * H * 2 + (H + A) * 2 + 2 * H * 4 + 2 * B * C * A * 4
        variants["sampler_loop"] = {"ms_per_step": round(ms_sp, 4), "algorithmic_bytes": sp_bytes,
                                    "frac_of_hbm_peak": round(sp_bytes / (ms_sp * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                                    "note": f"whole {wl.n_steps}-step sampler per replay: action in-projection, "
                                            "stack with precomputed modulation, final norm + out-projection + "
                                            "Euler update"}
        sp.close()
        sp_stack.close()
        assert torch.isfinite(x.float()).all(), "non-finite activations"
        x.copy_(dev(rq.x[None]))
        torch.cuda.synchronize()
        progress("variants timed")

    step_bytes = L * algorithmic_bytes_per_layer(B, C, P, visible)
    step_flops = L * layer_flops(B, C, visible)
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # per-kernel timing (after the timed region) and the dominant kernel, on
    # a 64-layer timing stack whose operands exceed the memory-side cache
    kernels = {}
    st.close()
    if args.kernel_reps > 0:
        tst = timing_stack(dmx, wd, kp, vp, mask, cond, pos0, x)
        for stage, name in enumerate(dmx.STAGE_NAMES):
            us = time_stage(tst, stage, TIMING_LAYERS, stream, args.kernel_reps)
            per_step = 1 if stage in (dmx.STAGE_MODS, dmx.STAGE_PACK) else L
            nbytes = stage_bytes(stage, B, C, P, visible, L)
            kernels[name] = {"us_per_launch": round(us, 3), "launches_per_step": per_step,
                             "share_of_step": round(us * per_step / (ms_step * 1e3), 4),
                             "algorithmic_bytes": nbytes,
                             "gbs": round(nbytes / (us * 1e-6) / 1e9, 1) if nbytes else None}
        tst.close()
        del tst
        # the attention's own launch: with a modulation table the launch
        # carries no modulation GEMVs on its idle CUs; the difference to the
        # step's attention launch is what those GEMVs add
        ttb = timing_stack(dmx, wd, kp, vp, mask, cond, pos0, x, mod_table=True)
        us_own = time_stage(ttb, dmx.STAGE_ATTN, TIMING_LAYERS, stream, args.kernel_reps)
        ttb.close()
        del ttb
        own_bytes = stage_bytes(dmx.STAGE_ATTN, B, C, P, visible, 1)  # no modulation weights
        kernels["attention (own)"] = {
            "us_per_launch": round(us_own, 3), "launches_per_step": L, "algorithmic_bytes": own_bytes,
            "gbs": round(own_bytes / (us_own * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(own_bytes / (us_own * 1e-6) / 1e9 / PEAK_HBM_GBS, 4),
            "note": "the attention launch alone (modulation vectors from a table): KV, queries, suffix K/V, context"}
        side = kernels["attention"]["algorithmic_bytes"] - own_bytes
        extra = kernels["attention"]["us_per_launch"] - us_own
        kernels["side modulation GEMVs"] = {
            "us_added_per_launch": round(extra, 3), "algorithmic_bytes": side,
            "note": "the next layer's two modulation GEMVs on the CUs the attention leaves idle: what they add to "
                    "the attention launch"}
        torch.cuda.synchronize()
        progress("per-kernel timings done")
    extras = {}
    if args.extras:
        for name in ("c1", "c2", "c4", "c5"):
            extras[f"layer_{name}"] = layer_case(name)
            progress(f"layer {name} timed")
        extras["prefix_qkv_c4"] = prefix_qkv_case()
        extras["prefix_layer_2048"] = prefix_layer_case()
        progress("prefix workloads timed")
        extras["stack_c3"] = stack_c3(dmx)
        torch.cuda.synchronize()
        progress("c3 stack timed")
    copy_gbs = copy_bandwidth()
    # a plain 256 MiB device copy, the run's last: the reference dispatch for
    # HBM byte counters
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst

    roofline = {"bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": None,
                "traffic": None, "measured_copy_gbs": copy_gbs}
    if kernels:
        name = max((k for k in kernels if "share_of_step" in kernels[k]), key=lambda k: kernels[k]["share_of_step"])
        k = kernels[name]
        tag = name.replace(" ", "_").replace("+", "_")
        roofline.update({"kernel": name, "achieved": k["gbs"],
                         "frac": round(k["gbs"] / PEAK_HBM_GBS, 4) if k["gbs"] else None,
                         "traffic": recorded_traffic(f"{tag}_{args.workload}"),
                         "us_per_launch": k["us_per_launch"], "algorithmic_bytes_per_launch": k["algorithmic_bytes"]})
    out = {
        "metric": "ms per denoise step (action-expert stack) at P=1024, chunk 50; % HBM roofline",
        "value": round(ms_step, 4),
        "unit": "ms/step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,0.02) weights, N(0,1) prefix KV, sin/cos time embedding)",
        "config": {"workload": wl.note, "layers": L, "batch": B, "chunk": C, "p_bucket": P,
                   "visible_prefix_rows": visible, "steps_per_replay": 1},
        "roofline": roofline,
        "step": {"algorithmic_bytes": step_bytes, "flops": step_flops, "achieved_gbs": round(step_gbs, 1),
                 "frac_of_hbm_peak": round(step_gbs / PEAK_HBM_GBS, 4)},
        "kernels": kernels,
        "variants": variants,
        "extras": extras,
    }
    if args.cpu_steps > 0:
        out["cpu_baseline"] = cpu_baseline(wl, wbits, rq, conds, args.cpu_steps, args.cpu_single_layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
