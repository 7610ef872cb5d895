"""Benchmark: ms per denoise step of the 18-layer action-expert stack at the
P_b=1024 prefix bucket, chunk 50, batch 1, and its fraction of the MI355X HBM
roofline.

One step = the whole hot path once: 18 action-expert layers (AdaRMS, QKV +
QK-norm + RoPE, masked GQA attention over prefix + suffix KV, gated residuals,
GEGLU MLP) for one denoising step, replayed from a hipGraph captured for the
1024 bucket.  Inputs (seeded synthetic weights, KV cache, mask, time
embedding) are resident in HBM before timing starts.

Prints one JSON line.  --gpus above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
LAYER_WEIGHT_BYTES = 50_344_960  # 10 weight tensors of one layer, bf16


def algorithmic_bytes_per_layer(batch, chunk, p_bucket, visible_rows_total):
    """Bytes one layer must move: its weights, the visible prefix K/V rows, and
    its own inputs and outputs (x in and out, cond, mask, pos0)."""
    kv = 2 * 4 * 256 * 2 * visible_rows_total
    io = batch * (2 * chunk * 1024 * 2 + 1024 * 2 + p_bucket + 4)
    return LAYER_WEIGHT_BYTES + kv + io


def layer_flops(batch, chunk, visible_rows_total):
    proj = 2 * batch * chunk * (1024 * 4096 + 2048 * 1024 + 1024 * 8192 + 4096 * 1024)
    mod = 2 * batch * 2 * 1024 * 3072
    attn = 4 * 8 * 256 * chunk * (visible_rows_total + batch * chunk)
    return proj + mod + attn


def dev(bits, raw=False):
    import torch
    a = np.ascontiguousarray(bits)
    t = torch.from_numpy(a) if raw else torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    return t.cuda()


def cpu_baseline(wl, wbits, rq, conds, n_layers_sample):
    """Time the float64 oracle on the host for a few layers of the same
    workload and scale to one denoise step."""
    import oracle as orc
    from masked_gqa_attention_action_amd import synth
    threads = orc.set_threads(int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)))
    f = synth.bf16_to_f64
    x = f(rq.x)
    t0 = time.perf_counter()
    for l in range(n_layers_sample):
        ow = {k: f(v) for k, v in wbits[l].items()}
        x = orc.layer(x, f(conds[0]), ow, f(rq.k_pre[l]), f(rq.v_pre[l]), rq.mask, rq.pos0)
    dt = time.perf_counter() - t0
    ms_step = dt / n_layers_sample * wl.n_layers * 1e3
    return {"value": round(ms_step, 3), "unit": "ms/step", "cores": threads, "kind": "oracle",
            "sample": f"{n_layers_sample} of the step's {wl.n_layers} layers (float64 C oracle, same inputs), "
                      f"{dt:.2f} s wall, scaled to one step"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="step1024")
    ap.add_argument("--cpu-layers", type=int, default=3, help="oracle layers timed for the CPU baseline (0: skip)")
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
    x0 = dev(rq.x[None])
    x = x0.clone()
    st = dmx.Stack(wd, kp, vp, mask, cond, pos0, x)
    stream = torch.cuda.Stream()
    st.capture(stream)

    for _ in range(args.warmup):
        st.replay(stream)
    stream.synchronize()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(args.steps):
        st.replay(stream)
    ev1.record(stream)
    ev1.synchronize()
    torch.cuda.synchronize()
    ms_step = ev0.elapsed_time(ev1) / args.steps
    st.close()
    assert torch.isfinite(x.float()).all(), "non-finite activations"

    step_bytes = L * algorithmic_bytes_per_layer(B, C, P, visible)
    step_flops = L * layer_flops(B, C, visible)
    achieved = step_bytes / (ms_step * 1e-3) / 1e9
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
        "roofline": {"bound": "hbm", "kernel": "denoise-step graph (all kernels of 18 layers)",
                     "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes": step_bytes, "flops": step_flops},
    }
    if args.cpu_layers > 0:
        out["cpu_baseline"] = cpu_baseline(wl, wbits, rq, conds, args.cpu_layers)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
