"""GPU: no entry point reads memory it has not written first.

Every workspace and every buffer the ABI writes is filled with zero bytes for
one run and with 0xFF bytes (NaN in bf16 / fp32) for another; the outputs of
the two runs must be bit-identical (and finite).  Covered: the layer at one
request and at 16 requests, the stack eagerly and from a graph, the prefix
layer (output and K/V cache rows), and a whole denoising run of the sampler
(schedule, stack workspace, trajectory).
"""
from __future__ import annotations

import numpy as np
import pytest

from masked_gqa_attention_action_amd import synth
from tests.helpers import device_weights, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

FILLS = (0x00, 0xFF)


@pytest.fixture(scope="module")
def dmx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_gqa_attention_action_amd as m
    m.lib()
    return m


def filled(shape, dtype, byte):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(byte)
    return t


def same_bits(a, b, what):
    assert a.dtype == b.dtype and a.shape == b.shape, what
    assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{what}: a poisoned buffer changed the result"


@pytest.mark.parametrize("wname", ["c2", "c5"])
def test_layer_poisoned_workspace_and_output(dmx, wname):
    wl = synth.WORKLOADS[wname]
    wd = device_weights(synth.layer_weights(wl.weight_seed(0)))
    reqs = [synth.make_request(wl.request_seed(b), wl.chunk, wl.p_bucket, wl.len_lo, wl.len_hi, 1, wl.hole_p)
            for b in range(wl.batch)]
    B, C, P = wl.batch, wl.chunk, wl.p_bucket
    x = to_dev(np.stack([r.x for r in reqs]))
    cond = to_dev(np.stack([r.cond for r in reqs]))
    kp = to_dev(np.stack([r.k_pre[0] for r in reqs]))
    vp = to_dev(np.stack([r.v_pre[0] for r in reqs]))
    mask = to_dev(np.stack([r.mask for r in reqs]), "raw")
    pos0 = to_dev(np.array([r.pos0 for r in reqs], np.int32), "raw")
    n = int(dmx.lib().dmx_workspace_bytes(B, C, P))
    outs = []
    for byte in FILLS:
        print(f"layer {wname}: buffers filled with {byte:#04x}", flush=True)
        ws = filled((n,), torch.uint8, byte)
        out = filled(x.shape, torch.bfloat16, byte)
        dmx.suffix_layer_forward(wd, kp, vp, mask, x, cond, pos0, ws, out=out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.isfinite(outs[1].float()).all()
    same_bits(outs[0], outs[1], f"layer {wname}")


def test_stack_poisoned_workspace_eager_and_graph(dmx):
    L, S, C, P = 4, 2, 50, 1024
    seed = synth.BASE_SEED + 9650
    wd = [device_weights(synth.layer_weights(seed + 100 + l)) for l in range(L)]
    rq = synth.make_request(seed, C, P, 700, 1024, L)
    conds = np.stack([synth.time_embedding(t) for t in synth.step_times(S)])
    kp = [to_dev(rq.k_pre[l][None]) for l in range(L)]
    vp = [to_dev(rq.v_pre[l][None]) for l in range(L)]
    mask = to_dev(rq.mask[None], "raw")
    cond = to_dev(conds[:, None, :])
    pos0 = to_dev(np.array([rq.pos0], np.int32), "raw")
    x0 = to_dev(rq.x[None])
    n = int(dmx.lib().dmx_stack_workspace_bytes(L, 1, C, P))
    res = []
    for byte in FILLS:
        print(f"stack {L} layers x {S} steps: workspace filled with {byte:#04x}", flush=True)
        x = x0.clone()
        ws = filled((n,), torch.uint8, byte)
        st = dmx.Stack(wd, kp, vp, mask, cond, pos0, x, ws=ws)
        st.run()
        torch.cuda.synchronize()
        eager = x.clone()
        ws.fill_(byte)
        x.copy_(x0)
        stream = torch.cuda.Stream()
        st.capture(stream)
        st.replay(stream)
        stream.synchronize()
        st.close()
        res.append((eager, x.clone()))
    assert torch.isfinite(res[1][0].float()).all()
    same_bits(res[0][0], res[1][0], "stack eager")
    same_bits(res[0][1], res[1][1], "stack graph replay")
    same_bits(res[0][0], res[0][1], "stack graph replay vs eager")


def test_prefix_layer_poisoned_workspace_output_and_cache(dmx):
    T, kv_rows = 300, 320
    wbits = synth.prefix_layer_weights(synth.BASE_SEED + 9500)
    wd = dmx.pack_prefix_weights({k: to_dev(v) for k, v in wbits.items()})
    x, valid = synth.prefix_inputs(synth.BASE_SEED + 9660, T, 280, 0.05)
    xd, vd = to_dev(x), to_dev(valid, "raw")
    n = int(dmx.lib().dmx_prefix_workspace_bytes(T))
    res = []
    for byte in FILLS:
        print(f"prefix layer T={T}: buffers filled with {byte:#04x}", flush=True)
        ws = filled((n,), torch.uint8, byte)
        out = filled((T, 2560), torch.bfloat16, byte)
        kc = filled((4, kv_rows, 256), torch.bfloat16, byte)
        vc = filled((4, kv_rows, 256), torch.bfloat16, byte)
        dmx.prefix_layer_forward(wd, xd, vd, kc, vc, ws=ws, out=out)
        torch.cuda.synchronize()
        res.append((out, kc[:, :T].contiguous(), vc[:, :T].contiguous(), kc[:, T:].contiguous()))
    assert torch.isfinite(res[1][0].float()).all()
    same_bits(res[0][0], res[1][0], "prefix layer output")
    same_bits(res[0][1], res[1][1], "prefix k cache")
    same_bits(res[0][2], res[1][2], "prefix v cache")
    # rows past the tokens keep the caller's bytes
    assert (res[0][3].view(torch.uint8) == 0x00).all() and (res[1][3].view(torch.uint8) == 0xFF).all()


def test_sampler_poisoned_schedule_workspace_and_trajectory(dmx):
    from tests.sampler_case import Case
    res = []
    for byte in FILLS:
        c = Case(2, 3, 1, 50, 1024, 700, 1024, 0.0, synth.BASE_SEED + 9670)
        print(f"sampler 2 layers x 3 steps: buffers filled with {byte:#04x}", flush=True)
        c.stack.ws.fill_(byte)
        c.traj.view(torch.uint8).fill_(byte)
        c.x.view(torch.uint8).fill_(byte)
        c.sampler.sched.fill_(byte)
        c.cond.view(torch.uint8).fill_(byte)
        c.sampler.fill_schedule()
        c.reset()
        c.sampler.run()
        torch.cuda.synchronize()
        res.append((c.actions.clone(), c.traj.clone()))
    assert torch.isfinite(res[1][1]).all()
    same_bits(res[0][0], res[1][0], "sampler actions")
    same_bits(res[0][1], res[1][1], "sampler trajectory")
