"""GPU: the persistent step kernel (a batch-1 stack in one launch,
dmx_stack_desc.persistent = 1), through the C ABI.

- every layer's output (the kernel's layer trace) against the oracle layer
  with teacher forcing: the oracle gets the GPU's bf16 input to that layer;
- the run's final output equals the trace's last layer;
- eager runs and graph replays are bit-identical (with unrelated eager work
  between replays), also over a workspace filled with NaN bytes;
- masked prefix rows filled with NaN / Inf do not change a single output bit;
- shapes: chunk 50 at the 1024 bucket (the benchmarked step), chunk 10 at 576,
  chunk 64 at 2048 with 5 % holes (three 32-key blocks per split), chunk 1,
  several steps with and without the modulation table.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
from masked_gqa_attention_action_amd import synth
from tests.helpers import LAYER_BRANCH_REL, delta_gate, device_weights, f64, from_dev, gate, oracle_weights, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dmx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_gqa_attention_action_amd as m
    m.lib()
    return m


def make_case(seed, n_layers, n_steps, chunk, p_bucket, len_lo, len_hi, hole_p=0.0):
    wbits = [synth.layer_weights(seed + 100 + l) for l in range(n_layers)]
    rq = synth.make_request(seed, chunk, p_bucket, len_lo, len_hi, n_layers, hole_p)
    conds = np.stack([synth.time_embedding(t) for t in synth.step_times(n_steps)])
    dev = dict(
        wd=[device_weights(w) for w in wbits],
        kp=[to_dev(rq.k_pre[l][None]) for l in range(n_layers)],
        vp=[to_dev(rq.v_pre[l][None]) for l in range(n_layers)],
        mask=to_dev(rq.mask[None], "raw"),
        cond=to_dev(conds[:, None, :]),
        pos0=to_dev(np.array([rq.pos0], np.int32), "raw"),
        x0=to_dev(rq.x[None]),
    )
    return dict(wbits=wbits, rq=rq, conds=conds, n_layers=n_layers, n_steps=n_steps, chunk=chunk, dev=dev)


def persistent_stack(dmx, c, x, trace=None, mod_table=False, kp=None, vp=None, ws=None):
    d = c["dev"]
    return dmx.Stack(d["wd"], kp or d["kp"], vp or d["vp"], d["mask"], d["cond"], d["pos0"], x, ws=ws,
                     mod_table=mod_table, persistent=True, trace=trace)


def run_once(dmx, c, **kw):
    d = c["dev"]
    x = d["x0"].clone()
    tr = torch.full((c["n_steps"], c["n_layers"], 1, c["chunk"], 1024), float("nan"), dtype=torch.bfloat16,
                    device="cuda")
    st = persistent_stack(dmx, c, x, trace=tr, **kw)
    print(f"persistent run: L={c['n_layers']} steps={c['n_steps']} C={c['chunk']} P={d['mask'].shape[1]} "
          f"{kw.get('mod_table', False) and 'table' or ''}", flush=True)
    st.run()
    st.sync_check()
    return x, tr, st


def check_teacher_forced(c, x, tr, layers=None):
    rq = c["rq"]
    L, S = c["n_layers"], c["n_steps"]
    assert torch.equal(x[0], tr[S - 1, L - 1, 0]), "final output differs from the last traced layer"
    for s in range(S):
        for l in range(L):
            if layers is not None and (s, l) not in layers:
                continue
            if s == 0 and l == 0:
                xin = f64(rq.x)
            elif l == 0:
                xin = from_dev(tr[s - 1, L - 1, 0])
            else:
                xin = from_dev(tr[s, l - 1, 0])
            ref = orc.layer(xin, f64(c["conds"][s]), oracle_weights(c["wbits"][l]), f64(rq.k_pre[l]),
                            f64(rq.v_pre[l]), rq.mask, rq.pos0)
            got = from_dev(tr[s, l, 0])
            gate(f"step {s} layer {l}", got, ref)
            delta_gate(f"step {s} layer {l} branch", got, ref, xin, rel=LAYER_BRANCH_REL)


CASES = {
    # name: (seed, layers, steps, chunk, p_bucket, len_lo, len_hi, hole_p)
    "step1024": (synth.BASE_SEED + 9100, 18, 1, 50, 1024, 700, 1024, 0.0),
    "c1": (synth.BASE_SEED + 9200, 4, 1, 10, 576, 512, 512, 0.0),
    "p2048_c64": (synth.BASE_SEED + 9300, 3, 1, 64, 2048, 1900, 2048, 0.05),
    "chunk1": (synth.BASE_SEED + 9400, 2, 1, 1, 704, 600, 704, 0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_step_every_layer_teacher_forced(dmx, name):
    c = make_case(*CASES[name])
    x, tr, st = run_once(dmx, c)
    torch.cuda.synchronize()
    assert torch.isfinite(x.float()).all()
    check_teacher_forced(c, x, tr)


@pytest.mark.parametrize("mod_table", [False, True])
def test_step_several_steps(dmx, mod_table):
    """Three steps of three layers in one launch: every step's conditioning,
    the modulation vectors computed ahead (two layers ahead, across the step
    boundary) or read from the table."""
    c = make_case(synth.BASE_SEED + 9500, 3, 3, 50, 896, 769, 896)
    x, tr, st = run_once(dmx, c, mod_table=mod_table)
    torch.cuda.synchronize()
    check_teacher_forced(c, x, tr)


def test_step_deterministic_graph_and_poisoned_workspace(dmx):
    c = make_case(synth.BASE_SEED + 9600, 4, 2, 50, 1024, 700, 1024)
    x1, tr1, st1 = run_once(dmx, c)
    x2, tr2, st2 = run_once(dmx, c)
    torch.cuda.synchronize()
    assert torch.equal(x1, x2) and torch.equal(tr1, tr2), "two eager runs differ"
    # a workspace full of NaN bytes (the run resets its own counters)
    n = int(dmx.lib().dmx_stack_workspace_bytes(4, 1, 50, 1024))
    ws = torch.full((n,), 0xFF, dtype=torch.uint8, device="cuda")
    x3, tr3, st3 = run_once(dmx, c, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(x1, x3) and torch.equal(tr1, tr3), "a NaN-filled workspace changed the result"
    # graph replays
    xg = c["dev"]["x0"].clone()
    trg = torch.zeros_like(tr1)
    stg = persistent_stack(dmx, c, xg, trace=trg)
    stream = torch.cuda.Stream()
    stg.capture(stream)
    for rep in range(3):
        xg.copy_(c["dev"]["x0"])
        torch.cuda.synchronize()
        stg.replay(stream)
        stream.synchronize()
        stg.sync_check(stream)
        assert torch.equal(xg, x1) and torch.equal(trg, tr1), f"graph replay {rep} differs"
        _ = (xg.float() * 2).sum().item()  # unrelated eager work between replays
    stg.close()


def test_step_masked_rows_never_read(dmx):
    c = make_case(synth.BASE_SEED + 9700, 2, 1, 50, 1024, 700, 800)
    x1, tr1, _ = run_once(dmx, c)
    inv = torch.from_numpy(c["rq"].mask == 0).cuda()
    kp, vp = [], []
    for l in range(c["n_layers"]):
        k = c["dev"]["kp"][l].clone()
        v = c["dev"]["vp"][l].clone()
        k[0, :, inv] = float("nan")
        v[0, :, inv] = float("inf")
        kp.append(k)
        vp.append(v)
    x2 = c["dev"]["x0"].clone()
    tr2 = torch.zeros_like(tr1)
    st = persistent_stack(dmx, c, x2, trace=tr2, kp=kp, vp=vp)
    st.run()
    st.sync_check()
    torch.cuda.synchronize()
    assert torch.equal(x1, x2) and torch.equal(tr1, tr2), "poison in masked rows reached the output"


def test_step_matches_stage_mode(dmx):
    """The persistent kernel and the stage kernels agree to the layer gate on
    one layer of the benchmarked shape (their summation orders differ); over
    the 18 layers of a step their outputs drift apart by bf16 rounding, so
    the whole step is held to the cosine only (the per-layer gates above
    are the parity checks)."""
    for L in (1, 18):
        c = make_case(synth.BASE_SEED + 9800, L, 1, 50, 1024, 700, 1024)
        x1, _, _ = run_once(dmx, c)
        d = c["dev"]
        x2 = d["x0"].clone()
        st = dmx.Stack(d["wd"], d["kp"], d["vp"], d["mask"], d["cond"], d["pos0"], x2)
        st.run()
        torch.cuda.synchronize()
        if L == 1:
            gate("persistent vs stage mode, one layer", from_dev(x1[0]), from_dev(x2[0]))
        else:
            gate(f"persistent vs stage mode, {L} layers", from_dev(x1[0]), from_dev(x2[0]), rel=float("inf"))
