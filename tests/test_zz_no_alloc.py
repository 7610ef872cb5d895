"""The allocation-free layer entry point (dmx_suffix_layer_forward_noalloc)
against the workspace entry point (dmx_suffix_layer_forward), through the C
ABI: the same kernels, so the outputs must agree bit for bit.  Two calls in a
row share the library's fixed scratch, the second at smaller sizes (so it
runs over whatever the first left there), and sizes beyond the scratch are
refused before anything is launched."""
from __future__ import annotations

import numpy as np
import pytest

from masked_gqa_attention_action_amd import synth
from tests.helpers import device_weights, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dmx():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_gqa_attention_action_amd as m
    m.lib()
    return m


def _inputs(wname):
    wl = synth.WORKLOADS[wname]
    wbits = synth.layer_weights(wl.weight_seed(0))
    reqs = [synth.make_request(wl.request_seed(b), wl.chunk, wl.p_bucket, wl.len_lo, wl.len_hi, 1, wl.hole_p)
            for b in range(wl.batch)]
    dev = dict(
        x=to_dev(np.stack([r.x for r in reqs])),
        cond=to_dev(np.stack([r.cond for r in reqs])),
        k=to_dev(np.stack([r.k_pre[0] for r in reqs])),
        v=to_dev(np.stack([r.v_pre[0] for r in reqs])),
        mask=to_dev(np.stack([r.mask for r in reqs]), "raw"),
        pos0=to_dev(np.array([r.pos0 for r in reqs], np.int32), "raw"),
    )
    return wbits, dev


def _with_workspace(dmx, wd, d):
    B, C, _ = d["x"].shape
    ws = dmx.new_workspace(B, C, d["k"].shape[2])
    ws.fill_(0xFF)  # NaN bytes: the layer must not read anything it did not write
    out = torch.full_like(d["x"], float("nan"))
    dmx.suffix_layer_forward(wd, d["k"], d["v"], d["mask"], d["x"], d["cond"], d["pos0"], ws, out=out)
    torch.cuda.synchronize()
    return out


def test_noalloc_layer_matches_workspace_entry_point_twice(dmx):
    # first call: chunk 50 at the 1024 bucket; second: chunk 10 at 576, over
    # the first call's scratch contents
    for wname in ("c2", "c1"):
        wbits, d = _inputs(wname)
        wd = device_weights(wbits)
        want = _with_workspace(dmx, wd, d)
        got = torch.full_like(d["x"], float("nan"))
        print(f"noalloc {wname}: B={d['x'].shape[0]} C={d['x'].shape[1]} P={d['k'].shape[2]}", flush=True)
        dmx.suffix_layer_forward_noalloc(wd, d["k"], d["v"], d["mask"], d["x"], d["cond"], d["pos0"], got)
        torch.cuda.synchronize()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"{wname}: outputs differ"


def test_noalloc_refuses_sizes_beyond_its_scratch(dmx):
    wbits, d = _inputs("c2")
    wd = device_weights(wbits)
    B, C, P = 2, 64, 2048  # needs about 23 MiB, above the 12 MiB scratch
    assert dmx.workspace_bytes(B, C, P) > dmx.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((B, C, 1024), dtype=torch.bfloat16, device="cuda")
    out = torch.full_like(x, 7.0)
    kp = torch.zeros((B, 4, P, 256), dtype=torch.bfloat16, device="cuda")
    mask = torch.zeros((B, P), dtype=torch.uint8, device="cuda")
    cond = torch.zeros((B, 1024), dtype=torch.bfloat16, device="cuda")
    pos0 = torch.zeros((B,), dtype=torch.int32, device="cuda")
    with pytest.raises(dmx.DmxError) as e:
        dmx.suffix_layer_forward_noalloc(wd, kp, kp, mask, x, cond, pos0, out)
    assert e.value.status == dmx.ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()), "a refused call must launch nothing"
