"""GPU: the denoise sampler around the action-expert stack, through the C ABI,
against the float64 oracle.

- schedule: the step conditioning (bf16, one copy per request) and the final
  norm's modulation of every step;
- every step with teacher forcing: the oracle starts from the GPU's actions
  before the step, and the step's velocity (a_k+1 - a_k) / dt is gated like a
  layer output;
- the sampler's tail alone (final AdaRMS, out-projection, Euler update) at the
  layer gate: the last step's velocity against the oracle's tail applied to
  the stack output the GPU produced;
- graph replay == eager run, bit for bit, also on new noise; with and without
  the modulation table, bit for bit;
- a small run end to end against the oracle's free run (cosine);
- the 18-layer, 10-step run at the P_b=896 bucket, every step teacher forced;
- action dimensions from 16 to 128 (one to four out-projection passes), every
  step teacher forced, with and without the table bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle as orc
from masked_gqa_attention_action_amd import synth
from tests.helpers import ERR_REL_RMS, f64, from_dev, gate, stage_gate

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from tests.sampler_case import Case


@pytest.fixture(scope="module")
def small():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Case(2, 3, 2, 10, 576, 500, 576, 0.05, synth.BASE_SEED + 7000)
    yield c
    c.sampler.close()
    c.stack.close()
    torch.cuda.synchronize()


def test_schedule_against_oracle():
    c = Case(1, 10, 3, 10, 576, 512, 512, 0.0, synth.BASE_SEED + 7100)
    torch.cuda.synchronize()
    sw, _ = c.oracle_inputs()
    cond = from_dev(c.cond)
    fmod = c.sampler.sched[: c.n_steps * 2 * synth.H * 4].view(torch.float32)
    fmod = from_dev(fmod).reshape(c.n_steps, 2 * synth.H)
    for k in range(c.n_steps):
        for b in range(1, c.B):
            assert np.array_equal(cond[k, b], cond[k, 0]), "conditioning differs between requests"
        want = orc.time_condition(orc.step_time(k, c.n_steps), sw)
        stage_gate(f"cond step {k}", cond[k, 0], want)
        m = sw["w_fmod"] @ want + sw["b_fmod"]
        gate(f"final modulation step {k}", fmod[k], m)


def teacher_forced_steps(c, sw, layers, steps=None):
    """Gate each step's velocity, the oracle starting from the GPU's actions
    before the step.  The step runs all n_layers layers without teacher
    forcing in between: each layer's output is within the layer gate
    (ERR_REL_RMS of its RMS, tested layer by layer in the stack tests), and
    independent per-layer errors add in quadrature, so the velocity is held
    to ERR_REL_RMS * sqrt(n_layers) of its RMS and to the layer's cosine."""
    traj = from_dev(c.traj)
    rel = ERR_REL_RMS * np.sqrt(c.n_layers)
    worst = 0.0
    for k in (range(c.n_steps) if steps is None else steps):
        for b in range(c.B):
            r = c.rqs[b]
            a_prev = c.noise[b].astype(np.float64) if k == 0 else traj[k - 1, b]
            _, v = orc.sampler_step(a_prev, k, c.n_steps, sw, layers, [f64(r.k_pre[l]) for l in range(c.n_layers)],
                                    [f64(r.v_pre[l]) for l in range(c.n_layers)], r.mask, r.pos0)
            v_gpu = (traj[k, b] - a_prev) * (-c.n_steps)
            ratio, _ = gate(f"velocity step {k} request {b}", v_gpu, v, rel=rel)
            worst = max(worst, ratio)
    return worst


def tail_teacher_forced(c, sw):
    """Gate the last step's velocity against the oracle's final AdaRMS and
    out-projection applied to the stack output the GPU produced (the stack's
    x still holds it after the run): the sampler's own tail at the layer gate,
    with none of the layers' rounding in between."""
    k = c.n_steps - 1
    traj = from_dev(c.traj)
    x_last = from_dev(c.x)
    cond = orc.time_condition(orc.step_time(k, c.n_steps), sw)
    worst = 0.0
    for b in range(c.B):
        a_prev = c.noise[b].astype(np.float64) if k == 0 else traj[k - 1, b]
        v_gpu = (traj[k, b] - a_prev) * (-c.n_steps)
        v = orc.final_velocity(x_last[b], cond, sw["w_fmod"], sw["b_fmod"], sw["w_out"], sw["b_out"])
        ratio, _ = gate(f"tail velocity step {k} request {b}", v_gpu, v)
        worst = max(worst, ratio)
    return worst


def test_steps_teacher_forced(small):
    c = small
    c.reset()
    c.sampler.run()
    torch.cuda.synchronize()
    assert torch.equal(c.actions, c.traj[-1]), "actions differ from the last trajectory entry"
    sw, layers = c.oracle_inputs()
    tail_teacher_forced(c, sw)
    teacher_forced_steps(c, sw, layers)


def test_free_run_end_to_end(small):
    """The GPU run from noise against the oracle's own run (no teacher
    forcing): bf16 storage drifts over steps and layers, so only the
    direction of the final actions is gated."""
    c = small
    c.reset()
    c.sampler.run()
    torch.cuda.synchronize()
    sw, layers = c.oracle_inputs()
    got = from_dev(c.actions)
    for b in range(c.B):
        r = c.rqs[b]
        ref = orc.sampler(c.noise[b], c.n_steps, sw, layers, [f64(r.k_pre[l]) for l in range(c.n_layers)],
                          [f64(r.v_pre[l]) for l in range(c.n_layers)], r.mask, r.pos0)[-1]
        g, w = got[b].ravel(), ref.ravel()
        cos = float(g @ w / (np.linalg.norm(g) * np.linalg.norm(w)))
        print(f"free run request {b}: cos={cos:.7f} max|err|={np.abs(g - w).max():.3e}", flush=True)
        assert cos >= 0.999


def test_graph_replay_matches_eager(small):
    c = small
    c.reset()
    c.sampler.run()
    torch.cuda.synchronize()
    eager = c.traj.clone()
    stream = torch.cuda.Stream()
    c.sampler.capture(stream)
    for i in range(3):
        c.reset()
        torch.cuda.synchronize()
        c.sampler.replay(stream)
        stream.synchronize()
        assert torch.equal(c.traj, eager), f"replay {i} differs from the eager run"
        torch.cuda.synchronize()
        _ = (c.x.float() * 2).sum()  # eager work between replays
    # new noise written into the same buffer: the replay follows it
    noise2 = synth.sampler_noise(synth.BASE_SEED + 7200, c.B, c.C)
    c.reset(noise2)
    c.sampler.run()
    torch.cuda.synchronize()
    eager2 = c.traj.clone()
    c.reset(noise2)
    torch.cuda.synchronize()
    c.sampler.replay(stream)
    stream.synchronize()
    assert torch.equal(c.traj, eager2)
    assert not torch.equal(eager2, eager)
    c.sampler.close()


def test_mod_table_is_bit_identical(small):
    c = small
    c.reset()
    c.sampler.run()
    torch.cuda.synchronize()
    plain = c.traj.clone()
    t = Case(2, 3, 2, 10, 576, 500, 576, 0.05, synth.BASE_SEED + 7000, mod_table=True)
    t.sampler.run()
    torch.cuda.synchronize()
    assert torch.equal(t.traj, plain)


def test_full_size_steps_teacher_forced():
    """18 layers x 10 steps, P_b=896 bucket (L in (768, 896]), chunk 50."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Case(18, 10, 1, 50, 896, 769, 896, 0.0, synth.BASE_SEED + 7300, mod_table=True)
    c.sampler.run()
    torch.cuda.synchronize()
    sw, layers = c.oracle_inputs()
    tail = tail_teacher_forced(c, sw)
    worst = teacher_forced_steps(c, sw, layers)
    print(f"worst velocity ratio over the 10 steps: {worst:.3e}; the tail alone: {tail:.3e}", flush=True)


@pytest.mark.parametrize("A", [16, 48, 128])
def test_action_dims(A):
    """The velocity kernels are instantiated per action dimension: one pass
    of 32 outputs (half idle at 16), two passes (the second half idle at 48),
    four passes at 128; the in-projection's weights are preloaded up to 32."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    c = Case(2, 3, 2, 10, 576, 500, 576, 0.05, synth.BASE_SEED + 7400 + A, A=A)
    c.sampler.run()
    torch.cuda.synchronize()
    sw, layers = c.oracle_inputs()
    tail_teacher_forced(c, sw)
    teacher_forced_steps(c, sw, layers)
    t = Case(2, 3, 2, 10, 576, 500, 576, 0.05, synth.BASE_SEED + 7400 + A, mod_table=True, A=A)
    t.sampler.run()
    torch.cuda.synchronize()
    assert torch.equal(t.traj, c.traj), "the cached table changes the run"
    for x in (t, c):
        x.sampler.close()
        x.stack.close()
