"""GPU: denoising runs through the lazy graph-profile cache.  Each 16-token
prefix bucket has its own fixed buffers; for every call the request's mask
(its prefix length) is written into them, and the cached run (eager, capture
or replay, as the policy decides) must give bit for bit the plain eager run's
trajectory on the same inputs."""
from __future__ import annotations

import pytest

import oracle as orc
from masked_gqa_attention_action_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import masked_gqa_attention_action_amd as dmx
    from tests.sampler_case import Case


def run_sequence(cache, cases, lengths, stream):
    base_masks = {p: c.mask.clone() for p, c in cases.items()}
    actions = []
    for n in lengths:
        p = dmx.lazy_bucket(n, 2048)
        c = cases[p]
        c.mask.copy_(base_masks[p])
        c.mask[:, n:] = 0
        c.reset()
        c.sampler.run()
        torch.cuda.synchronize()
        ref = c.traj.clone()
        c.traj.zero_()
        c.reset()
        torch.cuda.synchronize()
        actions.append(cache.run(c.sampler, stream))
        stream.synchronize()
        print(f"prefix length {n} -> bucket {p}: action {actions[-1]}", flush=True)
        assert torch.equal(c.traj, ref), f"cached run (action {actions[-1]}) differs at length {n}"
    return actions


@pytest.fixture(scope="module")
def bucket_cases():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cases = {512: Case(2, 3, 1, 10, 512, 512, 512, 0.0, synth.BASE_SEED + 7400),
             528: Case(2, 3, 1, 10, 528, 528, 528, 0.0, synth.BASE_SEED + 7500)}
    yield cases
    for c in cases.values():
        c.sampler.close()
        c.stack.close()
    torch.cuda.synchronize()


def test_profiles_eager_capture_replay(bucket_cases):
    lengths = [500, 505, 520, 510, 525, 515, 498]
    keys = [orc.lazy_bucket(n, 2048) for n in lengths]
    want, _ = orc.lazy_profile_actions([(k, 0) for k in keys], 8, True)
    cache = dmx.ProfileCache(8, True)
    stream = torch.cuda.Stream()
    got = run_sequence(cache, bucket_cases, lengths, stream)
    assert got == [a for a, _ in want]
    assert got == [orc.EAGER, orc.CAPTURE, orc.EAGER, orc.REPLAY, orc.CAPTURE, orc.REPLAY, orc.REPLAY]
    assert len(cache.keys()) == 2
    cache.close()


def test_profiles_eviction_keeps_results(bucket_cases):
    """One profile slot and alternating buckets: every call evicts the other
    bucket's profile and runs eager; a bucket called twice in a row captures."""
    cache = dmx.ProfileCache(1, True)
    stream = torch.cuda.Stream()
    got = run_sequence(cache, bucket_cases, [500, 520, 500, 520, 520, 520], stream)
    assert got == [orc.EAGER, orc.EAGER, orc.EAGER, orc.EAGER, orc.CAPTURE, orc.REPLAY]
    cache.close()
