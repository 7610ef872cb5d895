"""Lazily captured graph profiles: the library's policy (host code, no GPU)
against the hand-derived cases of the pages' rule (tests/golden) and against
an independent Python model of the same rule on random call sequences, bit
for bit: bucket, action, evicted profile and the final LRU order."""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle as orc

dmx = pytest.importorskip("masked_gqa_attention_action_amd")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lazy_profiles.txt")
ACT = {"E": orc.EAGER, "C": orc.CAPTURE, "R": orc.REPLAY}


def golden_cases():
    cases = []
    for line in open(GOLDEN):
        if line.startswith("#") or not line.strip():
            continue
        cap, ev, lens, acts, evs = [f.strip() for f in line.split("|")]
        cases.append((int(cap), bool(int(ev)), [int(v) for v in lens.split(",")], [ACT[a] for a in acts.split(",")],
                      [-1 if e == "-" else int(e) for e in evs.split(",")]))
    return cases


@pytest.mark.parametrize("case", golden_cases())
def test_golden_sequences(case):
    cap, evict, lens, acts, evs = case
    keys = [dmx.lazy_bucket(n, 4096) for n in lens]
    assert keys == [orc.lazy_bucket(n, 4096) for n in lens]
    c = dmx.ProfileCache(cap, evict)
    got = [c.plan(k, 0) for k in keys]
    assert [a for a, _ in got] == acts
    assert [e for _, e in got] == evs
    model, order = orc.lazy_profile_actions([(k, 0) for k in keys], cap, evict)
    assert got == model
    assert c.keys() == order
    c.close()


def test_bucket_rule():
    for n in list(range(1, 100)) + [1023, 1024, 1025, 2047, 2048]:
        assert dmx.lazy_bucket(n, 2048) == orc.lazy_bucket(n, 2048)
    assert dmx.lazy_bucket(16, 16) == 16 and dmx.lazy_bucket(17, 32) == 32
    for bad in (0, -5, 2049):
        with pytest.raises(dmx.DmxError):
            dmx.lazy_bucket(bad, 2048)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("cap,evict", [(8, True), (3, True), (1, True), (8, False), (2, False)])
def test_random_sequences_match_model(seed, cap, evict):
    r = np.random.Generator(np.random.PCG64(900 + seed))
    n_keys = int(r.integers(2, 14))
    keys = [16 * int(v) for v in r.integers(1, 129, n_keys)]
    calls = []
    for _ in range(200):
        k = keys[int(r.integers(0, n_keys))]
        fp = int(r.integers(0, 2)) if r.random() < 0.1 else 0  # now and then other buffers
        calls.append((k, fp))
    c = dmx.ProfileCache(cap, evict)
    got = [c.plan(k, fp) for k, fp in calls]
    want, order = orc.lazy_profile_actions(calls, cap, evict)
    assert got == want
    assert c.keys() == order
    assert len(order) <= cap
    c.close()


def test_other_buffers_restart_the_profile():
    c = dmx.ProfileCache(8, True)
    assert [c.plan(512, 7)[0] for _ in range(3)] == [orc.EAGER, orc.CAPTURE, orc.REPLAY]
    assert [c.plan(512, 8)[0] for _ in range(3)] == [orc.EAGER, orc.CAPTURE, orc.REPLAY]
    c.close()


def test_cache_argument_errors():
    with pytest.raises(dmx.DmxError):
        dmx.ProfileCache(0)
    with pytest.raises(dmx.DmxError):
        dmx.ProfileCache(9)
    c = dmx.ProfileCache(2)
    with pytest.raises(dmx.DmxError):
        c.plan(-3)
    c.close()
