"""Pins of the batching / utilisation model of the oracle (oracle/batching.py): hand-worked
schedules, closed forms of the two policies, the pages' utilisation figures (naive 1024 MB
reserved against 250 MB used = 24.4 %, 75 GB idle at 100 users, paged about 98.5 %), the
batching passage's direction (continuous beats static on throughput and by far on mean
latency for skewed lengths), and planted mutants.
"""
import math

import numpy as np
import pytest

from oracle import batching as Bt

BIG = 1 << 20


def _sim(out, slots, policy, alloc=Bt.PAGED, prompts=None, max_seq=4096, bs=16, blocks=BIG):
    prompts = [0] * len(out) if prompts is None else prompts
    return Bt.simulate(prompts, out, slots, policy, alloc, max_seq, bs, blocks)


def test_hand_worked_schedules():
    # two places, outputs 3, 1, 1, 1
    c = _sim([3, 1, 1, 1], 2, Bt.CONTINUOUS)
    assert c["steps"] == 3 and c["latency"] == [3, 1, 2, 3] and c["padding_slot_steps"] == 0
    assert c["service"] == [3, 1, 1, 1]
    s = _sim([3, 1, 1, 1], 2, Bt.STATIC)
    assert s["steps"] == 4 and s["latency"] == [3, 3, 4, 4] and s["padding_slot_steps"] == 2
    assert c["busy_slot_steps"] == s["busy_slot_steps"] == 6


@pytest.mark.parametrize("n,slots,L", [(10, 3, 5), (8, 8, 7), (1, 4, 2), (17, 4, 1)])
def test_equal_lengths_policies_coincide(n, slots, L):
    for pol in (Bt.STATIC, Bt.CONTINUOUS):
        r = _sim([L] * n, slots, pol)
        assert r["steps"] == math.ceil(n / slots) * L
        assert r["latency"] == [L * (1 + i // slots) for i in range(n)]
        assert r["padding_slot_steps"] == 0


def test_static_closed_form():
    rng = np.random.default_rng(3)
    out = [int(x) for x in rng.integers(1, 40, size=37)]
    slots = 6
    r = _sim(out, slots, Bt.STATIC)
    batches = [out[i:i + slots] for i in range(0, len(out), slots)]
    assert r["steps"] == sum(max(b) for b in batches)
    assert r["busy_slot_steps"] == sum(out)
    assert r["padding_slot_steps"] == sum(max(b) - x for b in batches for x in b)
    ends = np.cumsum([max(b) for b in batches])
    assert r["latency"] == [int(ends[i // slots]) for i in range(len(out))]


def test_continuous_limits():
    out = [5, 9, 2, 7, 1]
    wide = _sim(out, 8, Bt.CONTINUOUS)
    assert wide["steps"] == max(out) and wide["latency"] == out
    one = _sim(out, 1, Bt.CONTINUOUS)
    assert one["steps"] == sum(out) and one["latency"] == list(np.cumsum(out))


def test_paged_pages_and_utilisation_by_hand():
    # one request, 17 tokens, pages of 16: 1 page for tokens 1..16, 2 pages at 17
    r = _sim([17], 1, Bt.CONTINUOUS)
    assert r["peak_blocks"] == 2
    want = (sum(t / 16 for t in range(1, 17)) + 17 / 32) / 17
    assert abs(r["mean_utilisation"] - want) < 1e-15
    # naive reservation of max_seq = 64 tokens (4 pages) from the start
    r = _sim([17], 1, Bt.CONTINUOUS, alloc=Bt.NAIVE, max_seq=64)
    assert r["peak_blocks"] == 4
    assert abs(r["mean_utilisation"] - sum(t / 64 for t in range(1, 18)) / 17) < 1e-15


def test_full_pool_defers_and_stalls():
    # 3 pages: two requests with 16-token prompts take 2 pages; their 17th tokens need one
    # page each, so one of them stalls until the other is returned
    r = _sim([2, 2], 2, Bt.CONTINUOUS, prompts=[16, 16], blocks=3)
    assert r["stalls"] >= 1 and r["peak_blocks"] == 3
    # a third request waits for pages at admission
    r = _sim([1, 1, 1], 3, Bt.CONTINUOUS, prompts=[15, 15, 15], blocks=2)
    assert r["deferrals"] >= 1 and r["latency"] == [1, 1, 2] and r["service"] == [1, 1, 1]
    # both admitted requests need a page and none is left: no schedule exists
    with pytest.raises(RuntimeError):
        _sim([1, 1, 1], 3, Bt.CONTINUOUS, prompts=[16, 16, 16], blocks=2)


def test_page_figures():
    # 32 layers, 32 heads of 128, fp16: 524,288 bytes = 0.5 MB per token
    mb = 2 * 32 * 32 * 128 * 2 / 1024 / 1024
    assert mb == 0.5
    pre, used = 2048 * mb, 500 * mb
    assert (pre, used) == (1024.0, 250.0)
    assert round(used / pre * 100, 1) == 24.4
    assert round((pre - used) * 100 / 1024, 2) == 75.59
    assert abs(Bt.naive_utilisation([500] * 100, 2048) - 24.4140625) < 1e-12


@pytest.mark.parametrize("n", [10, 25, 50, 100, 200])
def test_section4_sweep(n):
    t = Bt.response_lengths(n, seed=n)
    nu, pu = Bt.naive_utilisation(t, 2048), Bt.paged_utilisation(t, 16)
    assert 18.0 < nu < 30.0
    assert 97.5 < pu < 99.5
    if n >= 100:
        assert abs(nu - 24.4) < 2.0 and abs(pu - 98.5) < 0.6


def skewed_lengths():
    """64 output lengths with the batching passage's summary: median 18, maximum 231, total
    1874 (a synthetic stand-in: the page gives only these statistics)."""
    from statistics import NormalDist
    q = (np.arange(64) + 0.5) / 64
    z = np.array([NormalDist().inv_cdf(x) for x in q])
    x = np.exp(math.log(18) + 1.05 * z)
    x = np.maximum(1, np.round(x)).astype(int)
    x[-1] = 231
    # bring the total to 1874 by adjusting the values above the median (keeps the median)
    rest = 1874 - x.sum()
    i = 62
    while rest != 0:
        step = 1 if rest > 0 else -1
        if x[i] + step > x[i - 1] and x[i] + step < 231:
            x[i] += step
            rest -= step
        i = 62 if i <= 33 else i - 1
    rng = np.random.default_rng(64)
    return [int(v) for v in rng.permutation(x)]


def test_batching_passage_direction():
    out = skewed_lengths()
    assert sorted(out)[31] <= 18 <= sorted(out)[32] and max(out) == 231 and sum(out) == 1874
    s = _sim(out, 8, Bt.STATIC)
    c = _sim(out, 8, Bt.CONTINUOUS)
    thr = s["steps"] / c["steps"]          # same work, constant cost per step
    svc = s["mean_service"] / c["mean_service"]
    assert c["service"] == out             # continuous: each request is served in its own length
    assert 1.2 < thr < 2.5                 # the page: 1.6x
    assert svc > 3.0                       # the page: more than ten times
    assert s["mean_latency"] > c["mean_latency"]


# ---- planted mutants ----
def _mut_static_as_continuous(out, slots, policy, **kw):
    return _sim(out, slots, Bt.CONTINUOUS, **kw)


def _mut_latency_from_zero(out, slots, policy, **kw):
    r = _sim(out, slots, policy, **kw)
    r["latency"] = [x - 1 for x in r["latency"]]
    return r


def _mut_no_padding(out, slots, policy, **kw):
    r = _sim(out, slots, policy, **kw)
    r["padding_slot_steps"] = 0
    return r


@pytest.mark.parametrize("mut", [_mut_static_as_continuous, _mut_latency_from_zero, _mut_no_padding])
def test_mutants_fail_the_hand_schedule(mut):
    s = mut([3, 1, 1, 1], 2, Bt.STATIC)
    assert not (s["steps"] == 4 and s["latency"] == [3, 3, 4, 4] and s["padding_slot_steps"] == 2)
