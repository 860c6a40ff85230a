"""The library's batching scheduler over the block pool (sched_simulate, host C++) against
the oracle's step-by-step definition (oracle/batching.py): every integer result equal (steps,
per-request latency and service, busy and padding places, peak blocks, deferrals, stalls)
and the mean utilisation equal to the last bit (same sums in the same order).
"""
import numpy as np
import pytest

from oracle import batching as Bt

kvp = pytest.importorskip("kv_cache_decode_paged_amd")


def _both(prompts, outs, slots, policy, alloc, max_seq=2048, bs=16, blocks=1 << 20):
    res, lat, svc = kvp.sched_simulate(prompts, outs, slots, policy, alloc, max_seq, bs, blocks)
    want = Bt.simulate(list(prompts), list(outs), slots, policy, alloc, max_seq, bs, blocks)
    return res, lat.tolist(), svc.tolist(), want


def _same(res, lat, svc, want):
    assert lat == want["latency"]
    assert svc == want["service"]
    for f in ("steps", "tokens", "busy_slot_steps", "padding_slot_steps", "peak_blocks", "deferrals", "stalls",
              "max_latency"):
        assert getattr(res, f) == want[f], f
    for f in ("mean_latency", "mean_service", "mean_utilisation"):
        assert getattr(res, f) == want[f], f


def test_hand_worked_schedules():
    for pol in (kvp.SCHED_CONTINUOUS, kvp.SCHED_STATIC):
        _same(*_both([0] * 4, [3, 1, 1, 1], 2, pol, kvp.ALLOC_PAGED))


@pytest.mark.parametrize("seed", range(12))
def test_random_schedules_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 120))
    slots = int(rng.integers(1, 33))
    bs = int(rng.choice([1, 4, 16, 32]))
    outs = [int(x) for x in rng.integers(1, 300, size=n)]
    prompts = [int(x) for x in rng.integers(0, 200, size=n)]
    for pol in (kvp.SCHED_CONTINUOUS, kvp.SCHED_STATIC):
        _same(*_both(prompts, outs, slots, pol, kvp.ALLOC_PAGED, bs=bs))
        _same(*_both(prompts, outs, slots, pol, kvp.ALLOC_NAIVE, max_seq=512, bs=bs))


@pytest.mark.parametrize("seed", range(6))
def test_small_pools_defer_and_stall_alike(seed):
    rng = np.random.default_rng(100 + seed)
    n = 40
    outs = [int(x) for x in rng.integers(1, 100, size=n)]
    prompts = [int(x) for x in rng.integers(0, 60, size=n)]
    for pol in (kvp.SCHED_CONTINUOUS, kvp.SCHED_STATIC):
        for blocks in (60, 90, 200):
            try:
                want = Bt.simulate(prompts, outs, 8, pol, Bt.PAGED, 2048, 16, blocks)
            except RuntimeError:
                with pytest.raises(kvp.KvpError):
                    kvp.sched_simulate(prompts, outs, 8, pol, kvp.ALLOC_PAGED, 2048, 16, blocks)
                continue
            res, lat, svc = kvp.sched_simulate(prompts, outs, 8, pol, kvp.ALLOC_PAGED, 2048, 16, blocks)
            _same(res, lat.tolist(), svc.tolist(), want)


def test_pool_too_small_is_an_error():
    with pytest.raises(kvp.KvpError):
        kvp.sched_simulate([16, 16, 16], [1, 1, 1], 3, kvp.SCHED_CONTINUOUS, kvp.ALLOC_PAGED, 2048, 16, 2)


def test_bad_arguments_are_refused():
    for bad in (dict(slots=0), dict(policy=5), dict(alloc=7), dict(block_size=0), dict(num_blocks=0)):
        kw = dict(slots=2, policy=kvp.SCHED_CONTINUOUS, alloc=kvp.ALLOC_PAGED, max_seq_len=64, block_size=16,
                  num_blocks=64)
        kw.update(bad)
        with pytest.raises(kvp.KvpError):
            kvp.sched_simulate([0], [1], **kw)
    with pytest.raises(kvp.KvpError):  # naive reservation shorter than the request
        kvp.sched_simulate([60], [10], 1, kvp.SCHED_CONTINUOUS, kvp.ALLOC_NAIVE, 64, 16, 64)
    with pytest.raises(kvp.KvpError):  # an empty output
        kvp.sched_simulate([0], [0], 1)
    res, lat, svc = kvp.sched_simulate([], [], 4)
    assert res.steps == 0 and lat.numel() == 0


def test_section4_utilisation_through_the_scheduler():
    # 200 requests of the SECTION 4 recipe, all admitted at once: the paged schedule's
    # utilisation at the last step (every request complete and resident) is the paged
    # utilisation of the page, the naive one 500 / 2048-like
    t = Bt.response_lengths(200, seed=7)
    outs = [int(x) for x in t]
    res_p, _, _ = kvp.sched_simulate([0] * 200, outs, 200, kvp.SCHED_STATIC, kvp.ALLOC_PAGED, 2048, 16)
    res_n, _, _ = kvp.sched_simulate([0] * 200, outs, 200, kvp.SCHED_STATIC, kvp.ALLOC_NAIVE, 2048, 16)
    assert res_p.peak_blocks == int(np.sum(-(-t // 16)))
    assert res_n.peak_blocks == 200 * 128
    assert res_p.mean_utilisation > 0.9 and res_n.mean_utilisation < 0.2
