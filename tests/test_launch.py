"""Host logic of the prefill launch policies (workloads.launch): timelines on hand-made
arrival times and step durations, checked against the policies' definitions."""
import numpy as np
import pytest

from workloads.launch import run_policy, summarize, wave_arrivals

SIZES = [40, 30, 20, 10]


def linear_ms(waves):  # a step's duration: 1 ms fixed cost + 0.1 ms per pair
    return 1.0 + 0.1 * sum(SIZES[w] for w in waves)


def test_arrivals_are_seeded_and_start_at_zero():
    a = wave_arrivals(7, 4, 0.5)
    assert a[0] == 0.0 and np.all(np.diff(a) >= 0) and len(a) == 4
    assert np.array_equal(a, wave_arrivals(7, 4, 0.5))
    assert np.array_equal(wave_arrivals(7, 4, 0.0), np.zeros(4))


def test_early_runs_each_wave_alone_in_arrival_order():
    arr = np.array([0.0, 1.0, 2.0, 30.0])
    tl = run_policy("early", arr, SIZES, linear_ms)
    assert [l.waves for l in tl.launches] == [(0,), (1,), (2,), (3,)]
    # wave 0: 0..5; wave 1 waits for the GPU: 5..9; wave 2: 9..12; wave 3 arrives at 30: 30..32
    assert [(l.start_ms, l.end_ms) for l in tl.launches] == [(0.0, 5.0), (5.0, 9.0), (9.0, 12.0), (30.0, 32.0)]
    s = summarize(tl, arr, SIZES)
    lat = np.array([5.0, 8.0, 10.0, 2.0])
    assert s["token_latency_ms"]["mean"] == pytest.approx(float(np.repeat(lat, SIZES).mean()))
    assert s["makespan_ms"] == 32.0 and s["gpu_busy_ms"] == 14.0


def test_all_waits_for_the_last_wave():
    arr = np.array([0.0, 1.0, 2.0, 3.0])
    tl = run_policy("all", arr, SIZES, linear_ms)
    assert len(tl.launches) == 1 and tl.launches[0].waves == (0, 1, 2, 3)
    assert tl.launches[0].start_ms == 3.0 and tl.launches[0].end_ms == 3.0 + 11.0


def test_minbatch_takes_everything_waiting_once_the_threshold_is_met():
    arr = np.array([0.0, 1.0, 2.0, 3.0])
    # threshold 60: wave 0 alone (40) waits; at t=1 waves 0+1 (70) launch; 2 and 3 arrive while
    # the GPU is busy (1..9) and go together once it is free (last wave in: no more to wait for)
    tl = run_policy("minbatch", arr, SIZES, linear_ms, min_batch=60)
    assert [l.waves for l in tl.launches] == [(0, 1), (2, 3)]
    assert [(l.start_ms, l.end_ms) for l in tl.launches] == [(1.0, 9.0), (9.0, 13.0)]


def test_minbatch_limits_reduce_to_the_other_policies():
    rng = np.random.default_rng(3)
    for _ in range(20):
        arr = np.sort(rng.exponential(2.0, 4))
        arr[0] = 0.0
        big = run_policy("minbatch", arr, SIZES, linear_ms, min_batch=10 ** 9)
        alls = run_policy("all", arr, SIZES, linear_ms)
        assert [(l.waves, l.start_ms, l.end_ms) for l in big.launches] == \
               [(l.waves, l.start_ms, l.end_ms) for l in alls.launches]
        zero = run_policy("minbatch", arr, SIZES, linear_ms, min_batch=0)
        # threshold 0: whatever is waiting launches as soon as the GPU is free
        for l in zero.launches:
            assert all(arr[w] <= l.start_ms for w in l.waves)
        seen = sorted(w for l in zero.launches for w in l.waves)
        assert seen == [0, 1, 2, 3]


def test_every_policy_carries_every_wave_once_and_never_before_it_arrives():
    rng = np.random.default_rng(11)
    for policy in ("early", "all", "minbatch"):
        for _ in range(30):
            arr = np.concatenate([[0.0], np.cumsum(rng.exponential(3.0, 3))])
            tl = run_policy(policy, arr, SIZES, linear_ms, min_batch=int(rng.integers(0, 120)))
            seen = sorted(w for l in tl.launches for w in l.waves)
            assert seen == [0, 1, 2, 3]
            prev_end = 0.0
            for l in tl.launches:
                assert l.start_ms >= prev_end - 1e-12  # one step at a time
                assert all(arr[w] <= l.start_ms + 1e-12 for w in l.waves)
                prev_end = l.end_ms
