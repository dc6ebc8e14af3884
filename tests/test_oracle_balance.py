"""Pins of the bias-update oracle (oracle/balance_ref.py), CPU only.

The rule is a stated reading (the pages leave it undescribed), so the pins
fix what that reading implies: a hand-worked step, the fp32 arithmetic, the
integer decision at the mean, the invariants of a sign rule, and the
closed-loop behaviour it exists for -- repeated steps through the router
oracle bring a strongly imbalanced router back to balance, which a flipped
sign or a bias that the choice ignores would not.  A small mutation pass
checks that these pins catch plausible mistakes.
"""
import numpy as np
import pytest

from oracle import balance_ref as B
from oracle import moe_ref as R


def test_hand_worked_step():
    # E = 4, k = 2: picks 0,1 | 0,2 | 0,3 | 2,0 -> loads 4, 1, 2, 1; mean 2
    ids = np.array([[0, 1], [0, 2], [0, 3], [2, 0]], dtype=np.int32)
    c = B.expert_load(ids, 4)
    assert c.tolist() == [4, 1, 2, 1]
    assert B.load_direction(c).tolist() == [-1, 1, 0, 1]
    b = np.array([0.5, -0.25, 0.0, 1.0], dtype=np.float32)
    nb = B.bias_update(b, c, 0.125)
    assert nb.dtype == np.float32
    assert nb.tolist() == [0.375, -0.125, 0.0, 1.125]


def test_ids_outside_the_layer_are_not_counted():
    ids = np.array([[0, -1], [3, 4], [2, 1 << 20]], dtype=np.int32)
    assert B.expert_load(ids, 4).tolist() == [1, 0, 1, 1]
    assert B.expert_load(np.zeros((0, 8), np.int32), 6).tolist() == [0] * 6


def test_update_is_one_fp32_addition():
    # 1 + 2^-30 is not an fp32 number: the bias stays 1; 2^-30 - 2^-30 is exact
    c = np.array([0, 2], dtype=np.int64)            # expert 0 under, 1 over
    nb = B.bias_update(np.array([1.0, 2.0 ** -30], np.float32), c, 2.0 ** -30)
    assert nb[0] == np.float32(1.0)
    assert nb[1] == np.float32(0.0)
    # halfway cases round to even: 1 + 2^-24 -> 1, (1 + 2^-23) + 2^-24 -> 1 + 2^-22;
    # 1 - 2^-24 is exact (fp32 numbers below 1 are 2^-24 apart)
    nb = B.bias_update(np.array([1.0, 1.0 + 2.0 ** -23, 1.0], np.float32), np.array([0, 0, 3]),
                       2.0 ** -24)
    assert nb.tolist() == [1.0, 1.0 + 2.0 ** -22, 1.0 - 2.0 ** -24]


def test_decision_at_the_mean_is_exact():
    # loads whose mean is a non-terminating binary fraction: 3 experts, total 10,
    # mean 3.333...; and an expert exactly at an integer mean keeps its bias
    c = np.array([3, 3, 4], dtype=np.int64)
    assert B.load_direction(c).tolist() == [1, 1, -1]
    c = np.array([5, 5, 5, 5, 7, 3], dtype=np.int64)
    assert B.load_direction(c).tolist() == [0, 0, 0, 0, -1, 1]
    # large loads that fp32 cannot hold apart: 2^25 + 1, 2^25 - 1 and 2^25
    # all round to 2^25 in fp32, but their directions are -1, +1 and 0
    c = np.array([(1 << 25) + 1, (1 << 25) - 1, 1 << 25], dtype=np.int64)
    assert B.load_direction(c).tolist() == [-1, 1, 0]
    assert B.bias_update(np.zeros(3, np.float32), c, 1.0).tolist() == [-1.0, 1.0, 0.0]


@pytest.mark.parametrize("seed", range(4))
def test_sign_rule_invariants(seed):
    rng = np.random.default_rng(seed)
    E = 64
    c = rng.integers(0, 50, E)
    d = B.load_direction(c)
    # balanced loads change nothing
    assert not B.load_direction(np.full(E, 17)).any()
    # the ordering of loads is reversed by the direction (monotone, non-increasing)
    order = np.argsort(c, kind="stable")
    assert np.all(np.diff(d[order]) <= 0)
    # reflecting the loads about their mean reverses every direction
    assert np.array_equal(B.load_direction(2 * c.max() - c), -B.load_direction(c) * 1)
    # scaling all loads keeps the directions
    assert np.array_equal(B.load_direction(3 * c), d)
    # sum of the bias changes is speed * (#under - #over)
    b = rng.standard_normal(E).astype(np.float32) * np.float32(1e-3)
    u = 2.0 ** -10
    nb = B.bias_update(b, c, u)
    delta = (nb.astype(np.float64) - b.astype(np.float64)) / u
    assert np.allclose(delta, d, atol=1e-3)


def _imbalance_loop(update, steps=300, seed=0):
    """Route fresh tokens through the router oracle with a strong per-expert
    affinity, updating the bias after each step; loads' max / mean before and
    after."""
    rng = np.random.default_rng(seed)
    T, d, E, k = 1024, 16, 16, 2
    w = rng.standard_normal((E, d)).astype(np.float32) * np.float32(0.3)
    w[:, 0] = np.linspace(-2.5, 2.5, E, dtype=np.float32)    # affinity through a constant feature
    bias = np.zeros(E, dtype=np.float32)
    ratios = []
    for _ in range(steps):
        h = rng.standard_normal((T, d)).astype(np.float32)
        h[:, 0] = 1.0
        ids = R.route(h, w, bias, k, 1.0, True)["ids"]
        c = B.expert_load(ids, E)
        ratios.append(c.max() / c.mean())
        bias = update(bias, c, 2.0 ** -7)
    return ratios[0], float(np.mean(ratios[-20:]))


def test_repeated_updates_balance_an_imbalanced_router():
    first, last = _imbalance_loop(B.bias_update)
    assert first > 3.0, first
    assert last < 1.3, last


# ------------------------------------------------------------ mutation pass
def _flipped(bias, counts, speed):
    return (np.asarray(bias, np.float32)
            - np.float32(speed) * B.load_direction(counts).astype(np.float32)).astype(np.float32)


def _float_mean_f32(bias, counts, speed):
    c = np.asarray(counts)
    m = np.float32(c.sum()) / np.float32(c.size)
    dirn = np.sign(m - c.astype(np.float32))
    return (np.asarray(bias, np.float32) + np.float32(speed) * dirn.astype(np.float32)).astype(np.float32)


def _proportional(bias, counts, speed):
    c = np.asarray(counts, np.float64)
    return (np.asarray(bias, np.float32)
            + np.float32(speed) * ((c.mean() - c) / max(c.mean(), 1.0)).astype(np.float32)).astype(np.float32)


def _fp64_update(bias, counts, speed):
    return (np.asarray(bias, np.float64) + speed * B.load_direction(counts)).astype(np.float64)


def _count_all_ids(ids, n_experts):
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    return np.bincount(np.clip(flat, 0, n_experts - 1), minlength=n_experts)


MUTATIONS = {
    "sign flipped": ("bias_update", _flipped),
    "direction from an fp32 mean": ("bias_update", _float_mean_f32),
    "proportional step": ("bias_update", _proportional),
    "fp64 bias": ("bias_update", _fp64_update),
    "out-of-range ids clamped into the layer": ("expert_load", _count_all_ids),
}

PINS = [test_hand_worked_step, test_ids_outside_the_layer_are_not_counted,
        test_update_is_one_fp32_addition, test_decision_at_the_mean_is_exact,
        lambda: [test_sign_rule_invariants(s) for s in range(4)],
        test_repeated_updates_balance_an_imbalanced_router]


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(B, attr, fn)
    failed = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed > 0, f"no pin caught: {name}"
