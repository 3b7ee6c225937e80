"""The comparison rules of tests/parity.py on the CPU (no GPU).

A rule that accepts anything proves nothing: each drift rule must accept the
oracle's own runs and reject logs with a planted mistake (a sub-optimal swap, a
stop although a swap lowers J, a swap log that does not lead to the final set).
"""
import numpy as np
import pytest

import oracle
import parity
from test_oracle_drift import layout, rand_kv

ROUNDS = 6


def _row(seed, force):
    lay = layout(frames=3, frame_len=8, frame_valid=6, block=2, D=4, scale=0.9)
    k, v = rand_kv(lay, 50 + seed)
    qbar = np.random.default_rng(60 + seed).standard_normal(4) * 1.5
    chat, z, Z = oracle.drift_row(qbar, k, v, lay)
    return chat, z / Z, oracle.forced_blocks(lay, force)


def _run(objective, chat, zhat, kb, forced):
    if objective == oracle.RENORM:
        return oracle.restore_row_renorm(chat, zhat, kb, ROUNDS, forced)
    return oracle.restore_row(chat, kb, ROUNDS, forced)


def _log(swaps):
    log = np.full((ROUNDS, 2), -1, dtype=np.int64)
    for r, (a, b) in enumerate(swaps):
        log[r] = (a, b)
    return log


def _check(objective, kept, log, chat, zhat, kb, forced):
    z = zhat if objective == oracle.RENORM else None
    return parity.drift_valid(kept, log, chat, kb, forced, zhat=z)


def _swapping_row(objective, force):
    for seed in range(40):
        chat, zhat, forced = _row(seed, force)
        kept, j, swaps = _run(objective, chat, zhat, 5, forced)
        if swaps:
            return chat, zhat, forced, kept, j, swaps
    pytest.fail("no seed swaps")


@pytest.mark.parametrize("objective", [oracle.RAW, oracle.RENORM])
@pytest.mark.parametrize("force", [False, True])
def test_oracle_runs_pass(objective, force):
    for seed in range(6):
        chat, zhat, forced = _row(seed, force)
        kept, j, swaps = _run(objective, chat, zhat, 5, forced)
        ok, why, jrep = _check(objective, kept, _log(swaps), chat, zhat, 5, forced)
        assert ok, why
        assert jrep == pytest.approx(j, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("objective", [oracle.RAW, oracle.RENORM])
def test_suboptimal_swap_rejected(objective):
    chat, zhat, forced, kept, j, swaps = _swapping_row(objective, False)
    d = np.sqrt((chat * chat).sum(axis=1))
    init = set(oracle.priority_order(d, forced)[:5])
    nb = chat.shape[0]
    a0, b0 = swaps[0]
    # the worst first swap instead of the best one, then stop
    worst, pair = -1.0, None
    for a in sorted(set(range(nb)) - init):
        for b in sorted(init):
            s = (init - {b}) | {a}
            jj = (oracle.drift_j_renorm(chat, zhat, sorted(s)) if objective == oracle.RENORM
                  else oracle.drift_j(chat, sorted(s)))
            if jj > worst:
                worst, pair = jj, (a, b)
    assert pair != (a0, b0)
    final = sorted((init - {pair[1]}) | {pair[0]})
    ok, why, _ = _check(objective, final, _log([pair]), chat, zhat, 5, forced)
    assert not ok and ("not optimal" in why or "raises" in why), why


@pytest.mark.parametrize("objective", [oracle.RAW, oracle.RENORM])
def test_early_stop_rejected(objective):
    chat, zhat, forced, kept, j, swaps = _swapping_row(objective, False)
    d = np.sqrt((chat * chat).sum(axis=1))
    init = sorted(oracle.priority_order(d, forced)[:5])
    ok, why, _ = _check(objective, init, _log([]), chat, zhat, 5, forced)
    assert not ok and "stopped" in why, why


@pytest.mark.parametrize("objective", [oracle.RAW, oracle.RENORM])
def test_log_inconsistent_with_final_set_rejected(objective):
    chat, zhat, forced, kept, j, swaps = _swapping_row(objective, False)
    wrong = sorted(set(kept) ^ {swaps[0][0], swaps[0][1]})   # undo the first swap only
    ok, why, _ = _check(objective, wrong, _log(swaps), chat, zhat, 5, forced)
    assert not ok


def test_objectives_disagree_somewhere():
    """The two rules are not the same rule: some row's renormalised run is not a
    valid dropped-sum run."""
    for seed in range(40):
        chat, zhat, forced = _row(seed, False)
        kept, j, swaps = oracle.restore_row_renorm(chat, zhat, 5, ROUNDS, forced)
        ok, _, _ = parity.drift_valid(kept, _log(swaps), chat, 5, forced)
        if not ok:
            return
    pytest.fail("renormalised runs all pass the dropped-sum rule")


def test_rerank_rule_accepts_the_oracle_and_rejects_planted_mistakes():
    rng = np.random.default_rng(44)
    chat = rng.standard_normal((9, 3))
    k = 4
    for tb in (True, False):
        kept, j, sets, js = oracle.rerank_row(chat, k, 5, (), track_best=tb)
        ok, why = parity.rerank_valid(sets, kept, chat, k, (), tb)
        assert ok, why
    kept, j, sets, js = oracle.rerank_row(chat, k, 5, (), track_best=True)
    # a round whose set is not its top-k: swap one kept block for a dropped one
    bad = [list(s) for s in sets]
    drop = [x for x in range(9) if x not in bad[2]]
    bad[2] = sorted(bad[2][1:] + [drop[0]])
    ok, _ = parity.rerank_valid(bad, bad[-1], chat, k, (), False)
    assert not ok
    # track-best returning the last set when an earlier one is better
    worst = max(range(len(sets)), key=lambda x: js[x])
    if js[worst] > min(js) * (1 + 1e-3):
        ok, _ = parity.rerank_valid(sets, sets[worst], chat, k, (), True)
        assert not ok
    # the planted row of the oracle pins: J rises, track-best keeps round 1
    from test_oracle_drift import PLANTED_RERANK
    kept, j, sets, js = oracle.rerank_row(PLANTED_RERANK, 2, 3, track_best=True)
    assert parity.rerank_valid(sets, kept, PLANTED_RERANK, 2, (), True)[0]
    assert not parity.rerank_valid(sets, sets[-1], PLANTED_RERANK, 2, (), True)[0]
    words = [sum(1 << j for j in s) for s in sets]
    assert [parity.mask_words_to_set([w], 4) for w in words] == sets
