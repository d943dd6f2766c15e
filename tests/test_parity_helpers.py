"""CPU checks of the parity-protocol helpers in tests/parity.py (no GPU)."""
import numpy as np

import oracle
from means_token_clustering_amd import inputs as gen
from tests import parity


def test_exact_distances_brute_force():
    rng = np.random.default_rng(0)
    Q = rng.standard_normal((2, 3, 5, 4))
    mu = rng.standard_normal((2, 3, 2, 4))
    D = parity.exact_distances(Q, mu)
    for s in np.ndindex(2, 3):
        for i in range(5):
            for k in range(2):
                want = sum((Q[s][i][t] - mu[s][k][t]) ** 2 for t in range(4))
                assert abs(D[s][i][k] - want) <= 1e-12 * max(1.0, want)


def test_distance_error_of_exact_scores_and_a_planted_error():
    rng = np.random.default_rng(1)
    Q = rng.standard_normal((1, 2, 6, 8))
    mu = rng.standard_normal((1, 2, 3, 8))
    scores = np.einsum("...ld,...kd->...lk", Q, mu) - 0.5 * np.einsum("...kd,...kd->...k", mu, mu)[..., None, :]
    assert parity.distance_error(Q, mu, scores) < 1e-13
    qn2 = float(Q[0, 1, 4] @ Q[0, 1, 4])
    bad = scores.copy()
    bad[0, 1, 4, 2] += 1e-3 * qn2   # D moves by 2e-3 ||q||^2
    assert abs(parity.distance_error(Q, mu, bad) - 2e-3) < 1e-9


def test_free_running_count():
    x = gen.make_inputs(1, 2, 40, 8, nclust=5, iters=3, seed=3, blobs=4)
    q, k, v = x.values("q"), x.values("k"), x.values("v")
    ref = oracle.forward(q, k, v, 5, 3, 8, 0.5, trace=False)["assign"]
    assert parity.free_running_mismatches(q, k, v, 5, 3, 8, 0.5, ref) == 0
    flipped = ref.copy()
    flipped[0, 1, 7] = (flipped[0, 1, 7] + 1) % 5
    assert parity.free_running_mismatches(q, k, v, 5, 3, 8, 0.5, flipped) == 1
