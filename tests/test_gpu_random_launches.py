"""Seeded random launches on MI355X against the oracle: 1-3 requests of
log-uniform length (1 .. 40,000 keys, so short rows, one page, partial pages
and multi-chunk rows all occur), 1-6 rows per request at random bounds inside
the request (not only verify rows), the rows of the requests interleaved in
a random order, a random top-k (1 .. 2,048), optional duplicated keys (ties)
and randomly relabelled pages.  Every case: scores within the tolerance of
the fp64 oracle, nothing written at or past a row's bound, the selection
bit-exact against the oracle's top-k of the GPU's own scores (ties to the
lower index, ascending, -1 padded), and overlap with the oracle's own
selection of at least 99.9 %."""
import math

import numpy as np
import pytest

import synthetic as syn
from gpu_util import (OVERLAP_MIN, check_scores_full, check_topk_exact, check_untouched_past_bound,
                      oracle_rows, overlap, run_launch, say)

pytestmark = pytest.mark.gpu

N_CASES = 64


def random_problem(seed: int) -> syn.Problem:
    rng = np.random.default_rng(90_000 + seed)
    n_req = int(rng.integers(1, 4))
    lens = [int(round(math.exp(rng.uniform(0.0, math.log(40_000))))) for _ in range(n_req)]
    rows = []
    for i, n in enumerate(lens):
        for _ in range(int(rng.integers(1, 7))):
            rows.append((i, int(rng.integers(0, n + 1)) if rng.random() < 0.5 else n - int(rng.integers(0, 4))))
    rows = [(i, max(0, b)) for i, b in rows]
    order = rng.permutation(len(rows))
    rows = [rows[j] for j in order]
    topk = int(rng.choice([1, 7, 100, 2048, int(rng.integers(1, 2049))]))
    dup = float(rng.choice([0.0, 0.02]))
    return syn.build_problem(f"random_{seed}", 91_000 + seed, lens, rows, topk=topk, dup_frac=dup)


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_launch(seed):
    p = random_problem(seed)
    say(f"[gpu] random launch {seed}: rows {p.rows}, bounds {p.row_bound.tolist()}, "
        f"page-table rows {p.row_pt.tolist()}, topk {p.topk}")
    if p.max_bound == 0:
        pytest.skip("every row empty (covered by test_every_row_empty)")
    scores, out = run_launch(p)
    check_untouched_past_bound(p, scores)
    live = [r for r in range(p.rows) if p.row_bound[r] > 0]
    ref = oracle_rows(p, live)
    check_scores_full(p, scores, ref, rows=live)
    check_topk_exact(p, scores, out)
    assert overlap(p, ref, out, rows=live) >= OVERLAP_MIN
