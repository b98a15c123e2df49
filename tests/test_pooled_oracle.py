"""Pins of the oracle's pooled selection (doc of the prefill row-group selector,
glm5next_dsa/layer.rs source page): candidacy, total order, expansion and the
per-row tail base. CPU only."""
import numpy as np
import pytest

import oracle


def dominance_ok(scores, pools, pvis):
    """Every selected visible pool comes before every unselected one under
    (score descending, pool ascending)."""
    sel = set(int(p) for p in pools)
    for p in sel:
        for q in range(pvis):
            if q in sel:
                continue
            if not (scores[p] > scores[q] or (scores[p] == scores[q] and p < q)):
                return False
    return True


@pytest.mark.parametrize("select_k", [1, 3, 8, 40])
def test_one_token_pools_are_the_per_token_selection(select_k):
    rng = np.random.default_rng(7)
    scores = rng.standard_normal((6, 50))
    lens = np.array([50, 1, 7, 23, 49, 8], np.int32)
    got = oracle.pooled_select(scores, lens, 1, select_k)
    want = oracle.topk(scores, lens, select_k)
    assert got.shape == want.shape
    np.testing.assert_array_equal(got, want)


@pytest.mark.parametrize("kp", [2, 3, 4, 16])
def test_selected_pools_dominate_the_rest(kp):
    rng = np.random.default_rng(kp)
    # integer scores in a small range: many exact ties
    scores = rng.integers(-2, 3, size=(8, 40)).astype(np.float64)
    lens = rng.integers(1, 40 * kp + 1, size=8).astype(np.int32)
    for select_k in (1, 4, 11):
        out = oracle.pooled_select(scores, lens, kp, select_k)
        for r in range(8):
            L = int(lens[r])
            pvis = L // kp
            rsk = min(select_k, pvis)
            head = out[r, :rsk * kp].reshape(rsk, kp) if rsk else np.zeros((0, kp), int)
            pools = head[:, 0] // kp
            # each pool expands to its kp consecutive tokens, pools ascending
            assert (head == pools[:, None] * kp + np.arange(kp)[None, :]).all()
            assert (np.diff(pools) > 0).all()
            assert (pools < pvis).all()
            assert dominance_ok(scores[r], pools, pvis)
            # the visible tail follows at the row's own base, then padding
            tail = out[r, rsk * kp: rsk * kp + (L - pvis * kp)]
            np.testing.assert_array_equal(tail, np.arange(pvis * kp, L))
            assert (out[r, rsk * kp + (L - pvis * kp):] == -1).all()


def test_invisible_and_incomplete_pools_are_never_selected():
    kp = 4
    scores = np.zeros((1, 10))
    scores[0, 5:] = 1e9          # pools 5.. are past the row's query
    out = oracle.pooled_select(scores, [22], kp, 3)   # pools 0..4 complete, tail 20, 21
    assert out[0, :12].max() < 20 and set(out[0, :12] // kp) <= {0, 1, 2, 3, 4}
    np.testing.assert_array_equal(out[0, 12:14], [20, 21])


def test_rows_shorter_than_a_pool_keep_only_their_tail():
    out = oracle.pooled_select(np.ones((2, 4)), [3, 1], 4, 2)
    np.testing.assert_array_equal(out[0, :3], [0, 1, 2])
    np.testing.assert_array_equal(out[1, :1], [0])
    assert (out[0, 3:] == -1).all() and (out[1, 1:] == -1).all()


def test_every_visible_pool_selected_gives_every_token():
    rng = np.random.default_rng(3)
    out = oracle.pooled_select(rng.standard_normal((1, 9)), [37], 4, 9)  # 9 pools visible
    np.testing.assert_array_equal(out[0, :37], np.arange(37))
    assert (out[0, 37:] == -1).all()


def test_the_tail_base_is_the_row_own_selection_size():
    # select_k = 6 but the row sees only 2 complete pools: the tail starts at
    # slot 2 * kp, not 6 * kp (the pages' per-row correction)
    out = oracle.pooled_select(np.arange(8.0)[None, :], [11], 4, 6)
    np.testing.assert_array_equal(out[0, :11], np.arange(11))
    assert (out[0, 11:] == -1).all()


# ---------------------------------------------------------------------------
# pool_valid, the second term of the candidacy test (same doc: "a pool is a
# candidate only when it is complete AND its last token is visible").

def test_all_pools_complete_is_the_ungated_selection():
    rng = np.random.default_rng(21)
    scores = rng.standard_normal((5, 120))
    lens = np.array([120, 7, 64, 33, 119], np.int32)
    ones = np.ones((5, 120), np.uint8)
    for kp, select_k in ((4, 6), (1, 40), (8, 2)):
        np.testing.assert_array_equal(
            oracle.pooled_select(scores, lens, kp, select_k, pool_valid=ones),
            oracle.pooled_select(scores, lens, kp, select_k))


@pytest.mark.parametrize("kp", [2, 4, 8])
def test_an_incomplete_pool_is_the_pool_scored_minus_infinity(kp):
    # While a row has at least row_select_k candidates, marking a pool
    # incomplete selects exactly what scoring it -inf (the pages' -FLT_MAX,
    # below every candidate) selects in the ungated walk, and changes
    # nothing if the pool was not selected.
    rng = np.random.default_rng(kp + 30)
    for trial in range(40):
        npool = int(rng.integers(3, 12))
        L = npool * kp + int(rng.integers(0, kp))
        scores = rng.integers(-3, 4, size=(1, npool)).astype(np.float64)
        select_k = int(rng.integers(1, npool))
        valid = np.ones((1, npool), np.uint8)
        off = rng.choice(npool, size=int(rng.integers(1, npool - select_k + 1)), replace=False)
        valid[0, off] = 0
        masked = scores.copy()
        masked[0, off] = -np.inf
        np.testing.assert_array_equal(
            oracle.pooled_select(scores, [L], kp, select_k, pool_valid=valid),
            oracle.pooled_select(masked, [L], kp, select_k))
        # a pool that is not selected anyway may be marked incomplete freely
        base = oracle.pooled_select(scores, [L], kp, select_k)
        chosen = set(int(t) // kp for t in base[0, :select_k * kp])
        free = [p for p in range(npool) if p not in chosen]
        if free:
            v2 = np.ones((1, npool), np.uint8)
            v2[0, free[0]] = 0
            np.testing.assert_array_equal(
                oracle.pooled_select(scores, [L], kp, select_k, pool_valid=v2), base)


def test_too_few_candidates_leave_pool_places_empty_and_the_tail_in_place():
    # 5 pools visible, select_k 4, only pools 1 and 3 complete: their tokens,
    # then -1 for the two places that no candidate fills, then the tail at
    # slot 4 * kp (the row's position alone sets it)
    kp = 4
    scores = np.array([[5.0, 1.0, 9.0, 2.0, 7.0]])
    valid = np.array([[0, 1, 0, 1, 0]], np.uint8)
    out = oracle.pooled_select(scores, [22], kp, 4, pool_valid=valid)
    np.testing.assert_array_equal(out[0, :8], [4, 5, 6, 7, 12, 13, 14, 15])
    assert (out[0, 8:16] == -1).all()
    np.testing.assert_array_equal(out[0, 16:18], [20, 21])
    assert (out[0, 18:] == -1).all()
    # no complete pool at all: only the tail
    out = oracle.pooled_select(scores, [22], kp, 4, pool_valid=np.zeros((1, 5), np.uint8))
    assert (out[0, :16] == -1).all()
    np.testing.assert_array_equal(out[0, 16:18], [20, 21])


def test_rows_of_one_sequence_share_its_pool_marks():
    rng = np.random.default_rng(40)
    scores = rng.standard_normal((4, 12))
    lens = np.array([40, 44, 48, 47], np.int32)   # two sequences of two rows
    valid = (rng.random((2, 12)) < 0.6).astype(np.uint8)
    got = oracle.pooled_select(scores, lens, 4, 5, pool_valid=valid, rows_per_seq=2)
    for r in range(4):
        one = oracle.pooled_select(scores[r:r + 1], lens[r:r + 1], 4, 5,
                                   pool_valid=valid[r // 2:r // 2 + 1])
        np.testing.assert_array_equal(got[r], one[0])
