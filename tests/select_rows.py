"""Crafted score rows for the selector route tests (seeded; no method
arithmetic). `crafted_rows` returns (name, length, values) triples for one
launch shape; the GPU route test runs them through dsa_topk_select and the
CPU model test confirms which route of the selector each one reaches."""
import numpy as np


def ties_at_cut(base: np.ndarray, top_k: int, n_ties: int, rng) -> np.ndarray:
    """`base` with n_ties random tokens set to the row's top_k-th score, so
    the k-th place is a block of exact ties."""
    row = base.astype(np.float32).copy()
    kth = np.sort(row)[::-1][top_k - 1]
    row[rng.choice(len(row), n_ties, replace=False)] = kth
    return row


def crafted_cut_rows(L: int = 131072, top_k: int = 2048, seed: int = 7):
    """Rows that pass the exact cut with a boundary bin of more than 256
    members, narrowed to a window of fewer than 12 bits (candidate key range
    of ~19-22 bits)."""
    rng = np.random.default_rng(seed)
    rows = {}
    rows["offset normal, 300 ties at the cut"] = ties_at_cut(
        (100.0 + rng.standard_normal(L)).astype(np.float32), top_k, 300, rng)
    rows["student-t(3), 300 ties at the cut"] = ties_at_cut(
        rng.standard_t(3, L).astype(np.float32), top_k, 300, rng)
    # 600 keys within 40 units of the k-th score of an offset normal row
    # (128-unit bins whose upper neighbours are all occupied): the boundary
    # bin holds the cluster and is then ranked key by key in a 7-bit window
    x = (100.0 + rng.standard_normal(L)).astype(np.float32)
    kth = np.sort(x)[::-1][top_k - 1]
    u0 = int(np.array([kth], np.float32).view(np.uint32)[0])
    cluster = (u0 - 20 + rng.integers(0, 40, 600)).astype(np.uint32).view(np.float32)
    x[rng.choice(L, 600, replace=False)] = cluster
    rows["600-key cluster within 40 units of the cut, bins above occupied"] = x
    return rows


def crafted_rows(max_len: int, top_k: int):
    rng = np.random.default_rng(2024)
    rows = []

    def add(name, L, values):
        L = min(L, max_len)
        full = np.zeros(max_len, np.float32)
        full[:L] = values[:L]
        rows.append((name, L, full))

    n = max_len
    add("normal, full length", n, rng.standard_normal(n).astype(np.float32))
    add("normal, 40000 tokens", 40000, rng.standard_normal(n).astype(np.float32))
    add("normal, 30000 tokens", 30000, rng.standard_normal(n).astype(np.float32))
    add("all equal, overflow to the full-row path", 20000, np.ones(n, np.float32))
    add("seven integer levels, overflow", n, rng.integers(-3, 4, n).astype(np.float32))
    add("ascending ramp", n, np.arange(n, dtype=np.float32))
    add("descending ramp", 100000, -np.arange(n, dtype=np.float32))
    add("student-t tails", n, rng.standard_t(3, n).astype(np.float32))
    add("every token a candidate", 4 * top_k - 5, rng.standard_normal(n).astype(np.float32))
    add("exactly top_k 4-token groups", 4 * top_k - 1, rng.standard_normal(n).astype(np.float32))
    add("one past top_k", top_k + 1, rng.standard_normal(n).astype(np.float32))
    add("shorter than top_k", top_k - 3, rng.standard_normal(n).astype(np.float32))
    zeros = np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0))
    zeros[rng.choice(min(70000, n), 100, replace=False)] = rng.random(100).astype(np.float32) + 0.5
    add("signed zeros with a few positives", 70000, zeros)
    add("ties at the threshold (one decimal)", n,
        np.round(rng.standard_normal(n), 1).astype(np.float32))
    add("negative scores only", 50000, -np.abs(rng.standard_normal(n)).astype(np.float32))
    # a tight cluster (keys within ~800 units) between two far outliers: the
    # candidates overflow the finishing workgroup and take the full-row path
    cluster = (1.0 + 1e-4 * rng.random(n)).astype(np.float32)
    cluster[rng.integers(0, n)] = np.float32(1e30)
    cluster[rng.integers(0, n)] = np.float32(-1e30)
    add("clustered keys between far outliers", n, cluster)
    # top-k packed into the row's last few thousand tokens
    late = rng.standard_normal(n).astype(np.float32)
    late[-3000:] += 50.0
    add("winners packed at the end", n, late)
    # boundary bins of more than 256 members narrowed below 12 bits
    Lc = min(n, 131072)
    for name, vals in crafted_cut_rows(Lc, top_k).items():
        add(name, Lc, vals)
    # non-negative rows (index scores are, when the head weights are): a bell
    # spread over its span, and a heavy tail whose outliers set the span (the
    # one-kernel cut bins the first by value, the second by key digits)
    rng2 = np.random.default_rng(2025)
    add("non-negative bell", n, (2.0 * np.abs(rng2.standard_normal(n))).astype(np.float32))
    add("non-negative heavy tail", n, np.abs(rng2.standard_cauchy(n)).astype(np.float32))
    return rows
