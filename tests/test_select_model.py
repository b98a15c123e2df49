"""CPU model of the GPU selector's threshold and exact cut (the algorithm of
the filter and finishing kernels, written out in numpy), checked against the
oracle's full sort under (score descending, index ascending).

The model follows the kernels step by step: the threshold tau from the
largest key of each 4-token or 32-token group (one 12-bit digit relative to
the group keys' range), the candidates {key >= tau}, then the exact cut -- relative 12-bit
digits narrow a key window onto the bin holding the top_k-th candidate
(after a first pass of value-linear bins when the candidates lie on both
sides of zero), and that bin's members are ranked directly. It exists to
show, on the CPU, that the crafted rows of the GPU route tests really reach
the narrowing route (a boundary bin of more than 256 members whose window is
then narrower than 12 bits), and that counting only the keys inside the
current window is what makes the cut exact there: a model that also counts
keys of higher bins that fall within 4096 units of the window's base selects
too few ids on these rows.
"""
import numpy as np
import pytest

import oracle
from select_rows import crafted_cut_rows, crafted_rows

DIGIT = 12
BINS = 1 << DIGIT
RANK_LIST = 256
FIN_CAP = 8192


def order_keys(scores: np.ndarray) -> np.ndarray:
    """Order-preserving uint32 image of fp32 scores, -0.0 mapped onto +0.0."""
    u = np.ascontiguousarray(scores, dtype=np.float32).view(np.uint32).copy()
    u[u == 0x80000000] = 0
    neg = (u & 0x80000000) != 0
    return np.where(neg, ~u, u | np.uint32(0x80000000)).astype(np.uint32)


def bit_len(x: int) -> int:
    return int(x).bit_length()


def key_values(keys: np.ndarray) -> np.ndarray:
    """fp32 values of order keys (the inverse of order_keys)."""
    k = keys.astype(np.uint32)
    u = np.where((k & 0x80000000) != 0, k & np.uint32(0x7FFFFFFF), ~k).astype(np.uint32)
    return u.view(np.float32)


def value_bins(keys: np.ndarray, lo: int, hi: int, value_any: bool = False):
    """The kernels' value-linear bins in fp32, or None when the key range
    [lo, hi] does not straddle zero (or its value span is not finite):
    bin = min(4095, floor((value - value(lo)) * (4096 / span))). With
    value_any (the one-kernel cut over a whole row) a range on one side of
    zero is binned by value too when the values' mean lies at least 1/16 of
    the way up their span (the kernel decides in fp32; here in fp64, which
    agrees away from that boundary)."""
    straddle = lo < 0x80000000 <= hi
    if not (straddle or value_any):
        return None
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        vlo = key_values(np.array([lo], np.uint32))[0]
        span = np.float32(key_values(np.array([hi], np.uint32))[0] - vlo)
        scale = np.float32(np.float32(BINS) / span)
        if not (span > 0 and np.isfinite(span) and np.isfinite(scale)):
            return None
        if not straddle:
            rel = key_values(keys).astype(np.float64) - np.float64(vlo)
            if not 16.0 * rel.sum() >= len(keys) * np.float64(span):
                return None
        x = np.float32(key_values(keys) - vlo) * scale
    return np.minimum(x.astype(np.float32), np.float32(BINS - 1)).astype(np.int64)


def walk_desc(hist: np.ndarray, need: int):
    """Highest-first walk: (bin where the running count reaches need, count
    above it, total)."""
    above = 0
    for b in range(len(hist) - 1, -1, -1):
        if above + int(hist[b]) >= need:
            return b, above, int(hist.sum())
        above += int(hist[b])
    return 0, 0, int(hist.sum())


def threshold(keys: np.ndarray, top_k: int):
    """The filter's tau from the row's group maxima, and the level it came
    from ('gm4 registers', 'gm4 memory', 'gm32'; tau 0 and 'every token' when
    the row has fewer than top_k 4-token groups)."""
    L = len(keys)
    pad4 = np.zeros(-(-L // 4) * 4, np.uint32)
    pad4[:L] = keys
    gm4 = pad4.reshape(-1, 4).max(axis=1)
    pad32 = np.zeros(-(-L // 32) * 32, np.uint32)
    pad32[:L] = keys
    gm32 = pad32.reshape(-1, 32).max(axis=1)
    ng4, ng32 = len(gm4), len(gm32)
    if ng4 >= top_k and ng4 <= 32 * 256:
        gk, level = gm4, "gm4 registers"
    elif ng32 >= top_k:
        gk, level = gm32, "gm32"
    elif ng4 >= top_k:
        gk, level = gm4, "gm4 memory"
    else:
        return 0, "every token"
    lo, hi = int(gk.min()), int(gk.max())
    shift = max(bit_len(hi - lo) - DIGIT, 0)
    hist = np.bincount(((gk.astype(np.int64) - lo) >> shift), minlength=BINS)
    b, _, _ = walk_desc(hist, top_k)
    return lo + (b << shift), level


def exact_cut(kk: np.ndarray, ids: np.ndarray, top_k: int, window_only: bool = True,
              value_any: bool = False):
    """The finishing workgroup's cut over candidates (kk, ids) in ascending id
    order. Returns (selected ids ascending, route details): the passes, whether
    a narrowed window was below 12 bits, and how the boundary bin was ranked
    ('member list' for at most 256 members, 'equal keys' by index otherwise)."""
    kk = kk.astype(np.int64)
    need = top_k
    passes = 0
    narrow = False
    pre = np.zeros(len(kk), bool)     # taken by the value pass
    valid = np.ones(len(kk), bool)
    vb = value_bins(kk.astype(np.uint32), int(kk.min()), int(kk.max()), value_any)
    if vb is not None:
        b, before, total = walk_desc(np.bincount(vb, minlength=BINS), need)
        passes += 1
        assert total >= top_k
        need -= before
        pre = vb > b
        valid = vb == b
        if valid.sum() <= RANK_LIST:
            members = np.flatnonzero(valid)
            order = sorted(members, key=lambda j: (-kk[j], ids[j]))
            take = pre.copy()
            take[np.array(order[:max(need, 0)], dtype=np.int64)] = True
            return np.sort(ids[take]), dict(passes=passes, narrow=narrow, rank="member list",
                                            value_pass=True)
    base = int(kk[valid].min())
    bits = bit_len(int(kk[valid].max()) - base)
    while True:
        shift = max(bits - DIGIT, 0)
        nb = 1 << (bits - shift) if window_only else BINS
        inside = valid & (kk >= base)
        d = (kk - base) >> shift
        inside &= d < nb
        hist = np.bincount(d[inside], minlength=BINS)
        b, before, total = walk_desc(hist, need)
        passes += 1
        if passes == 1:
            assert total >= top_k
        need -= before
        count_b = int(hist[b])
        bin_lo = base + (b << shift)
        if count_b <= RANK_LIST or shift == 0:
            break
        base, bits = bin_lo, shift
        narrow |= bits < DIGIT
    take = valid & (kk >= bin_lo + (1 << shift))
    inbin = valid & (kk >= bin_lo) & ~take
    take |= pre
    members = np.flatnonzero(inbin)
    order = sorted(members, key=lambda j: (-kk[j], ids[j]))
    take[np.array(order[:max(need, 0)], dtype=np.int64)] = True
    rank = "member list" if count_b <= RANK_LIST else "equal keys"
    return np.sort(ids[take]), dict(passes=passes, narrow=narrow, rank=rank, value_pass=vb is not None)


def gather_mode(cand: np.ndarray, L: int) -> str:
    """How the finishing workgroup's 1024 threads take the candidates: by
    slice (each slice's candidates fit a fixed block of 1024 / P threads, at
    most 8 each) or spread evenly by a search of the slice offsets."""
    P = -(-L // 4096)
    counts = np.bincount(cand // 4096, minlength=P)
    tps = 1024 // P
    srun = -(-int(counts.max()) // tps)
    return "by slice" if srun <= 8 else "spread"


def model_select(scores: np.ndarray, top_k: int, window_only: bool = True):
    """The selector end to end on one row: (ids or None, route dict). Route
    'all' (L <= top_k), 'full' (the full-row fallback, not modelled: ids are
    None) or 'cut'."""
    L = len(scores)
    if L <= top_k:
        return np.arange(L), dict(route="all")
    keys = order_keys(scores)
    tau, level = threshold(keys, top_k)
    cand = np.flatnonzero(keys >= tau)
    if len(cand) < top_k or len(cand) > FIN_CAP:
        return None, dict(route="full", level=level, candidates=len(cand))
    sel, cut = exact_cut(keys[cand], cand, top_k, window_only)
    return sel, dict(route="cut", level=level, gather=gather_mode(cand, L),
                     candidates=len(cand), **cut)


def oracle_ids(scores: np.ndarray, top_k: int) -> np.ndarray:
    ref = oracle.topk_row(scores.astype(np.float64), len(scores), top_k)
    return ref[ref >= 0]


@pytest.mark.parametrize("name", list(crafted_cut_rows()))
def test_crafted_rows_reach_the_narrowed_cut_and_the_model_is_exact(name):
    row = crafted_cut_rows()[name]
    top_k = 2048
    sel, info = model_select(row, top_k)
    assert info["route"] == "cut", f"{name}: {info}"
    assert info["passes"] >= 2 and info["narrow"], f"{name}: {info}"
    np.testing.assert_array_equal(sel, oracle_ids(row, top_k))
    # counting keys past the narrowed window (the bug this guards against)
    # loses ids on these rows
    bad, _ = model_select(row, top_k, window_only=False)
    assert len(bad) < top_k, f"{name}: the unwindowed count still selected {len(bad)}"


@pytest.mark.parametrize("seed", range(6))
def test_model_matches_the_oracle_on_random_rows(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(3000, 40000))
    top_k = int(rng.choice([64, 300, 1024, 2048]))
    kind = seed % 3
    if kind == 0:
        row = rng.standard_normal(L).astype(np.float32)
    elif kind == 1:
        row = np.round(rng.standard_t(3, L), 2).astype(np.float32)
    else:
        row = (50.0 + rng.standard_normal(L)).astype(np.float32)
    sel, info = model_select(row, top_k)
    if info["route"] == "full":
        pytest.skip("full-row route (not modelled)")
    np.testing.assert_array_equal(sel, oracle_ids(row, top_k))


# The launch shapes of the GPU route test (max_len, top_k).
GPU_ROUTE_SHAPES = [(131072, 2048), (135168, 2048), (131072, 2304)]


def test_gpu_route_rows_cover_every_route():
    """Every route of the selector is reached by some crafted row of the GPU
    route test, and every modelled route's ids equal the oracle's."""
    seen = set()
    for max_len, top_k in GPU_ROUTE_SHAPES:
        for name, L, vals in crafted_rows(max_len, top_k):
            row = vals[:L]
            sel, info = model_select(row, top_k)
            seen.add(info["route"])
            if info["route"] == "cut":
                seen.update({info["level"], info["gather"], info["rank"]})
                if info["value_pass"]:
                    seen.add("value-bin first cut pass")
                if info["passes"] >= 2:
                    seen.add("narrowed" + (" below 12 bits" if info["narrow"] else ""))
                if max_len == 131072 and top_k == 2048:
                    np.testing.assert_array_equal(sel, oracle_ids(row, top_k), err_msg=name)
            elif info["route"] == "full":
                seen.add(info["level"])
    want = {"all", "full", "cut", "gm4 registers", "gm4 memory", "gm32", "every token",
            "by slice", "spread", "member list", "equal keys", "narrowed below 12 bits",
            "value-bin first cut pass"}
    assert want <= seen, f"routes not reached: {sorted(want - seen)}"


# The one-kernel launch shapes of the GPU route test (max_len, top_k).
GPU_DIRECT_SHAPES = [(8192, 2048), (8192, 100), (6000, 2048), (12000, 2048), (16384, 2048),
                     (16388, 2048), (24576, 2048)]


def test_one_kernel_cut_rows_take_every_first_pass_and_are_exact():
    """The one-kernel selection cuts a whole row: its crafted rows reach the
    value-bin first pass across zero and on one side of it, and the key-digit
    first pass for a heavy tail on one side of zero; every cut equals the
    oracle's."""
    seen = set()
    for max_len, top_k in GPU_DIRECT_SHAPES:
        for name, L, vals in crafted_rows(max_len, top_k):
            if L <= top_k:
                continue
            row = vals[:L]
            keys = order_keys(row)
            sel, info = exact_cut(keys, np.arange(L), top_k, value_any=True)
            np.testing.assert_array_equal(sel, oracle_ids(row, top_k),
                                          err_msg=f"{name} ({max_len}, {top_k})")
            across = int(keys.min()) < 0x80000000 <= int(keys.max())
            seen.add(("value bins" if info["value_pass"] else "key digits")
                     + (" across zero" if across else " on one side of zero"))
    want = {"value bins across zero", "value bins on one side of zero",
            "key digits on one side of zero"}
    assert want <= seen, f"first passes not reached: {sorted(want - seen)}"
