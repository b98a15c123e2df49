"""Pins for the CPU oracle: each check ties it to something other than itself
(the published number formats through torch's casts, hand-worked examples,
closed forms, brute force over all subsets, dense attention, invariants)."""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_03_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf16(x):
    return wl.f32_to_bf16_codes(np.asarray(x, dtype=np.float32))


def e4m3(x):
    return wl.f32_to_e4m3_codes(np.asarray(x, dtype=np.float32))


def torch_e4m3_table():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


# ---------------------------------------------------------------- formats

def test_bf16_decode_matches_torch_on_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([oracle.bf16_to_f64(c) for c in codes[::7]])
    np.testing.assert_array_equal(np.isnan(got), np.isnan(ref[::7]))
    ok = ~np.isnan(ref[::7])
    np.testing.assert_array_equal(got[ok], ref[::7][ok])
    # and every code of the exponent-boundary region exactly
    for c in list(range(0, 0x90)) + list(range(0x7F00, 0x8090)) + list(range(0xFF00, 0x10000)):
        r = ref[c]
        g = oracle.bf16_to_f64(c)
        assert (math.isnan(r) and math.isnan(g)) or (g == r and math.copysign(1, g) == math.copysign(1, r))


def test_e4m3_decode_matches_torch_on_all_256_codes():
    ref = torch_e4m3_table()
    got = np.array([oracle.e4m3_to_f64(c) for c in range(256)])
    assert np.isnan(got).sum() == 2 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(got[ok], ref[ok])
    np.testing.assert_array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_e4m3_decode_matches_ocp_spec_values():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_ocp_values.json")))
    for code, val in g["values"].items():
        got = oracle.e4m3_to_f64(int(code, 16))
        assert got == val and math.copysign(1, got) == math.copysign(1, val), code
    for code in g["nan_codes"]:
        assert math.isnan(oracle.e4m3_to_f64(int(code, 16)))


def test_generator_e4m3_encode_is_nearest_and_saturating():
    table = torch_e4m3_table()
    finite = np.where(~np.isnan(table))[0]
    vals = table[finite]
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(4000) * 40, [500.0, -1e4, 448.0, 464.0, 2.0 ** -10]])
    codes = e4m3(x)
    dec = table[codes]
    assert not np.isnan(dec).any()
    for xi, di in zip(x.astype(np.float32).astype(np.float64), dec):
        xc = min(max(xi, -448.0), 448.0)
        best = np.min(np.abs(vals - xc))
        assert abs(di - xc) == best


# ---------------------------------------------------------------- scores

def test_scores_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "index_scores_worked.json")))
    q = bf16(np.array(g["q_idx"])[None])
    w = np.array(g["w"], dtype=np.float32)[None]
    k = bf16(np.array(g["keys"])[None])
    sl = np.array([len(g["keys"])], dtype=np.int32)
    sc = oracle.index_scores(q, w, k, sl)
    np.testing.assert_array_equal(sc[0], g["expected_scores"])


def test_scores_one_hot_keys_pick_a_query_column():
    rng = np.random.default_rng(1)
    Hi, D = 5, 16
    qf = rng.standard_normal((1, Hi, D)).astype(np.float32)
    q = bf16(qf)
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()
    w = rng.random((1, Hi)).astype(np.float32)
    keys = np.eye(D, dtype=np.float32)[None]
    sc = oracle.index_scores(q, w, bf16(keys), np.array([D], np.int32))
    expect = (w[0].astype(np.float64)[:, None] * np.maximum(qd[0], 0.0)).sum(axis=0)
    np.testing.assert_allclose(sc[0], expect, rtol=1e-15, atol=0)


def test_scores_single_head_unit_weight_is_relu_of_dot():
    rng = np.random.default_rng(2)
    D, L = 64, 50
    q = bf16(rng.standard_normal((1, 1, D)))
    k = bf16(rng.standard_normal((1, L, D)))
    qd = torch.from_numpy(q.view(np.int16)).view(torch.bfloat16).double().numpy()[0, 0]
    kd = torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).double().numpy()[0]
    sc = oracle.index_scores(q, np.ones((1, 1), np.float32), k, np.array([L], np.int32))
    expect = np.maximum(kd @ qd, 0.0)
    assert (expect == 0).sum() > 5 and (expect > 0).sum() > 5
    np.testing.assert_allclose(sc[0], expect, rtol=1e-13, atol=1e-13)


def test_scores_linear_in_weights_and_homogeneous_in_keys():
    rng = np.random.default_rng(3)
    Hi, D, L = 4, 32, 40
    q = bf16(rng.standard_normal((1, Hi, D)))
    kf = rng.standard_normal((1, L, D)).astype(np.float32)
    k = bf16(kf)
    k2 = bf16(torch.from_numpy(k.view(np.int16)).view(torch.bfloat16).float().numpy() * 2)
    w1 = rng.random((1, Hi)).astype(np.float32)
    w2 = rng.random((1, Hi)).astype(np.float32)
    sl = np.array([L], np.int32)
    s1 = oracle.index_scores(q, w1, k, sl)
    s2 = oracle.index_scores(q, w2, k, sl)
    s12 = oracle.index_scores(q, (w1.astype(np.float64) + w2).astype(np.float32), k, sl)
    np.testing.assert_allclose(s12, s1 + s2, rtol=1e-6)  # w1+w2 rounds to f32
    np.testing.assert_allclose(oracle.index_scores(q, w1, k2, sl), 2 * s1, rtol=1e-14)
    assert (oracle.index_scores(bf16(np.zeros((1, Hi, D))), w1, k, sl) == 0).all()


def test_scores_row_to_sequence_mapping_and_length_mask():
    rng = np.random.default_rng(4)
    S, K, Hi, D, cap = 2, 2, 2, 16, 12
    k = bf16(rng.standard_normal((S, cap, D)))
    q = bf16(rng.standard_normal((S * K, Hi, D)))
    w = rng.random((S * K, Hi)).astype(np.float32)
    sl = np.array([5, 6, 11, 12], np.int32)
    sc = oracle.index_scores(q, w, k, sl, rows_per_seq=K, max_len=12)
    for r in range(S * K):
        s = r // K
        alone = oracle.index_scores(q[r:r + 1], w[r:r + 1], k[s:s + 1], sl[r:r + 1], 1, 12)
        np.testing.assert_array_equal(sc[r], alone[0])
        assert (sc[r, sl[r]:] == 0).all()
    # a different sequence's keys give different scores
    assert not np.array_equal(sc[1, :5], oracle.index_scores(q[1:2], w[1:2], k[1:2], sl[:1], 1, 5)[0])


# ---------------------------------------------------------------- select

def brute_force_topk(scores, L, k):
    """The unique subset whose every member beats every non-member under
    (score desc, index asc), found by trying all subsets."""
    n = min(k, L)
    beats = lambda a, b: scores[a] > scores[b] or (scores[a] == scores[b] and a < b)
    found = []
    for sub in itertools.combinations(range(L), n):
        ss = set(sub)
        if all(beats(a, b) for a in sub for b in range(L) if b not in ss):
            found.append(sub)
    assert len(found) == 1
    return list(found[0]) + [-1] * (k - n)


def test_topk_equals_brute_force_over_all_subsets():
    rng = np.random.default_rng(5)
    for trial in range(60):
        L = int(rng.integers(0, 10))
        k = int(rng.integers(1, 6))
        sc = rng.integers(-2, 3, size=max(L, 1)).astype(np.float64)  # many ties
        got = oracle.topk_row(sc, L, k)
        assert list(got) == brute_force_topk(sc, L, k), (sc, L, k)


def test_topk_equals_numpy_lexsort_on_large_rows():
    rng = np.random.default_rng(6)
    R, L, k = 3, 5000, 300
    sc = np.round(rng.standard_normal((R, L)) * 8) / 8  # heavy ties
    sel = oracle.topk(sc, np.full(R, L, np.int32), k)
    for r in range(R):
        order = np.lexsort((np.arange(L), -sc[r]))
        np.testing.assert_array_equal(sel[r], np.sort(order[:k]))
        # invariants
        chosen = set(sel[r].tolist())
        mn = sc[r, sel[r]].min()
        for t in range(L):
            if t not in chosen:
                assert sc[r, t] < mn or (sc[r, t] == mn and t > max(i for i in chosen if sc[r, i] == mn))


def test_topk_ties_signed_zero_short_rows_and_nan():
    assert list(oracle.topk_row(np.ones(10), 10, 4)) == [0, 1, 2, 3]
    sc = np.array([0.0, -0.0, 0.0, -0.0, -1.0])
    assert list(oracle.topk_row(sc, 5, 3)) == [0, 1, 2]
    sc = np.array([-0.0, 0.0, -1.0])
    assert list(oracle.topk_row(sc, 3, 1)) == [0]
    assert list(oracle.topk_row(np.arange(5.0), 5, 8)) == [0, 1, 2, 3, 4, -1, -1, -1]
    assert list(oracle.topk_row(np.arange(5.0), 0, 3)) == [-1, -1, -1]
    assert list(oracle.topk_row(np.array([1.0, 5.0, 3.0, 5.0]), 4, 2)) == [1, 3]
    with pytest.raises(oracle.OracleError):
        oracle.topk_row(np.array([1.0, np.nan]), 2, 1)


# ---------------------------------------------------------------- attend

def dequant(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def bf16_to_f64(codes):
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(torch.bfloat16).double().numpy()


def test_attend_hand_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "attend_worked.json")))
    q = bf16(np.array(g["q"])[None, None])
    kv = np.array(g["latent_codes"], np.uint8)[None]  # one page of 2 slots
    out = oracle.mla_decode(q, kv, np.array([[0]], np.int32), np.array([2], np.int32),
                            np.array([[0, 1]], np.int32), g["kv_scale"], g["sm_scale"])
    np.testing.assert_allclose(out[0, 0], g["expected_out"], rtol=1e-15)


def small_attend_inputs(seed, L, top_k, H=3, Dl=24, ps=4, S=1, K=1):
    w = wl.custom(num_seqs=S, rows_per_seq=K, num_heads=H, latent_dim=Dl, index_heads=2,
                  index_dim=16, top_k=top_k, page_size=ps, seed=seed, context=L)
    return wl.make_inputs(w)


def test_attend_with_every_token_selected_is_dense_attention():
    for seed, L, ps in [(10, 13, 4), (11, 40, 8), (12, 7, 16)]:
        x = small_attend_inputs(seed, L, top_k=64, ps=ps)
        sel = oracle.topk(np.zeros((1, L)), x["seq_lens"], 64)
        out = oracle.mla_decode(x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"], sel,
                                x["kv_scale"], x["sm_scale"])
        # dense attention from scratch: gather every token through the table
        bt = x["block_tables"][0]
        c = np.stack([dequant(x["kv_cache"][bt[t // ps], t % ps]) for t in range(L)]) * x["kv_scale"]
        qd = bf16_to_f64(x["q"][0])
        z = x["sm_scale"] * qd @ c.T
        p = torch.softmax(torch.from_numpy(z), dim=-1).numpy()
        np.testing.assert_allclose(out[0], p @ c, rtol=1e-12, atol=1e-14)


def test_attend_single_row_identical_rows_and_weights():
    x = small_attend_inputs(20, L=9, top_k=4)
    kv, bt, sl = x["kv_cache"], x["block_tables"], x["seq_lens"]
    one = np.array([[5, -1, -1, -1]], np.int32)
    sl1 = np.array([6], np.int32)  # top_k 4 > ... use a row of length 1 instead
    out = oracle.mla_decode(x["q"], kv, bt, np.array([1], np.int32), np.array([[0, -1, -1, -1]], np.int32),
                            x["kv_scale"], x["sm_scale"])
    ps = x["page_size"]
    row0 = dequant(kv[bt[0, 0], 0]) * x["kv_scale"]
    for h in range(x["num_heads"]):
        np.testing.assert_array_equal(out[0, h], row0)
    # identical rows: copy token 0's row onto tokens 1..8
    kv2 = kv.copy()
    for t in range(1, 9):
        kv2[bt[0, t // ps], t % ps] = kv[bt[0, 0], 0]
    sel = np.array([[0, 3, 5, 8]], np.int32)
    out2 = oracle.mla_decode(x["q"], kv2, bt, sl, sel, x["kv_scale"], x["sm_scale"])
    np.testing.assert_allclose(out2[0], np.broadcast_to(row0, out2[0].shape), rtol=1e-14, atol=1e-15)
    p = oracle.softmax_weights(x["q"], kv, bt, sl, sel, x["kv_scale"], x["sm_scale"], 0, 1)
    assert abs(p.sum() - 1.0) < 1e-12 and (p > 0).all()
    del one, sl1


def test_attend_invariant_under_page_permutation_and_kv_scale_law():
    x = small_attend_inputs(30, L=29, top_k=8, ps=4, S=2, K=2)
    sel = np.array([[0, 3, 7, 9, 12, 20, 27, 28]] * 4, np.int32)
    sel[0, -1] = 1  # row 0 has length 29 too; keep every id < L
    base = oracle.mla_decode(x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"], sel,
                             x["kv_scale"], x["sm_scale"], rows_per_seq=2)
    rng = np.random.default_rng(0)
    perm = rng.permutation(x["num_pages"])
    kv = np.empty_like(x["kv_cache"])
    kv[perm] = x["kv_cache"]
    bt = np.where(x["block_tables"] >= 0, perm[np.maximum(x["block_tables"], 0)], -1).astype(np.int32)
    moved = oracle.mla_decode(x["q"], kv, bt, x["seq_lens"], sel, x["kv_scale"], x["sm_scale"],
                              rows_per_seq=2)
    np.testing.assert_array_equal(base, moved)
    # doubling kv_scale while halving sm_scale keeps the logits and doubles the output
    dbl = oracle.mla_decode(x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"], sel,
                            2 * x["kv_scale"], x["sm_scale"] / 2, rows_per_seq=2)
    np.testing.assert_allclose(dbl, 2 * base, rtol=1e-13, atol=1e-15)
    # each row reads its own sequence's table (r // K): the batched call equals
    # one-row calls made with that table alone
    for r in range(4):
        alone = oracle.mla_decode(x["q"][r:r + 1], x["kv_cache"], x["block_tables"][r // 2:r // 2 + 1],
                                  x["seq_lens"][r:r + 1], sel[r:r + 1], x["kv_scale"], x["sm_scale"])
        np.testing.assert_array_equal(alone[0], base[r])
    # rows 2,3 read sequence 1's table: swapping the sequences' tables changes them
    swapped = oracle.mla_decode(x["q"], x["kv_cache"], x["block_tables"][::-1].copy(), x["seq_lens"],
                                sel, x["kv_scale"], x["sm_scale"], rows_per_seq=2)
    assert not np.allclose(swapped[2:], base[2:])


def test_attend_empty_row_is_zero_and_bad_ids_are_refused():
    x = small_attend_inputs(40, L=9, top_k=4)
    out = oracle.mla_decode(x["q"], x["kv_cache"], x["block_tables"], np.array([0], np.int32),
                            np.full((1, 4), -1, np.int32), x["kv_scale"], x["sm_scale"])
    assert (out == 0).all()
    with pytest.raises(oracle.OracleError):
        oracle.mla_decode(x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"],
                          np.array([[0, 1, 2, 9]], np.int32), x["kv_scale"], x["sm_scale"])


# ---------------------------------------------------------------------------
# The cache-write side (latent RMSNorm + FP8 write, indexer key LayerNorm).

def brute_force_e4m3(y, table):
    """Nearest finite E4M3 code to y by exhaustive search, ties to the even
    code (mantissa LSB 0), saturating beyond +-448."""
    finite = [c for c in range(256) if not math.isnan(table[c])]
    best = None
    for c in finite:
        if (c & 0x80) != (0x80 if math.copysign(1.0, y) < 0 else 0):
            continue
        d = abs(table[c] - y)
        if best is None or d < best[0] - 1e-300 or (abs(d - best[0]) <= 1e-300 and c % 2 == 0):
            best = (d, c)
    return best[1]


def test_e4m3_encoder_is_the_nearest_code_ties_to_even():
    table = torch_e4m3_table()
    rng = np.random.default_rng(7)
    ys = list(rng.standard_normal(300) * 40.0) + list(rng.standard_normal(100) * 0.01)
    pos = sorted(v for v in table[:0x7F] if not math.isnan(v))
    # every midpoint between neighbouring magnitudes, and its neighbours
    for a, b in zip(pos[:-1], pos[1:]):
        mid = (a + b) / 2
        ys += [mid, -mid, math.nextafter(mid, 0.0), math.nextafter(mid, 1e9)]
    ys += [0.0, -0.0, 448.0, 447.9, 460.0, 1e6, -1e6, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11]
    for y in ys:
        assert oracle.e4m3_encode(y) == brute_force_e4m3(y, table), y


def test_e4m3_encoder_agrees_with_torch_cast_on_float32_values():
    rng = np.random.default_rng(8)
    x = (rng.standard_normal(4000) * 30.0).astype(np.float32)
    x = np.clip(x, -448.0, 448.0)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in x], dtype=np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_bf16_encoder_agrees_with_torch_cast_on_float32_values():
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(4000) * 3.0, rng.standard_normal(100) * 1e-30,
                        [0.0, -0.0, 1.0, -2.5, 65504.0]]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.bf16_encode(float(v)) for v in x], dtype=np.uint16)
    np.testing.assert_array_equal(got, ref)


def test_latent_row_rms_is_one_and_scale_free():
    rng = np.random.default_rng(10)
    x = rng.standard_normal(512) * 3.0
    ones = np.ones(512)
    y, _ = oracle.latent_row(x, ones, eps=0.0, kv_scale=1.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-12            # RMSNorm output has unit RMS
    y2, c2 = oracle.latent_row(x * 7.5, ones, eps=0.0, kv_scale=1.0)
    _, c1 = oracle.latent_row(x, ones, eps=0.0, kv_scale=1.0)
    np.testing.assert_array_equal(c1, c2)                # invariant to a positive scale
    w = rng.uniform(0.5, 1.5, 512)
    yw, _ = oracle.latent_row(x, w, eps=0.0, kv_scale=0.5)
    np.testing.assert_allclose(yw, y * w / 0.5, rtol=1e-13)  # plain weight (no 1 + w), 1/kv_scale
    # eps enters under the root: mean(x^2) + eps
    ye, _ = oracle.latent_row(x, ones, eps=0.25, kv_scale=1.0)
    np.testing.assert_allclose(ye, x / math.sqrt(np.mean(x * x) + 0.25), rtol=1e-13)


def test_layernorm_row_is_standardised_then_affine():
    rng = np.random.default_rng(11)
    x = rng.standard_normal(128) * 2.0 + 5.0
    y, _ = oracle.layernorm_row(x, np.ones(128), np.zeros(128), eps=0.0)
    assert abs(np.mean(y)) < 1e-12 and abs(np.mean(y * y) - 1.0) < 1e-12
    y_shift, _ = oracle.layernorm_row(x + 100.0, np.ones(128), np.zeros(128), eps=0.0)
    np.testing.assert_allclose(y_shift, y, atol=1e-12)   # mean subtraction
    w = rng.uniform(0.5, 1.5, 128)
    b = rng.standard_normal(128) * 0.1
    ya, codes = oracle.layernorm_row(x, w, b, eps=0.0)
    np.testing.assert_allclose(ya, y * w + b, rtol=1e-12, atol=1e-15)  # weight and BIAS
    ref = torch.from_numpy(ya.astype(np.float32)).to(torch.bfloat16).view(torch.int16)
    # the stored code is the bf16 of the value (equal to the float32 route
    # except where the float32 rounding lands exactly on a bf16 midpoint)
    assert (codes == ref.numpy().view(np.uint16)).mean() > 0.99


def test_cache_write_slot_arithmetic_and_untouched_elsewhere():
    """A hand-worked placement: page size 4, block table row [3, 0, 2]; the
    token at position 5 lands in logical block 1 -> physical page 0, slot 1."""
    Dl, D, ps = 8, 4, 4
    rng = np.random.default_rng(12)
    kv_a = bf16(rng.standard_normal((2, Dl)))
    k_proj = bf16(rng.standard_normal((2, D)))
    lw = bf16(np.ones(Dl))
    kw = bf16(np.ones(D))
    kb = bf16(np.zeros(D))
    bt = np.array([[3, 0, 2], [1, -1, -1]], np.int32)
    cache = np.full((4, ps, Dl), 0x55, np.uint8)
    keys = np.full((2, 12, D), 0x1234, np.uint16)
    seq_lens = np.array([6, 0], np.int32)                   # row 1 writes nothing
    c2, k2 = oracle.cache_write(kv_a, lw, k_proj, kw, kb, seq_lens, bt, 1, ps, 1e-6, 0.5,
                                cache, keys)
    changed = np.argwhere((c2 != cache).any(axis=2))
    assert changed.tolist() == [[0, 1]]                      # page 0, slot 1 only
    _, codes = oracle.latent_row(oracle._bf16_values(kv_a[0]), np.ones(Dl), 1e-6, 0.5)
    np.testing.assert_array_equal(c2[0, 1], codes)
    assert np.argwhere((k2 != keys).any(axis=2)).tolist() == [[0, 5]]
    # an unmapped page is skipped for the latent but the key row is stored
    c3, k3 = oracle.cache_write(kv_a, lw, k_proj, kw, kb, np.array([6, 2], np.int32),
                                np.array([[3, 0, 2], [-1, -1, -1]], np.int32), 1, ps, 1e-6, 0.5,
                                cache, keys)
    assert np.argwhere((c3 != cache).any(axis=2)).tolist() == [[0, 1]]
    assert np.argwhere((k3 != keys).any(axis=2)).tolist() == [[0, 5], [1, 1]]



def test_validity_marks_follow_the_key_rows_and_form_a_prefix():
    """The mark goes with the key row (layer.rs `indexer_forward`: the key
    and its validity mark are placed from the same device position). Writing
    a sequence's tokens one step at a time (positions 0, 1, 2, ...) leaves
    exactly the written prefix marked; an out-of-range row marks nothing, and
    a row whose latent page is unmapped still marks its position."""
    Dl, D, ps, cap = 8, 4, 4, 12
    rng = np.random.default_rng(13)
    lw, kw, kb = bf16(np.ones(Dl)), bf16(np.ones(D)), bf16(np.zeros(D))
    bt = np.array([[3, 0, 2], [-1, -1, -1]], np.int32)  # sequence 1: no latent page at all
    cache = np.zeros((4, ps, Dl), np.uint8)
    keys = np.zeros((2, cap, D), np.uint16)
    valid = np.zeros((2, cap), np.uint8)
    for step in range(1, 8):
        kv_a = bf16(rng.standard_normal((2, Dl)))
        k_proj = bf16(rng.standard_normal((2, D)))
        lens = np.array([step, step if step <= 5 else 0], np.int32)  # row 1 stops after 5
        cache, keys, valid = oracle.cache_write(kv_a, lw, k_proj, kw, kb, lens, bt, 1, ps, 1e-6,
                                                1.0, cache, keys, valid=valid)
        assert valid[0].tolist() == [1] * step + [0] * (cap - step)
        assert valid[1].tolist() == [1] * min(step, 5) + [0] * (cap - min(step, 5))
    # a row past the capacity writes no key and no mark
    _, _, v2 = oracle.cache_write(bf16(np.ones((1, Dl))), lw, bf16(np.ones((1, D))), kw, kb,
                                  np.array([cap + 1], np.int32), bt[:1], 1, ps, 1e-6, 1.0, cache,
                                  keys[:1], valid=valid[:1])
    np.testing.assert_array_equal(v2, valid[:1])

# ---------------------------------------------------------------------------
# Softmax weights, the attention error scale and the end-to-end pipeline at
# K > 1, each against torch's casts and softmax on the definitions.

def torch_weights_and_rows(x, r, sel_row):
    """Dense logits of row r over the ids sel_row (through torch's bf16 and
    E4M3 casts), their softmax, and the dequantised rows."""
    K, ps = x["rows_per_seq"], x["page_size"]
    s = r // K
    bt = x["block_tables"][s]
    c = np.stack([dequant(x["kv_cache"][bt[t // ps], t % ps]) for t in sel_row]) * x["kv_scale"]
    qd = bf16_to_f64(x["q"][r])                       # [H, Dl]
    z = x["sm_scale"] * (qd @ c.T)                    # [H, n]
    p = torch.softmax(torch.from_numpy(z), dim=-1).numpy()
    return p, c


def test_softmax_weights_equal_torch_softmax_of_the_dense_logits():
    x = small_attend_inputs(50, L=37, top_k=9, H=4, Dl=32, ps=4, S=2, K=2)
    x["seq_lens"] = np.array([37, 30, 33, 21], np.int32)
    rng = np.random.default_rng(3)
    sel = np.stack([np.sort(rng.choice(int(L), 9, replace=False)) for L in x["seq_lens"]]).astype(np.int32)
    for r in range(4):
        p_ref, _ = torch_weights_and_rows(x, r, sel[r])
        for h in range(4):
            p = oracle.softmax_weights(x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"], sel,
                                       x["kv_scale"], x["sm_scale"], r, h, rows_per_seq=2)
            np.testing.assert_allclose(p, p_ref[h], rtol=1e-12, atol=1e-15,
                                       err_msg=f"row {r} head {h}")
    # the weights move with sm_scale as the definition says: a wrong scale
    # inside the oracle would not give torch's weights at a second scale
    p2 = oracle.softmax_weights(x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"], sel,
                                x["kv_scale"], 3 * x["sm_scale"], 3, 2, rows_per_seq=2)
    x3 = dict(x, sm_scale=3 * x["sm_scale"])
    np.testing.assert_allclose(p2, torch_weights_and_rows(x3, 3, sel[3])[0][2], rtol=1e-12,
                               atol=1e-15)


def test_attention_error_scale_is_the_magnitude_weighted_output():
    x = small_attend_inputs(51, L=29, top_k=12, H=3, Dl=24, ps=8, S=2, K=2)
    rng = np.random.default_rng(4)
    sel = np.stack([np.sort(rng.choice(int(L), 12, replace=False)) for L in x["seq_lens"]]).astype(np.int32)
    args = (x["q"], x["kv_cache"], x["block_tables"], x["seq_lens"], sel, x["kv_scale"],
            x["sm_scale"])
    scale = oracle.mla_decode_abs(*args, rows_per_seq=2)
    out = oracle.mla_decode(*args, rows_per_seq=2)
    for r in range(4):
        p, c = torch_weights_and_rows(x, r, sel[r])
        np.testing.assert_allclose(scale[r], p @ np.abs(c), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(out[r], p @ c, rtol=1e-12, atol=1e-15)
    assert (scale >= np.abs(out) - 1e-15).all()
    # a latent whose values are all positive: the scale is the output itself
    pos = dict(x, kv_cache=np.where(x["kv_cache"] == 0x7F, 0x7F, x["kv_cache"] & 0x7F).astype(np.uint8))
    args_pos = (pos["q"], pos["kv_cache"], pos["block_tables"], pos["seq_lens"], sel,
                pos["kv_scale"], pos["sm_scale"])
    np.testing.assert_allclose(oracle.mla_decode_abs(*args_pos, rows_per_seq=2),
                               oracle.mla_decode(*args_pos, rows_per_seq=2), rtol=1e-13)


def test_decode_pipeline_with_several_rows_per_sequence():
    """oracle.decode at K = 3: every row's scores, selection and attention
    against torch computations of the three definitions on that row's own
    sequence (r // K) and its own length."""
    w = wl.custom(num_seqs=2, rows_per_seq=3, num_heads=4, latent_dim=32, index_heads=3,
                  index_dim=16, top_k=20, page_size=8, seed=52, lengths="verify", base=40)
    x = wl.make_inputs(w)
    scores, sel, att = oracle.decode(x)
    K = 3
    for r in range(6):
        s, L = r // K, int(x["seq_lens"][r])
        qi = bf16_to_f64(x["q_idx"][r])                            # [Hi, D]
        keys = bf16_to_f64(x["k_normed"][s, :L])                   # [L, D]
        dots = torch.from_numpy(keys @ qi.T)                       # [L, Hi]
        ref = (torch.relu(dots) * torch.from_numpy(x["w"][r].astype(np.float64))).sum(1).numpy()
        np.testing.assert_allclose(scores[r][:L], ref, rtol=1e-12, atol=1e-14, err_msg=f"row {r}")
        order = np.lexsort((np.arange(L), -ref))[:20]
        np.testing.assert_array_equal(sel[r], np.sort(order), err_msg=f"row {r}")
        p, c = torch_weights_and_rows(x, r, np.sort(order))
        np.testing.assert_allclose(att[r], p @ c, rtol=1e-12, atol=1e-14, err_msg=f"row {r}")
    # the rows of a sequence differ only by their horizon: row 2 sees two
    # more tokens than row 0 of the same sequence
    assert len(scores[2]) == len(scores[0]) + 2
