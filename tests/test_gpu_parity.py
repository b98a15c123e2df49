"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded
workloads small enough for the oracle to check every row, but spanning several
score tiles, selection chunks and attention chunks with ragged tails."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_03_amd import dsa
from sparse_attention_decode_03_amd import workloads as wl

from gpu_common import (assert_attention_row, check_attention, check_scores, check_selection,
                        check_selection_end_to_end, host, run_step, small, bf16_codes_to_f64)

pytestmark = pytest.mark.gpu


def full_check(inputs, rows=None):
    step = run_step(inputs)
    scores, sel, out = host(step)
    rows = range(inputs["seq_lens"].shape[0]) if rows is None else rows
    refs, _ = check_scores(inputs, scores, rows)
    check_selection(inputs, scores, sel, rows)
    check_selection_end_to_end(inputs, refs, sel, rows)
    check_attention(inputs, sel, out, rows)
    return step, scores, sel, out


def test_tiny_workload_end_to_end():
    inputs = wl.make_inputs(wl.WORKLOADS["tiny"])
    step, scores, sel, out = full_check(inputs)
    # the oracle's own pipeline picks the same tokens (no near-ties at this size)
    _, osel, oatt = oracle.decode(inputs)
    np.testing.assert_array_equal(sel, osel)
    assert np.abs(out - oatt).max() <= 2e-2


@pytest.mark.parametrize("case", [
    dict(num_seqs=3, rows_per_seq=1, lengths="ragged", lo=2500, hi=9000, top_k=2048, seed=11),
    dict(num_seqs=2, rows_per_seq=3, lengths="verify", base=5000, top_k=1024, seed=12),
    dict(num_seqs=2, rows_per_seq=1, context=4100, top_k=300, page_size=16, seed=13,
         num_heads=40),
    dict(num_seqs=2, rows_per_seq=2, lengths="ragged", lo=100, hi=1500, top_k=2048, seed=14,
         index_heads=4, index_dim=64, num_heads=8),
    dict(num_seqs=1, rows_per_seq=1, context=6000, top_k=2048, seed=15, key_dist="student_t3"),
    # 128-token tiles of the K-row pass: four rows (direct selection), and
    # two rows past 8192 tokens (group maxima for the threshold filter)
    dict(num_seqs=3, rows_per_seq=4, lengths="verify", base=3000, top_k=512, seed=16),
    dict(num_seqs=2, rows_per_seq=2, lengths="verify", base=9500, top_k=1024, seed=17),
    # six rows: three units of two rows per sequence, each walking the keys
    dict(num_seqs=2, rows_per_seq=6, lengths="verify", base=4000, top_k=512, seed=18),
])
def test_parity_across_tiles_chunks_and_tails(case):
    full_check(small(**case))


def test_rows_at_and_around_top_k():
    # L = k - 1, k, k + 1, 1: all selected below or at k, exact radix above
    inputs = small(num_seqs=4, rows_per_seq=1, lengths="ragged", lo=501, hi=501, top_k=500,
                   seed=21)
    inputs["seq_lens"] = np.array([499, 500, 501, 1], np.int32)
    step, scores, sel, out = full_check(inputs)
    assert (sel[0, :499] == np.arange(499)).all() and sel[0, 499] == -1
    assert (sel[1] == np.arange(500)).all()
    assert sel[3, 0] == 0 and (sel[3, 1:] == -1).all()


def test_every_e4m3_code_round_trips_through_attention():
    """A row that sees one token attends to exactly kv_scale * c, so every
    finite E4M3 code must come back as the bf16 of its exact value."""
    inputs = small(num_seqs=2, rows_per_seq=1, context=64, top_k=8, page_size=16, seed=31,
                   num_heads=16)
    codes = np.arange(256, dtype=np.uint8)
    codes[[0x7F, 0xFF]] = 0
    rng = np.random.default_rng(0)
    bt = inputs["block_tables"]
    for s in range(2):
        inputs["kv_cache"][bt[s, 0], 0] = np.concatenate([codes, rng.permutation(codes)])
    inputs["seq_lens"] = np.array([1, 1], np.int32)
    step = run_step(inputs)
    out = bf16_codes_to_f64(step.out.cpu().numpy().view(np.uint16))
    table = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double()
    for s in range(2):
        row = torch.from_numpy(inputs["kv_cache"][bt[s, 0], 0].astype(np.int64))
        # kv_scale is a power of two, so kv_scale * c is exact in bf16; the
        # sum p * c starts from +0, so the -0.0 code comes back as +0.0 (equal
        # as values, as in the fp64 oracle)
        exact = (table[row] * inputs["kv_scale"]).numpy()
        for h in range(inputs["num_heads"]):
            np.testing.assert_array_equal(out[s, h], exact, err_msg=f"seq {s} head {h}")


def test_massive_ties_and_signed_zeros_in_selection():
    """Scores with heavy exact ties (and -0.0 next to +0.0) go through the
    standalone selector; the result must equal the oracle's total order."""
    rng = np.random.default_rng(41)
    R, max_len, top_k = 6, 9000, 1000
    sc = rng.integers(-3, 4, size=(R, max_len)).astype(np.float32)
    sc[1] = 1.0                                  # every score equal
    sc[2, ::2] = -0.0                             # signed zeros interleaved
    sc[2, 1::2] = 0.0
    sc[3] = np.where(rng.random(max_len) < 0.5, -0.0, 0.0)
    sc[4, :] = rng.standard_normal(max_len).astype(np.float32)
    sc[4, 7000:] = 1e30                           # the tail beats everything
    lens = np.array([9000, 9000, 8999, 4097, 9000, 1000], np.int32)
    shape = dsa.Shape(num_seqs=R, rows_per_seq=1, num_heads=8, latent_dim=512, index_heads=4,
                      index_dim=64, top_k=top_k, page_size=64, max_len=max_len,
                      k_capacity=max_len, max_blocks_per_seq=(max_len + 63) // 64, num_pages=1)
    stride = dsa.score_stride(shape)
    padded = np.full((R, stride), np.nan, np.float32)  # past max_len: never read
    padded[:, :max_len] = sc
    d_sc = torch.from_numpy(padded).cuda()
    d_len = torch.from_numpy(lens).cuda()
    d_sel = torch.full((R, top_k), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    dsa.topk_select(shape, d_sc, d_len, d_sel, ws)
    torch.cuda.synchronize()
    got = d_sel.cpu().numpy()
    for r in range(R):
        ref = oracle.topk_row(sc[r, :lens[r]].astype(np.float64), int(lens[r]), top_k)
        np.testing.assert_array_equal(got[r], ref, err_msg=f"row {r}")
    assert (got[1] == np.arange(top_k)).all()


def test_page_permutation_is_bit_exact_and_results_are_deterministic():
    inputs = small(num_seqs=2, rows_per_seq=2, lengths="verify", base=3000, top_k=1024, seed=51)
    a = run_step(inputs)
    out_a, sel_a, sc_a = a.out.cpu().numpy(), a.sel.cpu().numpy(), a.scores.cpu().numpy()
    again = run_step(inputs)
    np.testing.assert_array_equal(again.out.cpu().numpy(), out_a)
    sc_b = again.scores.cpu().numpy()
    for r, L in enumerate(inputs["seq_lens"]):  # entries past L_r are not written
        np.testing.assert_array_equal(sc_b[r, :L], sc_a[r, :L])
    rng = np.random.default_rng(5)
    perm = rng.permutation(inputs["num_pages"])
    moved = dict(inputs)
    moved["kv_cache"] = np.empty_like(inputs["kv_cache"])
    moved["kv_cache"][perm] = inputs["kv_cache"]
    bt = inputs["block_tables"]
    moved["block_tables"] = np.where(bt >= 0, perm[np.maximum(bt, 0)], -1).astype(np.int32)
    b = run_step(moved)
    np.testing.assert_array_equal(b.sel.cpu().numpy(), sel_a)
    np.testing.assert_array_equal(b.out.cpu().numpy(), out_a)


def test_outputs_stay_inside_their_buffers():
    """Guard bands of poison around every output are left untouched."""
    inputs = small(num_seqs=2, rows_per_seq=2, lengths="ragged", lo=1500, hi=3000, top_k=512,
                   seed=61, num_heads=48)
    step = dsa.DeviceStep(inputs)
    G = 4096
    R, H = step.shape.num_rows, step.shape.num_heads
    big_sc = torch.full((step.scores.numel() + 2 * G,), 3.25, dtype=torch.float32, device="cuda")
    big_sel = torch.full((step.sel.numel() + 2 * G,), -77, dtype=torch.int32, device="cuda")
    big_out = torch.full((step.out.numel() + 2 * G,), 0x1234, dtype=torch.int16, device="cuda")
    step.scores = big_sc[G:G + step.scores.numel()].view(step.scores.shape)
    step.sel = big_sel[G:G + step.sel.numel()].view(step.sel.shape)
    step.out = big_out[G:G + step.out.numel()].view(R, H, 512)
    step.decode_k()
    torch.cuda.synchronize()
    for big, n, fill in [(big_sc, step.scores.numel(), 3.25), (big_sel, step.sel.numel(), -77),
                         (big_out, step.out.numel(), 0x1234)]:
        h = big.cpu().numpy()
        assert (h[:G] == fill).all() and (h[G + n:] == fill).all()
    scores, sel, out = host(step)
    check_selection(inputs, scores, sel, range(R))
    check_attention(inputs, sel, out, range(R))


def _tied_keys_and_unmapped_pages():
    # sequence 0: every key row equal, so every score of its rows ties and
    # the finishing workgroup takes the full-row path; sequence 1: two pages
    # inside its rows unmapped, so the attention skips their tokens
    x = small(num_seqs=2, rows_per_seq=2, lengths="ragged", lo=9000, hi=10000, top_k=1024,
              seed=72)
    x["k_normed"][0, :] = x["k_normed"][0, 0]
    x["block_tables"][1, 3] = -1
    x["block_tables"][1, 10] = -1
    return x


STAGE_CASES = {
    "ragged": lambda: small(num_seqs=2, rows_per_seq=2, lengths="ragged", lo=3000, hi=7000,
                            top_k=2048, seed=71),
    "tied keys, unmapped pages": _tied_keys_and_unmapped_pages,
    # rows no longer than top_k: every token selected, padding resolves to -1
    "rows within top_k": lambda: small(num_seqs=2, rows_per_seq=2, lengths="ragged", lo=100,
                                       hi=900, top_k=1024, seed=73),
    # 25000 pages of 4 tokens
    "many small pages": lambda: small(num_seqs=1, rows_per_seq=1, context=100000,
                                                    top_k=2048, page_size=4, seed=74),
}


@pytest.mark.parametrize("case", list(STAGE_CASES))
def test_stage_entry_points_match_the_fused_step(case):
    """The stage entry points, called one after another, give the fused
    step's bytes, and both give the oracle's results: ties broken by index
    through the full-row selection, unmapped pages skipped by the attention,
    rows within top_k, and block tables of many small pages."""
    inputs = STAGE_CASES[case]()
    print(f"case {case}: lengths {inputs['seq_lens'].tolist()}", flush=True)
    fused = run_step(inputs)
    staged = dsa.DeviceStep(inputs)
    staged.index_scores()
    staged.topk_select()
    staged.mla_decode()
    torch.cuda.synchronize()
    lens = inputs["seq_lens"]
    for r in range(len(lens)):
        np.testing.assert_array_equal(staged.scores[r, :lens[r]].cpu().numpy(),
                                      fused.scores[r, :lens[r]].cpu().numpy())
    np.testing.assert_array_equal(staged.sel.cpu().numpy(), fused.sel.cpu().numpy())
    np.testing.assert_array_equal(staged.out.cpu().numpy(), fused.out.cpu().numpy())
    scores, sel, out = host(fused)
    check_selection(inputs, scores, sel, range(len(lens)))
    # the attention skips selected tokens whose page is unmapped: the oracle
    # (which refuses them) attends over the mapped ones
    K, ps, bt = inputs["rows_per_seq"], inputs["page_size"], inputs["block_tables"]
    for r in range(len(lens)):
        ids = sel[r, :min(int(lens[r]), inputs["top_k"])]
        keep = ids[bt[r // K, ids // ps] >= 0].astype(np.int32)
        assert_attention_row(inputs, r, keep, out[r])


def test_empty_rows_and_out_of_contract_ids_are_safe():
    inputs = small(num_seqs=2, rows_per_seq=1, context=600, top_k=256, page_size=16, seed=81,
                   num_heads=16)
    inputs["seq_lens"] = np.array([0, 600], np.int32)
    step = run_step(inputs)
    out = step.out.cpu().numpy()
    assert (out[0] == 0).all()
    assert (step.sel.cpu().numpy()[0] == -1).all()
    # an id past L and a negative id are skipped by the attention (never read)
    sel = step.sel.clone()
    sel[1, 0] = 10_000
    sel[1, 1] = -5
    dsa.mla_decode(step.shape, step.q, step.kv_cache, step.block_tables, step.seq_lens, sel,
                   step.kv_scale, step.sm_scale, step.out, step.ws)
    torch.cuda.synchronize()
    got = bf16_codes_to_f64(step.out.cpu().numpy().view(np.uint16))[1]
    keep = sel.cpu().numpy()[1, 2:]
    # the reference attends over the 254 valid ids that remain
    assert_attention_row(inputs, 1, keep, got)


@pytest.mark.parametrize("rows", [6, 40])
def test_dominant_token_at_chunk_boundaries(rows):
    """One selected token carries about half of every head's softmax mass,
    placed at slot 0, 255, 256, 1023, 1024 or 2047 of a 2048-slot selection
    (8 chunks of 256 slots): the chunk edges and the row's end. A slot lost
    or counted twice at a chunk edge moves the output by ~0.2 per element,
    ten times the contract's 2e-2. Six rows run 16-head workgroups, forty
    rows 64-head ones (the kernel picks the group from the batch)."""
    L, top_k = 4096, 2048
    inputs = small(num_seqs=rows, rows_per_seq=1, context=L, top_k=top_k, seed=140 + rows)
    rng = np.random.default_rng(140 + rows)
    slots = [0, 255, 256, 1023, 1024, 2047]
    H, ps, kv_scale = inputs["num_heads"], inputs["page_size"], inputs["kv_scale"]
    sel = np.stack([np.sort(rng.choice(L, top_k, replace=False)) for _ in range(rows)]).astype(np.int32)
    # every head's query is N(s, 1) for one sign pattern s; the dominant
    # token's dequantised latent row is 0.375 * s (the E4M3 code of 0.75
    # times kv_scale 0.5, exact), so its logit is about 0.375 * 512 /
    # sqrt(512) = 8.5, while the other 2047 logits are ~N(0, 2) and their
    # exponentials sum to about 2047 e = e^8.6
    for r in range(rows):
        sgn = rng.choice([-1.0, 1.0], 512).astype(np.float32)
        qf = rng.standard_normal((H, 512)).astype(np.float32) + sgn
        inputs["q"][r] = wl.f32_to_bf16_codes(qf)
        t = int(sel[r, slots[r % len(slots)]])
        page = inputs["block_tables"][r, t // ps]
        inputs["kv_cache"][page, t % ps] = wl.f32_to_e4m3_codes(0.375 * sgn / kv_scale)
    step = dsa.DeviceStep(inputs)
    d_sel = torch.from_numpy(sel).cuda()
    dsa.mla_decode(step.shape, step.q, step.kv_cache, step.block_tables, step.seq_lens, d_sel,
                   step.kv_scale, step.sm_scale, step.out, step.ws)
    torch.cuda.synchronize()
    out = bf16_codes_to_f64(step.out.cpu().numpy().view(np.uint16))
    for r in range(rows):
        assert_attention_row(inputs, r, sel[r], out[r])
        # power: without the dominant token the oracle's output is far away
        j = slots[r % len(slots)]
        drop = np.delete(sel[r], j)
        ref_drop = oracle.mla_decode(inputs["q"][r:r + 1], inputs["kv_cache"],
                                     inputs["block_tables"][r:r + 1], inputs["seq_lens"][r:r + 1],
                                     drop[None], inputs["kv_scale"], inputs["sm_scale"], 1)[0]
        assert np.abs(out[r] - ref_drop).max() > 0.1, f"row {r}: slot {j} carries too little mass"


def test_check_metadata_on_device_arrays():
    """dsa_check_metadata reads the device arrays in stream order: a step's own
    lengths, block table and selection pass; a selected id past its row's
    length and an unmapped reachable page are named."""
    inputs = small(num_seqs=2, rows_per_seq=2, lengths="verify", base=3000, top_k=512, seed=150)
    step = run_step(inputs)
    dsa.check_metadata(step.shape, step.seq_lens, step.block_tables, step.sel)
    bad_sel = step.sel.clone()
    bad_sel[3, 7] = int(inputs["seq_lens"][3])
    with pytest.raises(dsa.DsaError) as e:
        dsa.check_metadata(step.shape, step.seq_lens, step.block_tables, bad_sel)
    assert e.value.code == dsa.DSA_EMETADATA and "sel[3][7]" in e.value.message
    bad_bt = step.block_tables.clone()
    bad_bt[1, 5] = inputs["num_pages"]
    with pytest.raises(dsa.DsaError) as e:
        dsa.check_metadata(step.shape, step.seq_lens, bad_bt, step.sel)
    assert "block_tables[1][5]" in e.value.message
