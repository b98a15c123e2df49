"""Attention launches with more (row, chunk) units of 64 heads than the GPU
has CUs run one workgroup per CU that walks its units in turn; a one-row call
runs the one-round kernel. A row's output must have the same bytes either
way (glm5next_dsa/layer.rs source page, `attend_rows`: one launch for every
row with each row's arithmetic untouched; `decode_k`: bit-identical to serial
decodes) and agree with the oracle. Rows with nothing visible, rows of one
chunk and rows shorter than the longest are mixed in, so that the walk skips
units, writes an empty row's zeros and stores one-chunk rows directly."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_03_amd import dsa

from gpu_common import bf16_codes_to_f64, check_attention, small

pytestmark = pytest.mark.gpu


def with_lengths_and_ids(inputs, lens, seed):
    """The inputs with row lengths `lens` and a selection of distinct random
    ids in [0, L_r) per row (-1 past min(top_k, L_r))."""
    rng = np.random.Generator(np.random.PCG64(seed))
    inputs = dict(inputs)
    inputs["seq_lens"] = np.asarray(lens, np.int32)
    top_k = inputs["top_k"]
    sel = np.full((len(lens), top_k), -1, np.int32)
    for r, L in enumerate(lens):
        n = min(top_k, L)
        sel[r, :n] = rng.permutation(L)[:n]
    return inputs, sel


def attend(inputs, sel):
    step = dsa.DeviceStep(inputs)
    step.sel.copy_(torch.from_numpy(sel))
    step.mla_decode()
    torch.cuda.synchronize()
    return step.out.cpu().numpy().view(np.uint16)


def one_row(inputs, r):
    sub = dict(inputs)
    S = inputs["num_seqs"]
    assert inputs["rows_per_seq"] == 1 and len(inputs["seq_lens"]) == S
    sub["num_seqs"] = 1
    for key in ("q_idx", "w", "q", "seq_lens"):
        sub[key] = np.ascontiguousarray(inputs[key][r:r + 1])
    sub["k_normed"] = np.ascontiguousarray(inputs["k_normed"][r:r + 1])
    sub["block_tables"] = np.ascontiguousarray(inputs["block_tables"][r:r + 1])
    return sub


def check_walk(inputs, sel, rows_serial, rows_oracle):
    out = attend(inputs, sel)
    for r in rows_serial:
        one = attend(one_row(inputs, r), sel[r:r + 1])
        assert np.array_equal(one[0], out[r]), f"row {r} (L = {inputs['seq_lens'][r]})"
    L = inputs["seq_lens"]
    for r in range(len(L)):
        if L[r] == 0:
            assert not out[r].any(), f"empty row {r} not zero"
    check_attention(inputs, sel, bf16_codes_to_f64(out), rows_oracle)


def test_unit_walk_with_empty_short_and_one_chunk_rows():
    # 40 rows x 8 chunks = 320 units of 64 heads: more than one per CU for
    # some workgroups, none with work for others
    lens = [4096, 0, 100, 256, 257, 2048, 2049, 3000, 0, 1, 511, 512, 4096, 4000] * 3
    lens = lens[:40]
    base = small(num_seqs=len(lens), rows_per_seq=1, context=4096, top_k=2048, seed=210)
    inputs, sel = with_lengths_and_ids(base, lens, 211)
    check_walk(inputs, sel, rows_serial=range(len(lens)), rows_oracle=[0, 1, 2, 3, 4, 6, 10, 13])


def test_unit_walk_with_two_head_groups():
    # 128 heads: two 64-head groups per (row, chunk), 24 x 8 x 2 = 384 units
    lens = [3000, 2048, 0, 700, 4096, 1500] * 4
    base = small(num_seqs=len(lens), rows_per_seq=1, num_heads=128, context=4096, top_k=2048,
                 seed=212)
    inputs, sel = with_lengths_and_ids(base, lens, 213)
    check_walk(inputs, sel, rows_serial=range(len(lens)), rows_oracle=[0, 2, 3, 4])


def test_unit_walk_of_one_chunk_rows():
    # top_k = 256: every row is one chunk and stores its output directly;
    # 300 rows = 300 units
    rng = np.random.Generator(np.random.PCG64(214))
    lens = rng.integers(0, 600, size=300).tolist()
    lens[0], lens[1] = 0, 600
    base = small(num_seqs=len(lens), rows_per_seq=1, context=600, top_k=256, seed=215)
    inputs, sel = with_lengths_and_ids(base, lens, 216)
    check_walk(inputs, sel, rows_serial=[0, 1, 2, 3, 150, 257, 299], rows_oracle=[1, 2, 3, 299])
