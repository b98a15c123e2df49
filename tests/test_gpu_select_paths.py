"""GPU selection on crafted score rows, through the standalone dsa_topk_select
entry point: every route of the selector (threshold from 32-token or 4-token
group maxima, group keys held in registers or re-read, every token a
candidate, the full-row fallback for rows whose candidates overflow) must
give exactly the oracle's top-k under (score descending, index ascending)
(glm5next_dsa/layer.rs source page: `select_row`, and the doc of the prefill
row-group selector before `batch_select_enabled`)."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_03_amd import dsa

pytestmark = pytest.mark.gpu

MAX_LEN = 131072
TOP_K = 2048


def crafted_rows():
    rng = np.random.default_rng(2024)
    rows = []

    def add(name, L, values):
        full = np.zeros(MAX_LEN, np.float32)
        full[:L] = values[:L]
        rows.append((name, L, full))

    add("normal, 32-token groups", MAX_LEN, rng.standard_normal(MAX_LEN).astype(np.float32))
    add("normal, 4-token group keys re-read", 40000,
        rng.standard_normal(MAX_LEN).astype(np.float32))
    add("all equal, overflow to the full-row path", 20000, np.ones(MAX_LEN, np.float32))
    add("seven integer levels, overflow", MAX_LEN,
        rng.integers(-3, 4, MAX_LEN).astype(np.float32))
    add("ascending ramp", MAX_LEN, np.arange(MAX_LEN, dtype=np.float32))
    add("descending ramp", 100000, -np.arange(MAX_LEN, dtype=np.float32))
    add("student-t tails", MAX_LEN, rng.standard_t(3, MAX_LEN).astype(np.float32))
    add("every token a candidate", 8191, rng.standard_normal(MAX_LEN).astype(np.float32))
    add("one past top_k", TOP_K + 1, rng.standard_normal(MAX_LEN).astype(np.float32))
    zeros = np.where(rng.random(MAX_LEN) < 0.5, np.float32(-0.0), np.float32(0.0))
    zeros[rng.choice(70000, 100, replace=False)] = rng.random(100).astype(np.float32) + 0.5
    add("signed zeros with a few positives", 70000, zeros)
    add("ties at the threshold (one decimal)", MAX_LEN,
        np.round(rng.standard_normal(MAX_LEN), 1).astype(np.float32))
    add("negative scores only", 50000, -np.abs(rng.standard_normal(MAX_LEN)).astype(np.float32))
    return rows


def test_every_selector_route_is_exact():
    rows = crafted_rows()
    R = len(rows)
    shape = dsa.Shape(num_seqs=R, rows_per_seq=1, num_heads=8, latent_dim=512, index_heads=4,
                      index_dim=64, top_k=TOP_K, page_size=64, max_len=MAX_LEN,
                      k_capacity=MAX_LEN, max_blocks_per_seq=MAX_LEN // 64, num_pages=1)
    stride = dsa.score_stride(shape)
    padded = np.full((R, stride), np.nan, np.float32)  # past L: never read
    lens = np.zeros(R, np.int32)
    for r, (_, L, vals) in enumerate(rows):
        padded[r, :L] = vals[:L]
        lens[r] = L
    d_sc = torch.from_numpy(padded).cuda()
    d_len = torch.from_numpy(lens).cuda()
    d_sel = torch.full((R, TOP_K), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(dsa.workspace_bytes(shape), dtype=torch.uint8, device="cuda")
    dsa.topk_select(shape, d_sc, d_len, d_sel, ws)
    torch.cuda.synchronize()
    got = d_sel.cpu().numpy()
    for r, (name, L, vals) in enumerate(rows):
        ref = oracle.topk_row(vals[:L].astype(np.float64), L, TOP_K)
        np.testing.assert_array_equal(got[r], ref, err_msg=name)
    # the same call again on the same workspace gives the same bytes
    d_sel2 = torch.full((R, TOP_K), -9, dtype=torch.int32, device="cuda")
    dsa.topk_select(shape, d_sc, d_len, d_sel2, ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(d_sel2.cpu().numpy(), got)
