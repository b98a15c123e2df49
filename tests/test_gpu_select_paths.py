"""GPU selection on crafted score rows, through the standalone dsa_topk_select
entry point: every route of the selector must give exactly the oracle's top-k
under (score descending, index ascending) (glm5next_dsa/layer.rs source page:
`select_row`, and the doc of the prefill row-group selector before
`batch_select_enabled`).

Four launch shapes for the threshold filter and the finish: rows up to
131072 tokens, rows past it (more slices than the others), a top_k past
2048, and rows one token past the one-kernel cap; and seven for the
one-kernel selection of rows of at most 24576 tokens (DSA_SELECT_DIRECT_MAX),
where the whole row is held, 8 to 24 tokens a thread, and cut exactly (the
same rows clamped to that length: all-equal, few levels, ramps, signed
zeros, ties at the cut). The rows (tests/select_rows.py)
reach these routes, as the CPU model of the selector confirms
(test_select_model.py::test_gpu_route_rows_cover_every_route): rows within
top_k; the threshold from 4-token group keys held in registers or re-read
from memory, or from 32-token group keys, or every token a candidate; the
finishing workgroup's candidates taken by slice or spread by an offset
search; the exact cut in one digit pass, narrowed over several (also into
windows under 12 bits, with more than 256 members in the boundary bin), and
its boundary bin ranked member by member or, for one shared key, by index;
and the full-row fallback when the candidates overflow it."""
import numpy as np
import pytest
import torch

import oracle
from sparse_attention_decode_03_amd import dsa

from select_rows import crafted_rows

pytestmark = pytest.mark.gpu

ROUTES = {
    "131072 tokens": (131072, 2048),
    "135168 tokens": (135168, 2048),
    "top_k 2304": (131072, 2304),
    "8192 tokens, one kernel": (8192, 2048),
    "8192 tokens, top_k 100, one kernel": (8192, 100),
    "6000 tokens, one kernel": (6000, 2048),
    "12000 tokens, one kernel (12 a thread)": (12000, 2048),
    "16384 tokens, one kernel (16 a thread)": (16384, 2048),
    "16388 tokens, one kernel (20 a thread)": (16388, 2048),
    "24576 tokens, one kernel (24 a thread)": (24576, 2048),
    "24577 tokens": (24577, 2048),
}


def test_one_kernel_routes_are_the_short_ones():
    assert all((max_len <= dsa.SELECT_DIRECT_MAX) == ("one kernel" in name)
               for name, (max_len, _) in ROUTES.items())


@pytest.mark.parametrize("route", list(ROUTES))
def test_every_selector_route_is_exact(route):
    MAX_LEN, TOP_K = ROUTES[route]
    rows = crafted_rows(MAX_LEN, TOP_K)
    R = len(rows)
    print(f"route {route}: max_len {MAX_LEN}, top_k {TOP_K}, {R} rows", flush=True)
    shape = dsa.Shape(num_seqs=R, rows_per_seq=1, num_heads=8, latent_dim=512, index_heads=4,
                      index_dim=64, top_k=TOP_K, page_size=64, max_len=MAX_LEN,
                      k_capacity=MAX_LEN, max_blocks_per_seq=(MAX_LEN + 63) // 64, num_pages=1)
    stride = dsa.score_stride(shape)
    assert stride >= MAX_LEN, "the launch shape is refused"
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
