"""decode_k: a K-row verify call is byte-identical to K serial calls that each
hold one row of every sequence (glm5next_dsa/layer.rs source page, `decode_k`
doc: bit-identical to K serial decodes; `attend_rows`: one launch for every
row with per-row arithmetic untouched)."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_03_amd import dsa
from sparse_attention_decode_03_amd import workloads as wl

from gpu_common import small

pytestmark = pytest.mark.gpu


def row_slice(inputs, rows):
    """The inputs of a call that holds only `rows` (one per sequence)."""
    sub = dict(inputs)
    sub["rows_per_seq"] = 1
    for key in ("q_idx", "w", "q", "seq_lens"):
        sub[key] = np.ascontiguousarray(inputs[key][rows])
    return sub


def assert_serial_equals_batched(inputs):
    K = inputs["rows_per_seq"]
    S = inputs["num_seqs"]
    batched = dsa.DeviceStep(inputs)
    batched.decode_k()
    torch.cuda.synchronize()
    b_sc = batched.scores.cpu().numpy()
    b_sel = batched.sel.cpu().numpy()
    b_out = batched.out.cpu().numpy()
    lens = inputs["seq_lens"]
    for j in range(K):
        rows = [s * K + j for s in range(S)]
        one = dsa.DeviceStep(row_slice(inputs, rows))
        one.decode_k()
        torch.cuda.synchronize()
        sc, se, ou = one.scores.cpu().numpy(), one.sel.cpu().numpy(), one.out.cpu().numpy()
        for i, r in enumerate(rows):
            L = lens[r]
            assert np.array_equal(sc[i, :L].view(np.uint32), b_sc[r, :L].view(np.uint32)), r
            assert np.array_equal(se[i], b_sel[r]), r
            assert np.array_equal(ou[i], b_out[r]), r


# K = 2 and 4: one unit of rows per sequence in the index pass (128-token
# tiles); 6, 8 and 12: units of two or four rows each walking the keys; 3:
# one odd unit (256-token tiles)
@pytest.mark.parametrize("K,seed", [(2, 1), (4, 2), (8, 3), (3, 4), (6, 5), (12, 6)])
def test_verify_rows_bit_identical_to_serial_calls(K, seed):
    # The K-row call has more (row, chunk) work than each serial call, so
    # the attention runs in larger head groups: 16 heads for the serial
    # calls, 16, 32 and 64 for K = 2, 4 and 8. The bytes must still agree (a
    # head's arithmetic never depends on the heads that share its workgroup).
    inputs = small(num_seqs=3, rows_per_seq=K, lengths="verify", base=4500, top_k=2048,
                   seed=100 + seed)
    assert_serial_equals_batched(inputs)


def test_row_group_of_sixteen_is_bit_identical_and_in_parity():
    """A row group of 16 rows of one sequence (the prefill row-group shape):
    every row's scores, selection over its own horizon and output equal a
    single-row call, and the group agrees with the oracle."""
    from gpu_common import check_attention, check_scores, check_selection, host
    inputs = small(num_seqs=2, rows_per_seq=16, lengths="verify", base=3000, top_k=512,
                   seed=120, page_size=32)
    assert_serial_equals_batched(inputs)
    step = dsa.DeviceStep(inputs)
    step.decode_k()
    torch.cuda.synchronize()
    scores, sel, out = host(step)
    rows = [0, 7, 15, 16, 31]
    check_scores(inputs, scores, rows)
    check_selection(inputs, scores, sel, rows)
    check_attention(inputs, sel, out, rows)


def test_verify_rows_bit_identical_when_rows_select_everything():
    # lengths straddle top_k: some rows select all tokens, others run the radix
    inputs = small(num_seqs=2, rows_per_seq=4, lengths="verify", base=2046, top_k=2048,
                   seed=110, page_size=16)
    assert_serial_equals_batched(inputs)


def test_verify_workload_at_full_size_is_bit_identical_to_serial_calls():
    """The K-token verify workload itself (16 sequences x 4 rows, L = 16385
    .. 16388): its one call scores with the four-row index pass and attends
    in 64-head workgroups over 512 workgroups, while each serial call (16
    rows) runs the one-row index pass and smaller head groups; the bytes
    must agree."""
    inputs = wl.make_inputs(wl.WORKLOADS["kverify"])
    assert_serial_equals_batched(inputs)


def test_timed_entry_point_writes_the_same_bytes():
    # dsa_decode_k_timed launches the same kernels as dsa_decode_k with a
    # start/stop HIP event pair bound to each: its outputs must match byte
    # for byte, every pair must span a non-negative time, and the pairs must
    # follow the stream order.
    inputs = small(num_seqs=2, rows_per_seq=4, lengths="verify", base=5000, top_k=2048, seed=77)
    a = dsa.DeviceStep(inputs)
    a.decode_k()
    b = dsa.DeviceStep(inputs)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(10)]
    for e in evs:
        e.record(stream)
    torch.cuda.synchronize()
    dsa.decode_k_timed(b.shape, b.q_idx, b.w, b.k_normed, b.q, b.kv_cache, b.block_tables,
                       b.seq_lens, b.kv_scale, b.sm_scale, b.scores, b.sel, b.out, b.ws, evs,
                       stream=stream)
    torch.cuda.synchronize()
    assert torch.equal(a.sel, b.sel)
    assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
    spans = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(5)]
    assert all(s >= 0.0 for s in spans), spans
    assert spans[0] > 0.0 and spans[3] > 0.0, spans
    gaps = [evs[2 * i + 1].elapsed_time(evs[2 * i + 2]) for i in range(4)]
    assert all(g >= 0.0 for g in gaps), gaps
