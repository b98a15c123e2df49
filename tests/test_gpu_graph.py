"""The whole step captured into a HIP graph and replayed (the capture-safe
contract of the boundary: no allocation, no memset, no host round trip inside
a call; grids sized from max_len, lengths read on the device). One capture is
replayed at two sets of lengths -- shorter rows, then rows grown in place up
to max_len -- with eager work and synchronisations between replays, and every
replay must equal the eager call at the same lengths byte for byte and agree
with the CPU oracle at those lengths (glm5next_dsa/layer.rs source page: the
graph-safe ceiling launch and the removal of host-to-device copies from
`decode_k`; its note that a ceiling baked in at capture made long replays
diverge)."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_03_amd import dsa

from gpu_common import (bf16_codes_to_f64, check_attention, check_scores, check_selection,
                        check_selection_end_to_end, small)

pytestmark = pytest.mark.gpu


def snapshot(step, lens):
    sc = step.scores.cpu().numpy()
    return ([sc[r, :L].copy() for r, L in enumerate(lens)], step.sel.cpu().numpy().copy(),
            step.out.cpu().numpy().copy())


def assert_same(a, b, what):
    for r, (x, y) in enumerate(zip(a[0], b[0])):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{what}: scores row {r}"
    assert np.array_equal(a[1], b[1]), f"{what}: sel"
    assert np.array_equal(a[2], b[2]), f"{what}: out"


def test_captured_step_replays_like_eager_at_any_length():
    inputs = small(num_seqs=2, rows_per_seq=2, lengths="verify", base=5000, top_k=1024, seed=91)
    long_lens = inputs["seq_lens"].copy()                    # 5001, 5002 per sequence
    short_lens = np.array([3000, 3001, 1500, 1501], np.int32)
    step = dsa.DeviceStep(inputs)
    side = torch.cuda.Stream()

    def eager(lens):
        step.seq_lens.copy_(torch.from_numpy(lens))
        with torch.cuda.stream(side):
            step.decode_k(stream=side)
        torch.cuda.synchronize()
        return snapshot(step, lens)

    ref_short = eager(short_lens)
    ref_long = eager(long_lens)

    step.seq_lens.copy_(torch.from_numpy(short_lens))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        step.decode_k(stream=side)
    torch.cuda.synchronize()

    for i, lens in enumerate([short_lens, long_lens, short_lens, long_lens]):
        # eager work between replays, then the new lengths in place
        scratch = torch.randn(1 << 20, device="cuda")
        scratch.mul_(2.0).sum().item()
        step.scores.fill_(-1.0)
        step.sel.fill_(-7)
        step.out.fill_(0x1357)
        step.seq_lens.copy_(torch.from_numpy(lens))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot(step, lens)
        assert_same(got, ref_short if lens is short_lens else ref_long, f"replay {i}")
        # and the replayed step against the oracle at these lengths
        at = dict(inputs, seq_lens=lens)
        rows = range(len(lens))
        scores = step.scores.cpu().numpy()
        sel = step.sel.cpu().numpy()
        out = bf16_codes_to_f64(step.out.cpu().numpy().view(np.uint16))
        refs, _ = check_scores(at, scores, rows)
        check_selection(at, scores, sel, rows)
        check_selection_end_to_end(at, refs, sel, rows)
        check_attention(at, sel, out, rows)
