"""dsa_decode_k_noalloc: the whole step with the library's per-device scratch
array as workspace, for callers that cannot allocate. It runs the same
kernels as dsa_decode_k, so its scores on [0, L_r), selection and output must
equal dsa_decode_k's byte for byte -- here on two calls in a row, the second
with a smaller input (the array keeps the first call's contents) -- and a
shape whose workspace exceeds the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from sparse_attention_decode_03_amd import dsa

from gpu_common import small


def test_refuses_a_shape_past_the_scratch_array_before_any_launch():
    # 64 rows of 65536 tokens need ~290 MiB of selection candidates alone
    sh = dsa.Shape(num_seqs=64, rows_per_seq=1, num_heads=64, latent_dim=512, index_heads=32,
                   index_dim=128, top_k=2048, page_size=64, max_len=65536, k_capacity=65536,
                   max_blocks_per_seq=1024, num_pages=65536)
    assert dsa.workspace_bytes(sh) > dsa.NOALLOC_SCRATCH_BYTES
    p = 4096  # never dereferenced: the size check comes first
    rc = dsa.load().dsa_decode_k_noalloc(ctypes.byref(sh), p, p, p, p, p, p, p, 0.5, 0.1, p, p,
                                         p, None)
    assert rc == dsa.DSA_EWORKSPACE
    assert "scratch array" in dsa.last_error()


def outputs(step, lens):
    sc = step.scores.cpu().numpy()
    return ([sc[r, :L].view(np.uint32).copy() for r, L in enumerate(lens)],
            step.sel.cpu().numpy().copy(), step.out.cpu().numpy().copy())


def run_both(inputs):
    """(outputs of dsa_decode_k, outputs of dsa_decode_k_noalloc) on the same
    device inputs, each into freshly poisoned output buffers."""
    step = dsa.DeviceStep(inputs)
    lens = inputs["seq_lens"]
    res = []
    for noalloc in (False, True):
        step.scores.fill_(-3.0)
        step.sel.fill_(-9)
        step.out.fill_(0x2468)
        if noalloc:
            dsa.decode_k_noalloc(step.shape, step.q_idx, step.w, step.k_normed, step.q,
                                 step.kv_cache, step.block_tables, step.seq_lens, step.kv_scale,
                                 step.sm_scale, step.scores, step.sel, step.out)
        else:
            step.decode_k()
        torch.cuda.synchronize()
        res.append(outputs(step, lens))
    return res


def assert_same(a, b, what):
    for r, (x, y) in enumerate(zip(a[0], b[0])):
        assert np.array_equal(x, y), f"{what}: scores row {r}"
    assert np.array_equal(a[1], b[1]), f"{what}: sel"
    assert np.array_equal(a[2], b[2]), f"{what}: out"


@pytest.mark.gpu
def test_noalloc_step_equals_the_workspace_step_on_two_calls():
    big = small(num_seqs=3, rows_per_seq=2, lengths="verify", base=9000, top_k=2048, seed=160)
    little = small(num_seqs=2, rows_per_seq=1, context=3000, top_k=1024, seed=161,
                   num_heads=32)
    assert dsa.workspace_bytes(dsa.shape_of(little)) < dsa.workspace_bytes(dsa.shape_of(big))
    for name, inputs in (("first call", big), ("second, smaller call", little)):
        print(f"{name}: rows {len(inputs['seq_lens'])}, lengths {inputs['seq_lens'].tolist()}",
              flush=True)
        ref, got = run_both(inputs)
        assert_same(ref, got, name)
