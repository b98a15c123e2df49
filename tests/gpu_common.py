"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
on seeded workloads and compare with the CPU oracle.

Attention is checked against two bounds per element:
  - the contract, |g - o| <= 2e-2 absolute;
  - a bound derived from the kernel's own arithmetic (the tighter one):
      |g - o| <= 2^-9 |o| + (2^-9 + 2^-9 + 2^-12) E,   E = sum_j p_j |c_j|
    2^-9 |o| is the final bf16 rounding of the output (round to nearest even
    with 8 significant bits); the first 2^-9 E bounds the bf16 rounding of
    every probability before the P.V product (each p_j moves by at most
    2^-9 p_j, so the output moves by at most 2^-9 sum_j p_j |c_j|); the
    second 2^-9 E bounds the bf16 rounding of the per-chunk partial outputs
    before the merge (each partial is a sum of p_j c_j over its chunk, so
    its rounding moves the output by at most 2^-9 times the chunk's share
    of E); 2^-12 E budgets the fp32 accumulation and exponentials. E comes
    from the oracle (oracle.mla_decode_abs).
"""
import numpy as np
import torch

import oracle
from sparse_attention_decode_03_amd import dsa
from sparse_attention_decode_03_amd import workloads as wl

SCORE_RTOL = 1e-3        # relative, per element
SCORE_ROW_FLOOR = 1e-6   # times the row's largest |score|, for exact zeros
ATT_ATOL = 2e-2          # absolute, per element, against the fp64 oracle
ATT_OUT_REL = 2.0 ** -9  # final bf16 rounding of the output
ATT_SCALE_REL = 2.0 ** -9 + 2.0 ** -9 + 2.0 ** -12  # P and partial roundings, fp32 budget
SEL_NEAR_TIE_REL = 1e-6  # end-to-end mode: a selection may differ only this close to the cut


def bf16_codes_to_f64(codes: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(codes).view(np.int16)).view(
        torch.bfloat16).double().numpy()


def run_step(inputs: dict, **shape_over) -> dsa.DeviceStep:
    step = dsa.DeviceStep(inputs, **shape_over)
    step.decode_k()
    torch.cuda.synchronize()
    return step


def host(step: dsa.DeviceStep):
    scores = step.scores.cpu().numpy()
    sel = step.sel.cpu().numpy()
    out = bf16_codes_to_f64(step.out.cpu().numpy().view(np.uint16))
    return scores, sel, out


def oracle_row_scores(inputs, r):
    K = inputs["rows_per_seq"]
    s = r // K
    L = int(inputs["seq_lens"][r])
    return oracle.index_scores(inputs["q_idx"][r:r + 1], inputs["w"][r:r + 1],
                               inputs["k_normed"][s:s + 1], inputs["seq_lens"][r:r + 1], 1, L)[0]


def check_scores(inputs, gpu_scores, rows):
    """Scores within tolerance on [0, L_r). Returns {row: oracle fp64 scores}
    and the largest error relative to the tolerance."""
    refs = {}
    worst = 0.0
    for r in rows:
        L = int(inputs["seq_lens"][r])
        ref = oracle_row_scores(inputs, r)
        got = gpu_scores[r, :L].astype(np.float64)
        tol = SCORE_RTOL * np.abs(ref) + SCORE_ROW_FLOOR * (np.abs(ref).max() if L else 0.0)
        err = np.abs(got - ref)
        bad = err > tol
        assert not bad.any(), f"row {r}: {bad.sum()} scores out of tolerance, first at {np.argmax(bad)}"
        if L:
            worst = max(worst, float((err / np.maximum(tol, 1e-300)).max()))
        refs[r] = ref
    return refs, worst


def check_selection(inputs, gpu_scores, gpu_sel, rows):
    """Exact: the oracle's selector run on the GPU's own fp32 scores."""
    top_k = inputs["top_k"]
    for r in rows:
        L = int(inputs["seq_lens"][r])
        ref = oracle.topk_row(gpu_scores[r, :L].astype(np.float64), L, top_k)
        np.testing.assert_array_equal(gpu_sel[r], ref, err_msg=f"row {r}")


def check_selection_end_to_end(inputs, ref_scores, gpu_sel, rows):
    """The oracle's own selection on its own fp64 scores against the GPU's.
    A row may differ only in tokens whose fp64 score lies within 1e-6
    relative of the row's cut (the min(top_k, L)-th largest score). Returns
    the number of rows that differ."""
    top_k = inputs["top_k"]
    differ = 0
    for r in rows:
        L = int(inputs["seq_lens"][r])
        s64 = ref_scores[r]
        ref = oracle.topk_row(s64, L, top_k)
        if np.array_equal(ref, gpu_sel[r]):
            continue
        differ += 1
        cut = np.sort(s64)[::-1][min(top_k, L) - 1]
        moved = np.setxor1d(ref[ref >= 0], gpu_sel[r][gpu_sel[r] >= 0])
        dist = np.abs(s64[moved] - cut)
        assert (dist <= SEL_NEAR_TIE_REL * abs(cut)).all(), (
            f"row {r}: {len(moved)} tokens differ from the fp64 selection, up to "
            f"{dist.max() / abs(cut):.3g} relative from the cut")
    return differ


def assert_attention_row(inputs, r, sel_row, got):
    """Row r of the GPU output against the oracle's attention over the ids
    sel_row (its first min(len(sel_row), L_r) entries), within both bounds.
    Returns (largest absolute error, largest error relative to the derived
    bound)."""
    K = inputs["rows_per_seq"]
    s = r // K
    args = (inputs["q"][r:r + 1], inputs["kv_cache"], inputs["block_tables"][s:s + 1],
            inputs["seq_lens"][r:r + 1], np.ascontiguousarray(sel_row, np.int32)[None],
            inputs["kv_scale"], inputs["sm_scale"], 1)
    ref = oracle.mla_decode(*args)[0]
    scale = oracle.mla_decode_abs(*args)[0]
    err = np.abs(got - ref)
    assert err.max() <= ATT_ATOL, f"row {r}: max abs error {err.max():.3g}"
    bound = ATT_OUT_REL * np.abs(ref) + ATT_SCALE_REL * scale
    over = err > bound
    assert not over.any(), (
        f"row {r}: {over.sum()} elements past the derived bound, worst "
        f"{(err / np.maximum(bound, 1e-300)).max():.3g}x at |o| "
        f"{np.abs(ref).flat[np.argmax(err - bound)]:.3g}")
    nz = bound > 0
    rel = float((err[nz] / bound[nz]).max()) if nz.any() else 0.0
    return float(err.max()), rel


def check_attention(inputs, gpu_sel, gpu_out, rows):
    """Within both bounds: the oracle's attention over the GPU's own
    selection. Returns (largest absolute error, largest error relative to the
    derived bound)."""
    worst_abs = worst_rel = 0.0
    for r in rows:
        a, b = assert_attention_row(inputs, r, gpu_sel[r], gpu_out[r])
        worst_abs, worst_rel = max(worst_abs, a), max(worst_rel, b)
    return worst_abs, worst_rel


def small(name="small", **kw):
    return wl.make_inputs(wl.custom(name, **kw))
