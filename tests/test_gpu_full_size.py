"""The four benchmark workloads at their full sizes, through dsa_decode_k in the
launch configuration the benchmark times, checked row by row against the CPU
oracle: scores within tolerance, selection exact on the GPU's own scores,
attention within tolerance over the GPU's own selection."""
import pytest

from sparse_attention_decode_03_amd import workloads as wl

from gpu_common import check_attention, check_scores, check_selection, host, run_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["single", "batched", "kverify", "long"])
def test_full_size_workload(name):
    inputs = wl.make_inputs(wl.WORKLOADS[name])
    step = run_step(inputs)
    scores, sel, out = host(step)
    rows = range(inputs["seq_lens"].shape[0])
    check_scores(inputs, scores, rows)
    check_selection(inputs, scores, sel, rows)
    check_attention(inputs, sel, out, rows)
