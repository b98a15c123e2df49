"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/dsa.h declares, sizes its workspace, and refuses bad
arguments before any HIP call."""
import ctypes
import os
import re

import pytest

from sparse_attention_decode_03_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = dsa.load()
    declared = header_functions()
    assert set(declared) == set(dsa.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def header_define(name):
    text = open(os.path.join(ROOT, "include", "dsa.h")).read()
    m = re.search(r"#define\s+" + name + r"\s+\(?([0-9u<< ]+)\)?", text)
    assert m, name
    return eval(m.group(1).replace("u", ""))


def test_binding_constants_mirror_the_header():
    # the Python side states the header's numbers, it does not guess them
    assert dsa.SELECT_DIRECT_MAX == header_define("DSA_SELECT_DIRECT_MAX")
    assert dsa.NOALLOC_SCRATCH_BYTES == header_define("DSA_NOALLOC_SCRATCH_BYTES")


def good_shape(**kw):
    f = dict(num_seqs=2, rows_per_seq=4, num_heads=64, latent_dim=512, index_heads=32,
             index_dim=128, top_k=2048, page_size=64, max_len=16388, k_capacity=16388,
             max_blocks_per_seq=257, num_pages=514)
    f.update(kw)
    return dsa.Shape(**f)


def test_workspace_bytes_grows_with_rows_and_refuses_bad_shapes():
    a = dsa.workspace_bytes(good_shape())
    b = dsa.workspace_bytes(good_shape(num_seqs=4))
    assert a > 0 and b > a and a % 256 == 0
    assert dsa.workspace_bytes(good_shape(latent_dim=256)) == 0
    assert dsa.workspace_bytes(good_shape(rows_per_seq=17)) == 0
    assert dsa.workspace_bytes(good_shape(rows_per_seq=16)) > 0
    assert dsa.workspace_bytes(good_shape(max_blocks_per_seq=10)) == 0


@pytest.mark.parametrize("field,value,code", [
    ("num_seqs", 0, dsa.DSA_EINVAL),
    ("rows_per_seq", 17, dsa.DSA_EUNSUPPORTED),
    ("latent_dim", 576, dsa.DSA_EUNSUPPORTED),
    ("num_heads", 129, dsa.DSA_EUNSUPPORTED),
    ("index_heads", 33, dsa.DSA_EUNSUPPORTED),
    ("index_dim", 96, dsa.DSA_EUNSUPPORTED),
    ("top_k", 16385, dsa.DSA_EUNSUPPORTED),
    ("max_len", (1 << 22) + 1, dsa.DSA_ERANGE),
    ("k_capacity", 100, dsa.DSA_ERANGE),
    ("max_blocks_per_seq", 256, dsa.DSA_ERANGE),
    ("page_size", 0, dsa.DSA_EINVAL),
])
def test_shape_refusals_before_launch(field, value, code):
    sh = good_shape(**{field: value})
    p = 4096  # never dereferenced: validation fails first
    rc = dsa.load().dsa_index_scores(ctypes.byref(sh), p, p, p, p, p, None)
    assert rc == code, dsa.last_error()
    assert dsa.last_error()


def test_pointer_and_workspace_refusals():
    lib = dsa.load()
    sh = good_shape()
    p = 4096
    assert lib.dsa_index_scores(ctypes.byref(sh), None, p, p, p, p, None) == dsa.DSA_EINVAL
    assert "q_idx" in dsa.last_error()
    assert lib.dsa_index_scores(ctypes.byref(sh), p + 4, p, p, p, p, None) == dsa.DSA_EINVAL
    assert "aligned" in dsa.last_error()
    need = dsa.workspace_bytes(sh)
    assert lib.dsa_topk_select(ctypes.byref(sh), p, p, p, p, need - 1, None) == dsa.DSA_EWORKSPACE
    assert lib.dsa_topk_select(ctypes.byref(sh), p, p, p, None, need, None) == dsa.DSA_EWORKSPACE
    assert lib.dsa_mla_decode(ctypes.byref(sh), p, p, p, p, p, 0.5, 0.0, p, p, need,
                              None) == dsa.DSA_EINVAL
    assert lib.dsa_decode_k(ctypes.byref(sh), p, p, p, p, p, p, p, -1.0, 0.1, p, p, p, p, need,
                            None) == dsa.DSA_EINVAL
    assert lib.dsa_decode_k(None, p, p, p, p, p, p, p, 0.5, 0.1, p, p, p, p, need,
                            None) == dsa.DSA_EINVAL


def test_bt_entries_needed_matches_the_pages_trim_tests():
    # literals of the bt_trim_tests module on the glm5next_dsa/layer.rs page:
    # the pool a whole 262,144-token context claims is 16,386 entries, past
    # the 16,384-entry buffer; a 20-token sequence verifying 3 needs 3
    assert dsa.bt_entries_needed(262_144, 0, 16) == 16_386
    assert dsa.bt_entries_needed(20, 3, 16) == 3
    assert dsa.bt_entries_needed(8, 1, 0) == 11
    assert dsa.bt_entries_needed(16_384, 4, 16) <= 16_384
    for seq_len, k, bs in [(0, 1, 16), (1, 1, 16), (15, 1, 16), (16, 1, 16), (17, 4, 16),
                           (4095, 4, 16), (131_072, 3, 16), (262_143, 4, 16), (1000, 1, 64)]:
        n = dsa.bt_entries_needed(seq_len, k, bs)
        highest = max(seq_len + k - 1, 0) // bs
        assert highest < n


def test_pooled_helpers_size_by_pools_and_refuse_bad_pool_sizes():
    sh = good_shape()
    # pool scores rows are max_len / kp pools, rounded up to 64 floats
    assert dsa.pool_score_stride(sh, 1) == dsa.score_stride(sh)
    assert dsa.pool_score_stride(sh, 4) == (16388 // 4 + 63) // 64 * 64
    assert dsa.pooled_workspace_bytes(sh, 4) > 0
    assert dsa.pooled_workspace_bytes(sh, 0) == 0
    assert dsa.pooled_workspace_bytes(sh, 1025) == 0
    # a pool longer than every row still has a layout (rows keep their tails)
    assert dsa.pooled_workspace_bytes(good_shape(max_len=100, k_capacity=100), 512) > 0


# ---------------------------------------------------------------------------
# dsa_check_metadata on host arrays (through the C ABI; no device touched)

def meta_case():
    import numpy as np
    sh = dsa.Shape(num_seqs=2, rows_per_seq=2, num_heads=8, latent_dim=512, index_heads=4,
                   index_dim=64, top_k=4, page_size=4, max_len=10, k_capacity=10,
                   max_blocks_per_seq=3, num_pages=6)
    lens = np.array([9, 10, 3, 4], np.int32)
    bt = np.array([[5, 0, 2], [4, -1, -1]], np.int32)     # sequence 1 reaches one page
    sel = np.array([[0, 3, 7, 8], [1, 2, 5, 9], [0, 1, 2, -1], [0, 1, 2, 3]], np.int32)
    return sh, lens, bt, sel


def test_check_metadata_accepts_in_contract_metadata():
    sh, lens, bt, sel = meta_case()
    dsa.check_metadata(sh, lens, bt, sel)
    dsa.check_metadata(sh, lens, bt)          # without a selection


@pytest.mark.parametrize("what,edit,needle", [
    ("length past max_len", lambda l, b, s: l.__setitem__(1, 11), "seq_lens[1] = 11"),
    ("negative length", lambda l, b, s: l.__setitem__(2, -1), "seq_lens[2] = -1"),
    ("reachable page unmapped", lambda l, b, s: b.__setitem__((0, 2), -1), "block_tables[0][2] = -1"),
    ("reachable page past the pool", lambda l, b, s: b.__setitem__((1, 0), 6), "block_tables[1][0] = 6"),
    ("id past the row's length", lambda l, b, s: s.__setitem__((2, 2), 3), "sel[2][2] = 3"),
    ("negative id", lambda l, b, s: s.__setitem__((0, 0), -1), "sel[0][0] = -1"),
    ("id twice", lambda l, b, s: s.__setitem__((3, 3), 2), "more than once"),
    ("padding not -1", lambda l, b, s: s.__setitem__((2, 3), 0), "padding"),
])
def test_check_metadata_names_the_first_violation(what, edit, needle):
    sh, lens, bt, sel = meta_case()
    edit(lens, bt, sel)
    with pytest.raises(dsa.DsaError) as e:
        dsa.check_metadata(sh, lens, bt, sel)
    assert e.value.code == dsa.DSA_EMETADATA, what
    assert needle in e.value.message, (what, e.value.message)


def test_check_metadata_ignores_unreachable_entries_and_counts_violations():
    sh, lens, bt, sel = meta_case()
    bt[1, 1:] = 99                 # past the pages sequence 1 reaches: never read
    dsa.check_metadata(sh, lens, bt, sel)
    bt[0, :] = 99                  # three reachable entries out of the pool
    with pytest.raises(dsa.DsaError) as e:
        dsa.check_metadata(sh, lens, bt, sel)
    assert e.value.message.startswith("3 out-of-contract values")
    lib = dsa.load()
    assert lib.dsa_check_metadata(ctypes.byref(sh), None, 4096, None, 1, None) == dsa.DSA_EINVAL
    assert lib.dsa_check_metadata(ctypes.byref(sh), 4096, 4096, None, 7, None) == dsa.DSA_EINVAL
