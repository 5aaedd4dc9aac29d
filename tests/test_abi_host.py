"""Host-side checks of the C ABI that need no GPU: the library loads, exports every
function include/csa2.h declares, and rejects invalid arguments before touching the
device (status codes of the header)."""
import ctypes
import os
import re

import pytest

import compressed_sparse_attention_csa2_amd as csa2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b(csa2_[a-z0-9_]+)\s*\(", text,
                                 flags=re.M)))


def test_library_exports_every_declared_function():
    lib = csa2.lib()
    names = _declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(csa2.EXPORTS) == names


def test_status_strings():
    for code in range(0, -8, -1):
        assert csa2.status_string(code).startswith("CSA2_")


def _p(v=1):
    return ctypes.c_void_p(0x1000 * v)  # never dereferenced: validation fails first


def test_errors_before_any_launch():
    L = csa2.lib()
    # null pointers
    assert L.csa2_quantize_kv(0, 0, 1, 1, 8, None, 0, 8, 8, None, 1, _p(), _p(), None) == -1
    # odd D for FP4
    assert L.csa2_quantize_kv(0, 0, 1, 1, 7, _p(), 0, 7, 7, None, 1, _p(), _p(), None) == -2
    # bad dtype / fmt / policy
    assert L.csa2_quantize_kv(0, 0, 1, 1, 8, _p(), 5, 8, 8, None, 1, _p(), _p(), None) == -3
    assert L.csa2_quantize_kv(9, 0, 1, 1, 8, _p(), 0, 8, 8, None, 1, _p(), _p(), None) == -3
    assert L.csa2_quantize_kv(1, 1, 1, 1, 8, _p(), 0, 8, 8, None, 1, _p(), _p(), None) == -3
    # K out of range, workspace missing
    assert L.csa2_topk(1, 1, 100, _p(), None, 0, _p(), None, _p(), 1 << 30, None) == -2
    assert L.csa2_topk(1, 1, 100, _p(), None, 4096, _p(), None, _p(), 1 << 30, None) == -2
    assert L.csa2_topk(1, 1, 100, _p(), None, 8, _p(), None, None, 0, None) == -5
    need = L.csa2_topk_workspace_size(1, 1, 100, 8)
    assert need > 0
    assert L.csa2_topk(1, 1, 100, _p(), None, 8, _p(), None, _p(), need - 1, None) == -5
    # fp8 indexer needs H == 32, dk == 64
    assert L.csa2_index_score(1, 1, 1, 16, 64, _p(), 1, _p(), _p(), _p(), 100, _p(), None, None, 0, _p(), None, 0,
                              None) == -6
    assert L.csa2_index_score(1, 1, 1, 32, 64, _p(), 1, _p(), _p(), None, 100, _p(), None, None, 0, _p(), None, 0,
                              None) == -1
    assert L.csa2_index_score(7, 1, 1, 32, 64, _p(), 1, _p(), _p(), _p(), 100, _p(), None, None, 0, _p(), None, 0,
                              None) == -3
    # attention: bf16 path needs Hq % 16 == 0 and D in {128, 256, 512}; fp32 query needs fp32 output
    assert L.csa2_sparse_attend(1, 1, 8, 512, _p(), 1, 0, _p(), _p(), 10, _p(), 8, None, 1.0, _p(), 1, None, None, 0,
                                None) == -6
    assert L.csa2_sparse_attend(1, 1, 16, 384, _p(), 1, 0, _p(), _p(), 10, _p(), 8, None, 1.0, _p(), 1, None, None, 0,
                                None) == -6
    assert L.csa2_sparse_attend(1, 1, 8, 128, _p(), 0, 0, _p(), _p(), 10, _p(), 8, None, 1.0, _p(), 1, None, None, 0,
                                None) == -3
    assert L.csa2_sparse_attend(1, 1, 16, 512, _p(), 1, 0, _p(), _p(), 10, _p(), 4096, None, 1.0, _p(), 1, None, None, 0,
                                None) == -2
    # main-KV layouts: per channel (0) or one E4M3 scale per 16 channels (2, D % 16 == 0); the
    # E4M3 per-token format (1) is not a main-KV layout
    assert L.csa2_sparse_attend(1, 1, 16, 512, _p(), 1, 1, _p(), _p(), 10, _p(), 8, None, 1.0, _p(), 1, None, None, 0,
                                None) == -3
    assert L.csa2_sparse_attend(1, 1, 8, 40, _p(), 0, 2, _p(), _p(), 10, _p(), 8, None, 1.0, _p(), 0, None, None, 0,
                                None) == -2
    # sliding window: 1 <= window <= 128, every pointer given
    for win, ptrs, code in [(0, True, -2), (129, True, -2), (16, False, -1)]:
        sw = csa2._Swa(_p() if ptrs else None, _p(), 100, _p(), win)
        assert L.csa2_sparse_attend(1, 1, 16, 512, _p(), 1, 0, _p(), _p(), 10, _p(), 8, ctypes.byref(sw), 1.0, _p(),
                                    1, None, None, 0, None) == code
    assert L.csa2_sparse_attend_workspace_size(2, 1, 64, 512, 512, 1, 0) == 0
    assert L.csa2_sparse_attend_workspace_size(2, 1, 64, 512, 512, 1, 128) >= 2 * 2 * 64 * 512 * 4
    assert L.csa2_gather_dequant(2, 1, 1, 8, 24, _p(), _p(), 10, _p(), _p(), None) == -2
    assert L.csa2_gather_dequant(5, 1, 1, 8, 32, _p(), _p(), 10, _p(), _p(), None) == -3
    assert L.csa2_quantize_kv(2, 0, 1, 1, 24, _p(), 0, 24, 24, None, 4, _p(), _p(), None) == -2


@pytest.mark.parametrize("modes,code", [
    ([2], -4), ([1, 2], -4), ([0, 2, 1, 2], None), ([0, 7], -4), ([], -4),
])
def test_layer_group_schedule_validation(modes, code):
    L = csa2.lib()
    arr = (csa2._Layer * max(1, len(modes)))()
    for i, m in enumerate(modes):
        arr[i] = csa2._Layer(m, _p(), _p(), _p(), _p(), None, _p())
    gc = csa2._GroupCache(1, 32, 64, 64, 512, 512, 1000, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04)
    rc = L.csa2_layer_group(arr, len(modes), ctypes.byref(gc), None, 0, None)
    if code is None:
        assert rc == -5  # schedule valid; fails next on the missing workspace
    else:
        assert rc == code


def test_pages_schedule_passes_validation():
    # Encoder [Full, Reuse x5] x3 and decoder [Full, Reuse x3] + [Reindex, Reuse x3] x4
    modes = ([0] + [2] * 5) * 3 + [0] + [2] * 3 + ([1] + [2] * 3) * 4
    L = csa2.lib()
    arr = (csa2._Layer * len(modes))()
    for i, m in enumerate(modes):
        arr[i] = csa2._Layer(m, _p(), _p(), _p(), _p(), None, _p())
    gc = csa2._GroupCache(1, 32, 64, 64, 512, 512, 1000, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04)
    assert L.csa2_layer_group(arr, len(modes), ctypes.byref(gc), None, 0, None) == -5


@pytest.mark.parametrize("block,blocks,code", [(8, -1, -2), (8, 2049, -2), (0, 16, -2), (8, 2048, -5), (0, 0, -5)])
def test_layer_group_pool_validation(block, blocks, code):
    L = csa2.lib()
    arr = (csa2._Layer * 2)()
    for i, m in enumerate([0, 1]):
        arr[i] = csa2._Layer(m, _p(), _p(), _p(), _p(), None, _p(), None)
    gc = csa2._GroupCache(1, 32, 64, 64, 512, 512, 1000, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04, block, blocks)
    assert L.csa2_layer_group(arr, 2, ctypes.byref(gc), None, 0, None) == code


def test_layer_group_pool_workspace_grows():
    L = csa2.lib()
    base = csa2._GroupCache(4, 32, 64, 64, 512, 512, 131072, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04)
    pooled = csa2._GroupCache(4, 32, 64, 64, 512, 512, 131072, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04, 8, 2048)
    big = csa2._GroupCache(4, 32, 64, 64, 512, 512, 1000, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04, 16, 2048)
    a = L.csa2_layer_group_workspace_size(ctypes.byref(base), 4)
    b = L.csa2_layer_group_workspace_size(ctypes.byref(pooled), 4)
    # pool positions and block maxima, plus one more selection per layer
    assert b >= a + 4 * 16384 * 4 + 4 * 16384 * 4
    # a pool wider than the cache sizes the scores and candidates for the pool
    assert L.csa2_layer_group_workspace_size(ctypes.byref(big), 4) >= 4 * 32768 * 4 * 2


def test_layer_group_noalloc_validates_and_rejects_shapes_beyond_its_scratch():
    """The no-allocation layer group returns csa2_layer_group's argument errors, and
    CSA2_ERR_WORKSPACE for a shape whose workspace exceeds the library's scratch array,
    both before any device call (so this runs without a GPU)."""
    L = csa2.lib()
    assert L.csa2_layer_group_noalloc(None, 1, None, None) == -1
    arr = (csa2._Layer * 2)()
    arr[0] = csa2._Layer(2, _p(), _p(), _p(), _p(), None, _p())  # Reuse first: invalid schedule
    arr[1] = csa2._Layer(0, _p(), _p(), _p(), _p(), None, _p())
    gc = csa2._GroupCache(16, 32, 64, 64, 512, 512, 1 << 22, _p(), _p(), _p(), _p(), _p(), 1, 1, 1, 0.04)
    assert L.csa2_layer_group_noalloc(arr, 2, ctypes.byref(gc), None) == -4
    arr[0] = csa2._Layer(0, _p(), _p(), _p(), _p(), None, _p())
    arr[1] = csa2._Layer(2, _p(), _p(), _p(), _p(), None, _p())
    assert L.csa2_layer_group_workspace_size(ctypes.byref(gc), 2) > csa2.NOALLOC_SCRATCH_BYTES
    assert L.csa2_layer_group_noalloc(arr, 2, ctypes.byref(gc), None) == -5


def test_product_path_does_not_import_oracle():
    pkg = os.path.join(ROOT, "compressed_sparse_attention_csa2_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "import oracle" not in text and "csa2_oracle" not in text and "orc_" not in text, f
