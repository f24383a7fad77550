"""The C-ABI library loads, exports every symbol include/dsa.h declares, and rejects bad
arguments on the host before touching the GPU (CPU only: no compute calls)."""
import ctypes
import os
import re

import pytest

import long_context_sparse_06_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

needs_lib = pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="libdsa.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_entry_points():
    names = declared_functions()
    for n in ("dsa_index_scores", "dsa_topk", "dsa_sparse_mla_decode", "dsa_sparse_mla_prefill",
              "dsa_cache_append"):
        assert n in names
    assert sorted(dsa.exported_symbols()) == names


@needs_lib
def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(dsa.LIB_PATH)
    for n in declared_functions():
        assert hasattr(L, n), n


@needs_lib
def test_status_strings():
    assert dsa.dsa_status_string(0) == "DSA_OK"
    assert dsa.dsa_status_string(4) == "DSA_ERR_WORKSPACE"
    assert dsa.dsa_status_string(99) == "DSA_ERR_UNKNOWN"


@needs_lib
def test_host_validation_paths():
    L = dsa.lib()
    FAKE = 0x1000  # never dereferenced: validation fails first
    c = dsa._Cache(FAKE, None, None, 0, 0, 1024)
    # index scores
    assert L.dsa_index_scores(dsa.E4M3, None, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, FAKE, 1024, None) == 1
    assert L.dsa_index_scores(dsa.BF16, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, FAKE, 1024, None) == 3
    assert L.dsa_index_scores(dsa.E4M3, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 0, 64, 128, FAKE, 1024, None) == 2
    assert L.dsa_index_scores(dsa.E4M3, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, FAKE, 512, None) == 2
    bad = dsa._Cache(FAKE, None, FAKE, 0, 10, 0)   # paged with page_size 0
    assert L.dsa_index_scores(dsa.E4M3, FAKE, None, FAKE, ctypes.byref(bad), FAKE, FAKE, 4, 64, 128, FAKE, 1024, None) == 2
    assert L.dsa_index_scores(dsa.F32, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 200, 100, FAKE, 1024, None) == 6
    # top-k
    assert L.dsa_topk(None, 1024, FAKE, 4, 16, FAKE, None, 0, None) == 1
    assert L.dsa_topk(FAKE, 1024, FAKE, 4, 0, FAKE, None, 0, None) == 2
    assert L.dsa_topk(FAKE, 1024, FAKE, 4, 20000, FAKE, None, 0, None) == 2
    need = L.dsa_topk_workspace_size(4, 131072, 2048)
    assert need > 0 and L.dsa_topk_workspace_size(4, 1024, 2048) == 0
    assert L.dsa_topk(FAKE, 131072, FAKE, 4, 2048, FAKE, None, 0, None) == 4
    assert L.dsa_topk(FAKE, 131072, FAKE, 4, 2048, FAKE, FAKE, need - 1, None) == 4
    # sparse MLA
    kv = dsa._Cache(FAKE, None, None, 0, 0, 4096)
    assert L.dsa_sparse_mla_decode(dsa.BF16, None, ctypes.byref(kv), FAKE, 8, 128, 576, 512, 2048, 0.04, FAKE, None, None, 0, None) == 1
    assert L.dsa_sparse_mla_decode(dsa.E4M3, FAKE, ctypes.byref(kv), FAKE, 8, 128, 576, 512, 2048, 0.04, FAKE, None, None, 0, None) == 3
    assert L.dsa_sparse_mla_decode(dsa.BF16, FAKE, ctypes.byref(kv), FAKE, 8, 128, 576, 600, 2048, 0.04, FAKE, None, None, 0, None) == 2
    mw = L.dsa_sparse_mla_decode_workspace_size(8, 128, 512, 2048)
    assert mw > 0
    assert L.dsa_sparse_mla_decode(dsa.BF16, FAKE, ctypes.byref(kv), FAKE, 8, 128, 576, 512, 2048, 0.04, FAKE, None, FAKE, mw - 1, None) == 4
    assert L.dsa_sparse_mla_prefill(dsa.BF16, FAKE, FAKE, FAKE, 0, 128, 576, 512, 2048, 0.04, FAKE, None, None) == 2
    assert L.dsa_sparse_mla_prefill(dsa.F32, FAKE, FAKE, FAKE, 16, 4, 2000, 64, 32, 0.1, FAKE, None, None) == 6
    # a prefill row's whole kept set sits in one bf16 workgroup: k <= 8192
    assert L.dsa_sparse_mla_prefill(dsa.BF16, FAKE, FAKE, FAKE, 16, 128, 576, 512, 8193, 0.04, FAKE, None, None) == 6
    # generic kernel: logits of one (row, head) plus the query row in 64 KB of LDS
    assert L.dsa_sparse_mla_decode(dsa.F32, FAKE, ctypes.byref(kv), FAKE, 8, 128, 576, 512, 16000, 0.04, FAKE, None, None, 0, None) == 6
    # split plan, read back from the workspace size (B * splits * H partial rows of 512 bf16
    # values + (max, sum)): ~256 workgroups at batch 8 (64 heads each); from 64 sequences on
    # the 128-head kernel, again ~256 workgroups; no workgroup holds more than 8192 kept tokens
    part = 512 * 2 + 8
    assert mw == 8 * 16 * 128 * part
    assert L.dsa_sparse_mla_decode_workspace_size(32, 128, 512, 2048) == 32 * 4 * 128 * part
    assert L.dsa_sparse_mla_decode_workspace_size(64, 128, 512, 2048) == 64 * 4 * 128 * part
    assert L.dsa_sparse_mla_decode_workspace_size(128, 128, 512, 2048) == 128 * 2 * 128 * part
    assert L.dsa_sparse_mla_decode_workspace_size(256, 128, 512, 2048) == 0       # one split
    assert L.dsa_sparse_mla_decode_workspace_size(128, 128, 512, 16384) == 128 * 2 * 128 * part
    assert L.dsa_sparse_mla_decode_workspace_size(512, 128, 512, 9000) == 512 * 2 * 128 * part
    # the no-allocation decode: same validation, plus the static array's size limit (checked on
    # the host before the array is looked up)
    assert L.dsa_noalloc_scratch_bytes() == 32 << 20
    assert L.dsa_sparse_mla_decode_noalloc(dsa.BF16, None, ctypes.byref(kv), FAKE, 8, 128, 576, 512, 2048, 0.04, FAKE, None, None) == 1
    assert L.dsa_sparse_mla_decode_noalloc(dsa.BF16, FAKE, ctypes.byref(kv), FAKE, 0, 128, 576, 512, 2048, 0.04, FAKE, None, None) == 2
    assert L.dsa_sparse_mla_decode_workspace_size(128, 128, 512, 16384) > L.dsa_noalloc_scratch_bytes()
    assert L.dsa_sparse_mla_decode_noalloc(dsa.BF16, FAKE, ctypes.byref(kv), FAKE, 128, 128, 576, 512, 16384, 0.04, FAKE, None, None) == 4
    # fused index + top-k
    fw = L.dsa_index_topk_workspace_size(4, 131072, 2048)
    assert fw > 4 * 131072 * 4
    assert L.dsa_index_topk(dsa.E4M3, None, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, 2048, FAKE, FAKE, fw, None) == 1
    assert L.dsa_index_topk(dsa.E4M3, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, 0, FAKE, FAKE, fw, None) == 2
    assert L.dsa_index_topk(dsa.BF16, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, 2048, FAKE, FAKE, fw, None) == 3
    need = L.dsa_index_topk_workspace_size(4, 1024, 2048)
    assert L.dsa_index_topk(dsa.E4M3, FAKE, None, FAKE, ctypes.byref(c), FAKE, FAKE, 4, 64, 128, 2048, FAKE, FAKE, need - 1, None) == 4
    # indexer-quality diagnostic
    qw = L.dsa_indexer_quality_workspace_size(8, 128, 4096)
    assert qw >= 8 * 128 * 4096 * 4
    assert L.dsa_indexer_quality(None, ctypes.byref(kv), FAKE, 4096, FAKE, FAKE, FAKE, 8, 128, 576, 2048, 0.04, FAKE, FAKE, None, FAKE, qw, None) == 1
    assert L.dsa_indexer_quality(FAKE, ctypes.byref(kv), FAKE, 4096, FAKE, FAKE, FAKE, 8, 120, 576, 2048, 0.04, FAKE, FAKE, None, FAKE, qw, None) == 6
    assert L.dsa_indexer_quality(FAKE, ctypes.byref(kv), FAKE, 1024, FAKE, FAKE, FAKE, 8, 128, 576, 2048, 0.04, FAKE, FAKE, None, FAKE, qw, None) == 2
    assert L.dsa_indexer_quality(FAKE, ctypes.byref(kv), FAKE, 4096, FAKE, FAKE, FAKE, 8, 128, 576, 2048, 0.04, FAKE, FAKE, None, FAKE, qw - 1, None) == 4
    # cache append
    ks = dsa._Cache(FAKE, FAKE, None, 0, 0, 1024)
    noscale = dsa._Cache(FAKE, None, None, 0, 0, 1024)
    assert L.dsa_cache_append(FAKE, FAKE, FAKE, FAKE, 4, 128, 576, ctypes.byref(noscale), ctypes.byref(kv), None) == 1
    assert L.dsa_cache_append(None, FAKE, FAKE, FAKE, 4, 128, 576, ctypes.byref(ks), ctypes.byref(kv), None) == 1
    assert L.dsa_cache_append(FAKE, FAKE, FAKE, FAKE, 0, 128, 576, ctypes.byref(ks), ctypes.byref(kv), None) == 2
    assert L.dsa_cache_append(FAKE, FAKE, FAKE, FAKE, 4, 8192, 576, ctypes.byref(ks), ctypes.byref(kv), None) == 2
    assert L.dsa_cache_append(FAKE, FAKE, FAKE, FAKE, 4, 128, 576, ctypes.byref(ks), ctypes.byref(bad), None) == 2

    # read probe (measurement only)
    assert L.dsa_read_probe_sink_words() > 0
    assert L.dsa_read_probe(None, 1024, FAKE, None) == 1
    assert L.dsa_read_probe(FAKE, 1024, None, None) == 1
    assert L.dsa_read_probe(FAKE, 1000, FAKE, None) == 2
    assert L.dsa_read_probe(FAKE, 0, FAKE, None) == 2
    assert L.dsa_read_probe(FAKE + 4, 1024, FAKE, None) == 2


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(dsa, "LIB_PATH", "/nonexistent/libdsa.so")
    monkeypatch.setattr(dsa, "_lib", None)
    with pytest.raises(dsa.DSALibraryMissing):
        dsa.lib()
