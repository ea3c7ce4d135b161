"""The C-ABI library loads and exports every function include/tsd.h declares; host-side
validation works without a GPU (CPU only: no kernel is launched)."""
import ctypes
import os
import re

import pytest

from quantized_gemv_kv_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared():
    src = open(os.path.join(ROOT, "include", "tsd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tsd_[a-z_0-9]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    names = declared()
    assert len(names) >= 18
    lib = ctypes.CDLL(binding.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(binding.EXPORTS) == names


def test_workspace_sizes_and_validation():
    c3 = synth.config("gpt2_medium_q4_0")
    n = binding.tsd_workspace_bytes(c3)
    # packed weights + fp16 cache + embedding tables + the prompt pass's row buffers (up to 4,096
    # rows) fit in a few hundred MB
    assert 300e6 < n < 380e6
    for bad, status in [(dict(c3, d_model=1000), 1), (dict(c3, n_head=15), 1), (dict(c3, head_dim=32, n_head=32, n_kv_head=32), 2),
                        (dict(c3, batch=3), 2), (dict(c3, wfmt="aff8", d_ff=4000), 1)]:
        with pytest.raises(binding.TsdError) as e:
            binding.tsd_workspace_bytes(bad)
        assert e.value.status == status, bad
    with pytest.raises(binding.TsdError):
        binding.tsd_gemv_packed_bytes("q8_0", 8, 100)
    assert binding.tsd_gemv_packed_bytes("q4_0", 3072, 1024) >= 3072 * 512 + 3072 * 32 * 2


def test_new_formats_workspace_and_validation():
    c3 = synth.config("gpt2_medium_q4_0")
    n4 = binding.tsd_workspace_bytes(c3)
    # Q5_0 adds a fifth-bit word per 32 weights; 4-bit affine adds a bias per group
    n5 = binding.tsd_workspace_bytes(dict(c3, wfmt="q5_0"))
    assert n4 < n5 < n4 * 1.2
    for f in ("aff4_g64", "aff4_g32"):
        assert n4 <= binding.tsd_workspace_bytes(dict(c3, wfmt=f)) < n4 * 1.2
    assert binding.tsd_gemv_packed_bytes("q5_0", 3072, 1024) >= 3072 * (512 + 32 * 2 + 32 * 4)
    assert binding.tsd_gemv_packed_bytes("aff4_g32", 3072, 1024) >= 3072 * (512 + 32 * 4)
    with pytest.raises(binding.TsdError):
        binding.tsd_gemv_packed_bytes("aff4_g64", 8, 96)       # K not a multiple of the group
    with pytest.raises(binding.TsdError) as e:
        binding.tsd_workspace_bytes(dict(synth.config("talker_cp_aff8"), wfmt="aff4_g64"))
    assert e.value.status == 2                                 # the batched frame is affine-8 only


def test_talker_workspace_and_validation():
    c5 = synth.config("talker_cp_aff8")
    n = binding.tsd_workspace_bytes(c5)
    # ~0.6 GB of packed weights, 0.14 GB of embedding tables, 0.94 GB of fp16 Talker cache
    assert 1.5e9 < n < 2.0e9
    for bad, status in [(dict(c5, wfmt="q8_0"), 2), (dict(c5, batch=17), 2), (dict(c5, n_codebooks=1), 1),
                        (dict(c5, n_codebooks=17), 1), (dict(c5, head_dim=96), 2), (dict(c5, cp_n_layer=0), 1),
                        (dict(c5, d_ff=8192), 2)]:
        with pytest.raises(binding.TsdError) as e:
            binding.tsd_workspace_bytes(bad)
        assert e.value.status == status, bad
    assert binding.tsd_gemm_rows_scratch_bytes(1024, 3072, 4) >= 4 * 16 * 1024 * 4      # the split-K slices


def test_debug_gemv_host_validation():
    """tsd_debug_gemv rejects bad arguments on the host, before anything reaches the device."""
    lib = binding.lib()
    one = ctypes.c_void_p(1)
    cases = [(0, None, 18, one, one, 1, 32, 1),       # null weights
             (9, one, 18, one, one, 1, 32, 1),        # unknown format
             (0, one, 18, one, one, 1, 48, 1),        # K not a multiple of 32
             (2, one, 96 + 4, one, one, 1, 96, 1),    # affine-8: K not a multiple of 64
             (0, one, 17, one, one, 1, 32, 1),        # not the canonical size of 1 x 32 Q4_0
             (1, one, 34, one, one, 1, 32, 0)]        # no batch rows
    for fmt, w, nb, x, y, N, K, B in cases:
        rc = lib.tsd_debug_gemv(fmt, w, nb, x, y, N, K, B, None)
        assert rc == 1, (fmt, nb, N, K, B)
