"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/uno.h declares, sizes its workspaces, and rejects bad
arguments before anything is launched."""
import ctypes
import os
import re

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "uno.h")
LIB = os.path.join(ROOT, "lossless_decoding_uno_amd", "libuno.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libuno.so not built")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(uno_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    import lossless_decoding_uno_amd as U
    lib = U.load_library()
    names = _declared()
    assert set(names) == set(U.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_workspace_sizes_and_status_strings():
    import lossless_decoding_uno_amd as U
    lib = U.load_library()
    cfg = U.make_config(synth.QWEN3_8B)
    ws1 = lib.uno_workspace_bytes(ctypes.byref(cfg), 1, 16, 1024)
    ws64 = lib.uno_workspace_bytes(ctypes.byref(cfg), 64, 16, 9216)
    assert 0 < ws1 < ws64 < 4 << 30
    assert lib.uno_spec_accept_workspace_bytes(64, 16) >= 2 * 64 * 16 * 12
    assert lib.uno_status_string(0) == b"ok"
    assert lib.uno_status_string(4) == b"workspace too small"
    bad = U.make_config(dict(synth.QWEN3_8B, head_dim=96))
    assert lib.uno_workspace_bytes(ctypes.byref(bad), 1, 16, 1024) == 0


def test_entry_points_reject_bad_arguments_on_the_host():
    import lossless_decoding_uno_amd as U
    lib = U.load_library()
    cfg = U.make_config(synth.TINY)
    w = U.UnoWeights()
    kv = U.UnoKV()
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    # null anchor / logits
    assert lib.uno_draft_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), None, 1, 4,
                               64, 1.0, 0, fake, fake, fake, None, None, fake, 1 << 20,
                               None) == 1
    # K out of range
    assert lib.uno_draft_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, 1, 65,
                               64, 1.0, 0, fake, fake, fake, None, None, fake, 1 << 20,
                               None) == 1
    # bad temperature
    assert lib.uno_draft_sample(fake, None, 1, 4, 512, 0.0, 0, fake, fake, None, None) == 1
    # workspace too small
    assert lib.uno_spec_accept(fake, fake, None, None, fake, 2, 4, 512, 1.0, 0, fake, None, fake,
                               fake, fake, None, fake, 8, None) == 4
    # only one of the two row-maximum arrays
    assert lib.uno_spec_accept(fake, fake, fake, None, fake, 2, 4, 512, 1.0, 0, fake, None, fake,
                               fake, fake, None, fake, 1 << 20, None) == 1
    # the no-allocation accept step: shapes past its static scratch
    assert lib.uno_spec_accept_noalloc(fake, fake, None, None, fake, 2049, 16, 512, 1.0, 0, fake,
                                       None, fake, fake, fake, None, None) == 4
    assert lib.uno_spec_accept_noalloc(None, fake, None, None, fake, 2, 4, 512, 1.0, 0, fake,
                                       None, fake, fake, fake, None, None) == 1
    # unsupported head_dim
    bad = U.make_config(dict(synth.TINY, head_dim=48))
    assert lib.uno_verify_block(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(kv), fake, 1, 4,
                                64, 1, fake, None, None, fake, 1 << 20, None) == 2
    # unknown noise prior
    bad = U.make_config(dict(synth.TINY, noise_prior=2))
    assert lib.uno_verify_block(ctypes.byref(bad), ctypes.byref(w), ctypes.byref(kv), fake, 1, 4,
                                64, 1, fake, None, None, fake, 1 << 20, None) == 1
    # verify: empty kv struct
    assert lib.uno_verify_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, 1, 4,
                                64, 1, fake, None, None, fake, 1 << 30, None) == 1
    # verify: row maxima without logits
    assert lib.uno_verify_block(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, 1, 4,
                                64, 1, None, fake, None, fake, 1 << 30, None) == 1
    assert lib.uno_kv_commit(None, fake, 1, 4, None, None, None) == 1
    # weight packing: shapes off the 16 x 32 tile grid, aliasing
    assert lib.uno_pack_weight(fake, ctypes.c_void_p(0x2000), 24, 64, None) == 1
    assert lib.uno_pack_weight(fake, ctypes.c_void_p(0x2000), 32, 48, None) == 1
    assert lib.uno_pack_weight(fake, fake, 32, 64, None) == 1


def test_tree_entry_points_shape_rules_and_host_validation():
    import lossless_decoding_uno_amd as U
    lib = U.load_library()
    # N = 1 + n_keep (K - 1); n_keep <= min(64, topk^(K-1)); 2 <= K <= 32; topk <= 8
    assert lib.uno_tree_rows(16, 2, 8) == 1 + 8 * 15
    assert lib.uno_tree_rows(3, 2, 4) == 9
    assert lib.uno_tree_rows(3, 2, 5) == 0          # only 4 candidates
    assert lib.uno_tree_rows(2, 1, 1) == 2
    assert lib.uno_tree_rows(1, 2, 1) == 0
    assert lib.uno_tree_rows(33, 2, 1) == 0
    assert lib.uno_tree_rows(16, 9, 1) == 0
    assert lib.uno_tree_rows(16, 2, 65) == 0
    assert lib.uno_tree_rows(32, 8, 64) == 1 + 64 * 31
    assert lib.uno_tree_workspace_bytes(4, 16, 4) >= 4 * 15 * 4 * 12
    assert lib.uno_tree_workspace_bytes(4, 1, 4) == 0
    fake = ctypes.c_void_p(0x1000)   # never dereferenced: validation fails first
    cfg = U.make_config(synth.TINY)
    w, kv = U.UnoWeights(), U.UnoKV()
    # unsupported tree shape
    assert lib.uno_tree_build(fake, fake, 1, 3, 512, 2, 5, fake, fake, fake, fake, fake, None,
                              fake, 1 << 20, None) == 1
    # workspace too small
    assert lib.uno_tree_build(fake, fake, 1, 3, 512, 2, 4, fake, fake, fake, fake, fake, None,
                              fake, 8, None) == 4
    # null node arrays, empty kv struct
    assert lib.uno_verify_tree(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), None, fake,
                               fake, 1, 9, 64, fake, None, fake, 1 << 30, None) == 1
    assert lib.uno_verify_tree(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(kv), fake, fake,
                               fake, 1, 9, 64, fake, None, fake, 1 << 30, None) == 1
    # bad temperature, rows fewer than the block
    assert lib.uno_tree_accept(fake, fake, fake, fake, fake, 1, 3, 9, 512, 0.0, 0, fake, fake,
                               fake, fake, fake, fake, None, None) == 1
    assert lib.uno_tree_accept(fake, fake, fake, fake, fake, 1, 16, 9, 512, 1.0, 0, fake, fake,
                               fake, fake, fake, fake, None, None) == 1
    assert lib.uno_tree_commit(ctypes.byref(cfg), None, fake, fake, 1, 3, None, None, None) == 1


def test_device_status_bits_match_the_header():
    """The binding's device status bits are the header's UNO_DEV_* values."""
    import lossless_decoding_uno_amd as U
    hdr = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                            "include", "uno.h")).read()
    bits = {m.group(1): int(m.group(2)) for m in re.finditer(r"UNO_DEV_(\w+) = (\d+)", hdr)}
    assert bits == {"CAPACITY": U.DEV_CAPACITY, "BAD_TOKEN": U.DEV_BAD_TOKEN,
                    "BAD_PAGE": U.DEV_BAD_PAGE, "NONFINITE": U.DEV_NONFINITE,
                    "BAD_ACCEPT": U.DEV_BAD_ACCEPT, "SYNC_TIMEOUT": U.DEV_SYNC_TIMEOUT}
    assert sorted(bits.values()) == [1 << i for i in range(len(bits))]
