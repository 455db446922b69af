"""CPU-only checks of the C ABI boundary: the library loads, exports every
function include/moe.h declares, and its host-side validation and size
queries behave as documented (no kernel is launched here)."""
import ctypes
import os
import re

import pytest

import dispatch_grouped_gemm_moe_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 10
    assert sorted(moe.EXPORTS) == names
    lib = ctypes.CDLL(moe.build.lib_path())
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_status_strings():
    assert moe.moe_abi_version() == 2
    lib = moe.lib()
    assert lib.moe_status_string(0) == b"ok"
    assert lib.moe_status_string(3) == b"buffer too small"
    assert lib.moe_status_string(99) == b"unknown status"


@pytest.mark.parametrize("kw,want", [
    (dict(), moe.MOE_OK),
    (dict(T=0), moe.MOE_E_INVALID),
    (dict(k=9), moe.MOE_E_INVALID),  # k > E
    (dict(k=0), moe.MOE_E_INVALID),
    (dict(prec=7), moe.MOE_E_INVALID),
    (dict(flags=1 << 9), moe.MOE_E_INVALID),
    (dict(minibatch=-1), moe.MOE_E_INVALID),
    (dict(H=96), moe.MOE_E_UNSUPPORTED),
    (dict(I=32), moe.MOE_E_UNSUPPORTED),
    (dict(E=300, k=2), moe.MOE_E_UNSUPPORTED),
    (dict(E=32, k=17), moe.MOE_E_UNSUPPORTED),
    (dict(flags=moe.MOE_F_BF16_WGRAD), moe.MOE_E_INVALID),  # MXFP8 only
    (dict(flags=moe.MOE_F_BF16_WGRAD, prec=moe.MOE_PREC_MXFP8), moe.MOE_OK),
])
def test_validate_cfg(kw, want):
    base = dict(T=64, H=128, I=64, E=8, k=2)
    base.update(kw)
    assert moe.moe_validate_cfg(moe.make_cfg(**base)) == want


def test_32bit_operand_offsets_are_enforced():
    # the kernels address operand rows with 32-bit byte offsets: the token
    # matrix (T*H*2), a minibatch's padded rows (R*H*2, R*4I) and one expert's
    # weights (4*I*H) must stay below 4 GiB
    ok = moe.make_cfg(65536, 7168, 2048, 32, 8)  # automatic minibatch of 8192
    assert moe.moe_validate_cfg(ok) == moe.MOE_OK
    # 299,594 tokens of 7168 bf16 values pass 4 GiB
    assert moe.moe_validate_cfg(moe.make_cfg(299593, 7168, 2048, 32, 8, minibatch=4096)) == moe.MOE_OK
    big_t = moe.make_cfg(299594, 7168, 2048, 32, 8, minibatch=4096)
    assert moe.moe_validate_cfg(big_t) == moe.MOE_E_UNSUPPORTED
    # one minibatch of 40000 tokens at k=8: R >= 320000 padded rows, R*H*2 > 4 GiB
    big_mb = moe.make_cfg(40000, 7168, 2048, 32, 8, minibatch=40000)
    assert moe.moe_validate_cfg(big_mb) == moe.MOE_E_UNSUPPORTED
    for cfg in (big_t, big_mb):
        with pytest.raises(RuntimeError):
            moe.moe_query_sizes(cfg)
    # R = 256 * (ceil(4096 * 8 / 256) + 31) = 40704 rows: R*4I = 2^32 - ... at I = 26368
    # is over, at I = 26304 (R*4I < 2^32) under, with H small enough for the rest
    R = 256 * ((4096 * 8 + 255) // 256 + 32 - 1)
    i_over = ((1 << 32) // (4 * R) + 64) // 64 * 64
    assert R * 4 * i_over >= 1 << 32 and R * 4 * (i_over - 64) < 1 << 32
    assert moe.moe_validate_cfg(moe.make_cfg(4096, 64, i_over - 64, 32, 8, minibatch=4096)) == moe.MOE_OK
    assert moe.moe_validate_cfg(moe.make_cfg(4096, 64, i_over, 32, 8, minibatch=4096)) == moe.MOE_E_UNSUPPORTED


def test_query_sizes_h7168_i2048():
    cfg = moe.make_cfg(16384, 7168, 2048, 32, 8, minibatch=2560)
    s = moe.moe_query_sizes(cfg)
    assert s.minibatch == 2560 and s.num_minibatches == 7 and s.ring_slots == 9 and s.comm_cus == 0
    # packed: gate|up [E,2I,H] + down [E,H,I], bf16
    assert s.packed_weights >= 32 * 3 * 7168 * 2048 * 2
    # per slot the Y buffer alone holds (rows + padding) x H bf16
    assert s.workspace_fwd >= 9 * (2560 * 8) * 7168 * 2
    # explicit ring size and combine workgroups are honoured (ring at most one slot per minibatch)
    s2 = moe.moe_query_sizes(moe.make_cfg(16384, 7168, 2048, 32, 8, minibatch=2560, ring_slots=2, comm_cus=8))
    assert s2.ring_slots == 2 and s2.comm_cus == 8 and s2.workspace_fwd < s.workspace_fwd
    assert moe.moe_query_sizes(moe.make_cfg(64, 128, 64, 8, 2, ring_slots=5)).ring_slots == 1
    assert s.saved >= 16384 * 8 * 8


def test_query_sizes_automatic_minibatch_and_shared_expert():
    s = moe.moe_query_sizes(moe.make_cfg(4096, 2048, 1024, 64, 6))
    assert 1 <= s.num_minibatches <= 2 and s.minibatch * s.num_minibatches >= 4096
    # H=7168 I=2048 E=32 k=8: two waves of gate|up tiles and the balance rows come
    # at 1280 tokens, but the expected padding of the experts' last M tiles
    # (E x 128 rows) falls to a sixteenth of the rows only at 8192 tokens
    s = moe.moe_query_sizes(moe.make_cfg(16384, 7168, 2048, 32, 8))
    assert s.minibatch == 8192 and s.num_minibatches == 2
    s = moe.moe_query_sizes(moe.make_cfg(65536, 7168, 2048, 32, 8))
    assert s.minibatch == 8192 and s.num_minibatches == 8
    a = moe.moe_query_sizes(moe.make_cfg(1024, 512, 256, 8, 2))
    b = moe.moe_query_sizes(moe.make_cfg(1024, 512, 256, 8, 2, flags=moe.MOE_F_SHARED_EXPERT))
    assert b.packed_weights > a.packed_weights and b.workspace_fwd > a.workspace_fwd


def test_diag_mfma_loop_rejects_bad_arguments():
    lib = moe.lib()
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: validation fails first
    assert lib.moe_diag_mfma_loop(2, fake, 1 << 16, 256, 16, fake, fake, None) == moe.MOE_E_INVALID
    assert lib.moe_diag_mfma_loop(0, None, 1 << 16, 256, 16, fake, fake, None) == moe.MOE_E_INVALID
    assert lib.moe_diag_mfma_loop(0, fake, 1024, 256, 16, fake, fake, None) == moe.MOE_E_INVALID
    assert lib.moe_diag_mfma_loop(1, fake, 1 << 16, 0, 16, fake, fake, None) == moe.MOE_E_INVALID
    assert lib.moe_diag_mfma_loop(1, fake, 1 << 16, 256, 0, fake, fake, None) == moe.MOE_E_INVALID
    assert lib.moe_diag_mfma_loop(0, ctypes.c_void_p((1 << 20) + 8), 1 << 16, 256, 16, fake, fake,
                                  None) == moe.MOE_E_INVALID


def test_null_pointers_are_rejected_before_any_launch():
    lib = moe.lib()
    cfg = moe.make_cfg(64, 128, 64, 8, 2)
    st = lib.moe_route(ctypes.byref(cfg), None, None, None, None, None, None, None, None, None)
    assert st == moe.MOE_E_INVALID
    st = lib.moe_dispatch_layout(ctypes.byref(cfg), None, None, None, None, None, None)
    assert st == moe.MOE_E_INVALID
    st = lib.moe_layer_fwd(ctypes.byref(cfg), None, None, None, None, 0, None, 0, None)
    assert st == moe.MOE_E_INVALID
    st = lib.moe_route(None, None, None, None, None, None, None, None, None, None)
    assert st == moe.MOE_E_INVALID
    # the dispatch-quantisation outputs come as a pair, the codes 16-byte aligned
    fake = ctypes.c_void_p(1 << 20)
    st = lib.moe_route(ctypes.byref(cfg), fake, fake, None, fake, fake, None, fake, None, None)
    assert st == moe.MOE_E_INVALID
    st = lib.moe_route(ctypes.byref(cfg), fake, fake, None, fake, fake, None, ctypes.c_void_p((1 << 20) + 8),
                       fake, None)
    assert st == moe.MOE_E_INVALID


def test_small_buffers_are_rejected():
    lib = moe.lib()
    cfg = moe.make_cfg(64, 128, 64, 8, 2)
    s = moe.moe_query_sizes(cfg)
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced: the size check fails first
    w = moe.moe_weights(fake.value, None, fake.value, s.packed_weights)
    st = lib.moe_layer_fwd(ctypes.byref(cfg), ctypes.byref(w), fake, fake, None, 0, fake,
                           s.workspace_fwd - 1, None)
    assert st == moe.MOE_E_WORKSPACE
    w.packed_bytes = s.packed_weights - 1
    st = lib.moe_layer_fwd(ctypes.byref(cfg), ctypes.byref(w), fake, fake, None, 0, fake,
                           s.workspace_fwd, None)
    assert st == moe.MOE_E_WORKSPACE
    st = lib.moe_prepare_weights(ctypes.byref(cfg), fake, fake, fake, None, None, None, fake,
                                 s.packed_weights - 1, None)
    assert st == moe.MOE_E_WORKSPACE
    # the shared expert needs its three weights
    cfg_s = moe.make_cfg(64, 128, 64, 8, 2, flags=moe.MOE_F_SHARED_EXPERT)
    st = lib.moe_prepare_weights(ctypes.byref(cfg_s), fake, fake, fake, None, None, None, fake,
                                 1 << 40, None)
    assert st == moe.MOE_E_INVALID


def test_misaligned_pointers_are_rejected():
    lib = moe.lib()
    cfg = moe.make_cfg(64, 128, 64, 8, 2)
    s = moe.moe_query_sizes(cfg)
    good = (1 << 20)
    w = moe.moe_weights(good, None, good, s.packed_weights)
    st = lib.moe_layer_fwd(ctypes.byref(cfg), ctypes.byref(w), ctypes.c_void_p(good + 2),
                           ctypes.c_void_p(good), None, 0, ctypes.c_void_p(good), s.workspace_fwd, None)
    assert st == moe.MOE_E_INVALID
