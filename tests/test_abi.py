"""CPU checks of the C ABI library: it loads, exports every symbol include/gq8.h declares, and
its host-only functions (sizes, status strings, argument checks that return before any device
work) behave as documented. No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gq8.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gq8_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    from gemm_q8_amd import gq8
    return gq8


def test_library_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) >= 20
    raw = ctypes.CDLL(lib.LIB_PATH)
    missing = [n for n in names if not hasattr(raw, n)]
    assert not missing, missing
    # the binding wraps each one under the same name
    assert not [n for n in names if not hasattr(lib, n)]


def test_status_strings_and_version(lib):
    assert lib.gq8_abi_version() == 3
    assert lib.gq8_status_str(0) == "ok"
    assert lib.gq8_status_str(-4).startswith("workspace")
    assert lib.gq8_status_str(12345) == "unknown status"


def test_q8_0_bytes(lib):
    assert lib.gq8_q8_0_bytes(1024, 4096) == 4_456_448
    assert lib.gq8_q8_0_bytes(320, 16384) == 5_570_560
    assert lib.gq8_q8_0_bytes(16384, 320) == 5_570_560
    assert lib.gq8_q8_0_bytes(3, 33) == 0            # K not a multiple of 32


def test_w8a8_packed_bytes_pads_to_fragments(lib):
    assert lib.gq8_w8a8_packed_bytes(4096, 1536) == 4096 * 1536
    assert lib.gq8_w8a8_packed_bytes(80, 17) == 128 * 32


def test_workspace_sizes(lib):
    # only the down read (split over K slabs) and the routed experts need a workspace
    assert lib.gq8_workspace_bytes(lib.OP_HC_DOWN, 1, 320, 16384) >= (16384 // 512) * 320 * 4
    assert lib.gq8_workspace_bytes(lib.OP_HC_DOWN, 6, 320, 16384) > \
        lib.gq8_workspace_bytes(lib.OP_HC_DOWN, 1, 320, 16384)
    for op, rows, n, k in [(lib.OP_Q8_0_GEMV, 1, 1024, 4096), (lib.OP_HC_UP, 4, 16384, 320),
                           (lib.OP_W8A8, 16, 1536, 4096), (99, 1, 1, 32)]:
        assert lib.gq8_workspace_bytes(op, rows, n, k) == 0
        assert lib.gq8_workspace_counter_bytes(op, rows, n, k) == 0
    # the split reads open their workspace with one arrival counter per 64-row group (the
    # last-arriver combine), inside gq8_workspace_bytes: 256 bytes for every N <= 4096
    for op, rows, n, k in [(lib.OP_HC_DOWN, 4, 320, 16384), (lib.OP_HC_PAIR, 16, 320, 16384),
                           (lib.OP_Q8_0_GEMV, 8, 1024, 4096)]:
        cb = lib.gq8_workspace_counter_bytes(op, rows, n, k)
        assert cb >= 4 * ((n + 63) // 64) and cb % 256 == 0
        assert lib.gq8_workspace_bytes(op, rows, n, k) > cb
        assert cb == (256 if n <= 4096 else -(-4 * ((n + 63) // 64) // 256) * 256)
    assert lib.gq8_workspace_counter_bytes(lib.OP_HC_DOWN, 1, 4160, 64) == 512
    # the GEMV takes a workspace from T = 5 on (MFMA over slabs, then a combine)
    assert lib.gq8_workspace_bytes(lib.OP_Q8_0_GEMV, 4, 1024, 4096) == 0
    assert lib.gq8_workspace_bytes(lib.OP_Q8_0_GEMV, 8, 1024, 4096) >= 8 * 8 * 1024 * 4
    assert lib.gq8_moe_plan_words(4, 8) == 1 + 4 * 32
    assert lib.gq8_moe_workspace_bytes(4, 8, 2048, 512) > 32 * (2048 + 512) * 4


def test_argument_checks_return_before_device_work(lib):
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced: every case below fails validation first
    # K not a multiple of 32
    assert raw.gq8_q8_0_gemv(dummy, dummy, dummy, 1, 8, 48, None, 0, None) == lib.ESHAPE
    # T above 16
    assert raw.gq8_q8_0_gemv(dummy, dummy, dummy, 17, 8, 64, None, 0, None) == lib.ESHAPE
    # negative size
    assert raw.gq8_hc_q8_down(dummy, dummy, dummy, 1e-6, dummy, None, -1, 8, 64, None, 0, None) == lib.EINVAL
    # up read with K above 1024
    assert raw.gq8_hc_q8_up(dummy, dummy, dummy, 1, 8, 2048, None, 0, None) == lib.ESHAPE
    # W8A8 M above 32, K not a multiple of 16
    assert raw.gq8_w8a8_gemm(dummy, dummy, dummy, dummy, dummy, 33, 16, 64, None, 0, None) == lib.ESHAPE
    assert raw.gq8_w8a8_gemm(dummy, dummy, dummy, dummy, dummy, 4, 16, 40, None, 0, None) == lib.ESHAPE
    # misaligned weight pointer
    assert raw.gq8_q8_0_gemv(dummy + 4, dummy, dummy, 1, 8, 64, None, 0, None) == lib.EALIGN
    # missing / short workspace for the split down read
    assert raw.gq8_hc_q8_down(dummy, dummy, dummy, 1e-6, dummy, None, 1, 320, 16384, None, 0, None) == lib.EWORKSPACE
    assert raw.gq8_hc_q8_down(dummy, dummy, dummy, 1e-6, dummy, None, 1, 320, 16384, dummy, 64, None) == lib.EWORKSPACE
    # GEMV at T >= 5 without its workspace
    assert raw.gq8_q8_0_gemv(dummy, dummy, dummy, 8, 64, 4096, None, 0, None) == lib.EWORKSPACE
    # W8A8 depth limit
    assert raw.gq8_w8a8_gemm(dummy, dummy, dummy, dummy, dummy, 4, 16, 8192 + 16, None, 0, None) == lib.ESHAPE
    # empty calls are no-ops
    assert raw.gq8_q8_0_gemv(None, None, None, 0, 8, 64, None, 0, None) == lib.OK
    assert raw.gq8_w8a8_gemm(None, None, None, None, None, 0, 16, 64, None, 0, None) == lib.OK
    # null output
    assert raw.gq8_q8_0_gemv(dummy, dummy, None, 1, 8, 64, None, 0, None) == lib.EINVAL
    # down/up pair: depth above 1024, depth not a multiple of 32, missing lo, short workspace
    assert raw.gq8_hc_q8_pair(dummy, dummy, dummy, 1e-6, dummy, dummy, None, dummy, 1, 2048, 4096,
                              None, 0, None) == lib.ESHAPE
    assert raw.gq8_hc_q8_pair(dummy, dummy, dummy, 1e-6, dummy, dummy, None, dummy, 1, 48, 4096,
                              None, 0, None) == lib.ESHAPE
    assert raw.gq8_hc_q8_pair(dummy, dummy, dummy, 1e-6, dummy, None, None, dummy, 1, 320, 4096,
                              None, 0, None) == lib.EINVAL
    assert raw.gq8_hc_q8_pair(dummy, dummy, dummy, 1e-6, dummy, dummy, None, dummy, 1, 320, 4096,
                              dummy, 64, None) == lib.EWORKSPACE
    assert lib.gq8_workspace_bytes(lib.OP_HC_PAIR, 6, 320, 16384) == \
        lib.gq8_workspace_bytes(lib.OP_HC_DOWN, 6, 320, 16384)
    # MoE limits
    assert raw.gq8_moe_q8_0_routed(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                   4, 8, 512, 2048, 2048, None, 0, None) == lib.ESHAPE


def test_pending_write_argument_checks(lib):
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced
    # R_out and P are required
    assert raw.gq8_hc_q8_down_pending(dummy, dummy, None, dummy, 1e-6, dummy, dummy, None, 1, 320,
                                      16384, dummy, 1 << 30, None) == lib.EINVAL
    assert raw.gq8_hc_q8_pair_pending(dummy, dummy, dummy, dummy, 1e-6, dummy, None, dummy, None,
                                      dummy, 1, 320, 16384, dummy, 1 << 30, None) == lib.EINVAL
    # misaligned R_out, shapes as the calls without the pending write
    assert raw.gq8_hc_q8_down_pending(dummy, dummy, dummy, dummy, 1e-6, dummy + 2, dummy, None, 1,
                                      320, 16384, dummy, 1 << 30, None) == lib.EALIGN
    assert raw.gq8_hc_q8_pair_pending(dummy, dummy, dummy, dummy, 1e-6, dummy, dummy, dummy, None,
                                      dummy, 1, 330, 16384, dummy, 1 << 30, None) == lib.ESHAPE
    assert raw.gq8_hc_q8_down_pending(dummy, dummy, dummy, dummy, 1e-6, dummy, dummy, None, 17,
                                      320, 16384, dummy, 1 << 30, None) == lib.ESHAPE
    # N == 0: the plain down read has nothing to do; the pending write needs the down read's
    # work-groups, so the pending call refuses it rather than leave R_out unwritten
    assert raw.gq8_hc_q8_down(dummy, dummy, dummy, 1e-6, dummy, None, 1, 0, 16384, None, 0,
                              None) == lib.OK
    assert raw.gq8_hc_q8_down_pending(dummy, dummy, dummy, dummy, 1e-6, dummy, dummy, None, 1, 0,
                                      16384, None, 0, None) == lib.ESHAPE


def test_moe_bf16_input_argument_checks(lib):
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced
    # F above 1024, D not a multiple of 32, T*topk above 256
    assert raw.gq8_moe_q8_0_routed_bf16(dummy, dummy, dummy, dummy, dummy, dummy,
                                        4, 8, 512, 2048, 2048, None, 0, None) == lib.ESHAPE
    assert raw.gq8_moe_q8_0_routed_bf16(dummy, dummy, dummy, dummy, dummy, dummy,
                                        4, 8, 512, 2056, 512, None, 0, None) == lib.ESHAPE
    assert raw.gq8_moe_q8_0_routed_bf16(dummy, dummy, dummy, dummy, dummy, dummy,
                                        16, 17, 512, 2048, 512, None, 0, None) == lib.ESHAPE
    # a null input, a misaligned input, a missing workspace
    assert raw.gq8_moe_q8_0_routed_bf16(None, dummy, dummy, dummy, dummy, dummy,
                                        4, 8, 512, 2048, 512, None, 0, None) == lib.EINVAL
    assert raw.gq8_moe_q8_0_routed_bf16(dummy + 2, dummy, dummy, dummy, dummy, dummy,
                                        4, 8, 512, 2048, 512, None, 0, None) == lib.EALIGN
    assert raw.gq8_moe_q8_0_routed_bf16(dummy, dummy, dummy, dummy, dummy, dummy,
                                        4, 8, 512, 2048, 512, None, 0, None) == lib.EWORKSPACE
    # T = 0 is a no-op
    assert raw.gq8_moe_q8_0_routed_bf16(None, None, None, None, None, None,
                                        0, 8, 512, 2048, 512, None, 0, None) == lib.OK
    # the workspace also holds the q8_1 form of a bf16 input (used when D > 4096)
    assert lib.gq8_moe_workspace_bytes(2, 4, 8192, 256) >= 2 * 8192 + 2 * 256 * 2


def test_moe_flags_argument_checks(lib):
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced
    assert lib.MOE_X_BF16 == 1 and lib.MOE_H_Q8_1 == 2 and lib.MOE_DOWN_TILED == 4
    # unknown flag bits
    assert raw.gq8_moe_q8_0_routed_flags(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                         4, 8, 512, 2048, 512, 8, None, 0, None) == lib.EINVAL
    # tiled down weights: the token kernel's shapes only (F in {256, 512, 1024}, topk <= 16)
    for flags in (lib.MOE_DOWN_TILED, lib.MOE_DOWN_TILED | lib.MOE_H_Q8_1 | lib.MOE_X_BF16):
        assert raw.gq8_moe_q8_0_routed_flags(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                             4, 8, 512, 2048, 320, flags, None, 0, None) == lib.ESHAPE
        assert raw.gq8_moe_q8_0_routed_flags(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                             1, 17, 512, 2048, 512, flags, None, 0, None) == lib.ESHAPE
        assert raw.gq8_moe_q8_0_routed_flags(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                             4, 8, 512, 2048, 512, flags, None, 0, None) == lib.EWORKSPACE
    # q8_1(h) needs F in {256, 512, 1024}
    assert raw.gq8_moe_q8_0_routed_flags(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                         4, 8, 512, 2048, 96, lib.MOE_H_Q8_1, None, 0, None) == lib.ESHAPE
    # q8_1(h) keeps one result row per slot on chip: at most 16 slots
    assert raw.gq8_moe_q8_0_routed_flags(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                         1, 17, 512, 2048, 512, lib.MOE_H_Q8_1, None, 0, None) == lib.ESHAPE
    # the int8 input needs its scales; the bf16 input does not
    assert raw.gq8_moe_q8_0_routed_flags(dummy, None, dummy, dummy, dummy, dummy, dummy,
                                         4, 8, 512, 2048, 512, 0, None, 0, None) == lib.EINVAL
    assert raw.gq8_moe_q8_0_routed_flags(dummy, None, dummy, dummy, dummy, dummy, dummy,
                                         4, 8, 512, 2048, 512, lib.MOE_X_BF16, None, 0, None) == lib.EWORKSPACE


def test_tile16_argument_checks(lib):
    """gq8_q8_0_tile16 refuses shapes that are not whole tiles, misaligned or overlapping buffers
    and null pointers before any device work; empty inputs are no work."""
    raw = lib.raw()
    a, b = 1 << 20, 1 << 24          # never dereferenced
    assert raw.gq8_q8_0_tile16(a, -16, 64, 1, b, None) == lib.EINVAL
    assert raw.gq8_q8_0_tile16(a, 16, 64, -1, b, None) == lib.EINVAL
    assert raw.gq8_q8_0_tile16(a, 24, 64, 1, b, None) == lib.ESHAPE        # rows % 16
    assert raw.gq8_q8_0_tile16(a, 16, 96, 1, b, None) == lib.ESHAPE        # K % 64
    assert raw.gq8_q8_0_tile16(a, 16, 64, 1 << 30, b, None) == lib.ESHAPE  # too many pieces
    assert raw.gq8_q8_0_tile16(None, 16, 64, 0, None, None) == lib.OK
    assert raw.gq8_q8_0_tile16(None, 0, 64, 5, None, None) == lib.OK
    assert raw.gq8_q8_0_tile16(None, 16, 64, 1, b, None) == lib.EINVAL
    assert raw.gq8_q8_0_tile16(a + 8, 16, 64, 1, b, None) == lib.EALIGN
    # one matrix of 16 x 64 is 1088 bytes: buffers 1088 bytes apart do not overlap, closer do
    assert raw.gq8_q8_0_tile16(a, 16, 64, 1, a + 1072, None) == lib.EINVAL
    assert raw.gq8_q8_0_tile16(a + 1072, 16, 64, 1, a, None) == lib.EINVAL
    assert raw.gq8_q8_0_tile16(a, 16, 64, 2, a + 1088, None) == lib.EINVAL


def test_tiled_up_argument_checks(lib):
    """The tiled up read and pair need whole 16-row tiles and an up depth that is a multiple of
    320, checked before any device work."""
    raw = lib.raw()
    d = 1 << 20      # never dereferenced
    assert raw.gq8_hc_q8_up_tiled(d, d, d, 1, 24, 320, None, 0, None) == lib.ESHAPE     # N % 16
    assert raw.gq8_hc_q8_up_tiled(d, d, d, 1, 32, 64, None, 0, None) == lib.ESHAPE      # K % 320
    assert raw.gq8_hc_q8_up_tiled(d, d, d, -1, 32, 320, None, 0, None) == lib.EINVAL
    assert raw.gq8_hc_q8_up_tiled(None, d, d, 1, 32, 320, None, 0, None) == lib.EINVAL
    assert raw.gq8_hc_q8_up_tiled(d + 8, d, d, 1, 32, 320, None, 0, None) == lib.EALIGN
    assert raw.gq8_hc_q8_pair_tiled(d, d, d, 1e-6, d, d, None, d, 1, 64, 1024, None, 0,
                                    None) == lib.ESHAPE                                  # Nlr % 320
    assert raw.gq8_hc_q8_pair_tiled(d, d, d, 1e-6, d, d, None, d, 1, 320, 1024, None, 0,
                                    None) == lib.EWORKSPACE


def test_per_token_argument_checks(lib):
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced
    # K not a multiple of 16, a negative size, a null scale output, misaligned input / quants
    assert raw.gq8_quantize_per_token(dummy, 4, 40, dummy, dummy, None) == lib.ESHAPE
    assert raw.gq8_quantize_per_token(dummy, -1, 64, dummy, dummy, None) == lib.EINVAL
    assert raw.gq8_quantize_per_token(dummy, 4, 64, dummy, None, None) == lib.EINVAL
    assert raw.gq8_quantize_per_token(dummy + 2, 4, 64, dummy, dummy, None) == lib.EALIGN
    assert raw.gq8_quantize_per_token(dummy, 4, 64, dummy + 8, dummy, None) == lib.EALIGN
    assert raw.gq8_quantize_per_token(None, 0, 64, None, None, None) == lib.OK
    # fused product: M above 32, K off 16 or above 8192, a null weight, misaligned x / x_q out
    args = lambda x, xq, M, K: (x, dummy, dummy, dummy, xq, dummy, M, 16, K, None, 0, None)  # noqa: E731
    assert raw.gq8_w8a8_gemm_bf16x(*args(dummy, None, 33, 64)) == lib.ESHAPE
    assert raw.gq8_w8a8_gemm_bf16x(*args(dummy, None, 4, 40)) == lib.ESHAPE
    assert raw.gq8_w8a8_gemm_bf16x(*args(dummy, None, 4, 8192 + 16)) == lib.ESHAPE
    assert raw.gq8_w8a8_gemm_bf16x(None, dummy, dummy, dummy, None, None, 4, 16, 64,
                                   None, 0, None) == lib.EINVAL
    assert raw.gq8_w8a8_gemm_bf16x(dummy, None, dummy, dummy, None, None, 4, 16, 64,
                                   None, 0, None) == lib.EINVAL
    assert raw.gq8_w8a8_gemm_bf16x(*args(dummy + 2, None, 4, 64)) == lib.EALIGN
    assert raw.gq8_w8a8_gemm_bf16x(*args(dummy, dummy + 4, 4, 64)) == lib.EALIGN
    assert raw.gq8_w8a8_gemm_bf16x(*args(None, None, 0, 64)) == lib.OK
    # past 8 rows or 16384 values x_q / x_scale are staged: in both outputs, else in a workspace
    assert lib.gq8_workspace_bytes(lib.OP_W8A8_BF16X, 4, 1536, 4096) == 0
    assert lib.gq8_workspace_bytes(lib.OP_W8A8_BF16X, 8, 1536, 2048) == 0
    assert lib.gq8_workspace_bytes(lib.OP_W8A8_BF16X, 8, 1536, 4096) == 8 * 4096 + 8 * 4
    assert lib.gq8_workspace_bytes(lib.OP_W8A8_BF16X, 16, 1536, 4096) == 16 * 4096 + 16 * 4
    assert lib.gq8_workspace_bytes(lib.OP_W8A8_BF16X, 9, 8, 48) == 512 + 9 * 4
    assert raw.gq8_w8a8_gemm_bf16x(dummy, dummy, dummy, dummy, None, None, 16, 16, 64,
                                   None, 0, None) == lib.EWORKSPACE
    assert raw.gq8_w8a8_gemm_bf16x(dummy, dummy, dummy, dummy, dummy, None, 16, 16, 64,
                                   dummy, 16 * 64, None) == lib.EWORKSPACE


def test_size_limits_return_eshape(lib):
    """Sizes past the documented limits are rejected before any device work (no int overflow in
    the checks, no launch past 2^32 work-items)."""
    raw = lib.raw()
    dummy = 1 << 20  # never dereferenced
    # Q8_0 reads: rows above 2^21, depth above 2^24, rows x depth above 2^36
    assert raw.gq8_q8_0_gemv(dummy, dummy, dummy, 1, (1 << 21) + 32, 64, None, 0, None) == lib.ESHAPE
    assert raw.gq8_q8_0_gemv(dummy, dummy, dummy, 1, 8, (1 << 24) + 32, None, 0, None) == lib.ESHAPE
    assert raw.gq8_q8_0_gemv(dummy, dummy, dummy, 1, 1 << 21, 1 << 18, None, 0, None) == lib.ESHAPE
    assert raw.gq8_hc_q8_down(dummy, dummy, dummy, 1e-6, dummy, None, 1, 320, (1 << 24) + 32,
                              None, 0, None) == lib.ESHAPE
    assert raw.gq8_hc_q8_up(dummy, dummy, dummy, 1, (1 << 21) + 16, 320, None, 0, None) == lib.ESHAPE
    assert raw.gq8_hc_q8_pair(dummy, dummy, dummy, 1e-6, dummy, dummy, None, dummy, 1, 320,
                              (1 << 24) + 32, None, 0, None) == lib.ESHAPE
    # W8A8 columns above 2^24: product, packer and packed size
    assert raw.gq8_w8a8_gemm(dummy, dummy, dummy, dummy, dummy, 4, (1 << 24) + 16, 64, None, 0,
                             None) == lib.ESHAPE
    assert raw.gq8_w8a8_pack(dummy, 64, (1 << 24) + 16, dummy, None) == lib.ESHAPE
    assert lib.gq8_w8a8_packed_bytes(64, (1 << 24) + 16) == 0
    assert lib.gq8_w8a8_packed_bytes(2**31 - 1, 16) == 16 * 2**31        # no overflow in K + 63
    assert raw.gq8_w8a8_pack(dummy, 2**31 - 16, 1 << 12, dummy, None) == lib.ESHAPE
    # quantizers: more than 2^32 - 256 blocks
    assert raw.gq8_q8_0_quantize(dummy, 1 << 20, 1 << 18, dummy, None) == lib.ESHAPE
    assert raw.gq8_q8_0_split_from_blocks(dummy, 1 << 20, 1 << 18, dummy, None) == lib.ESHAPE
    assert raw.gq8_q8_1_quantize(dummy, 1 << 20, 1 << 18, dummy, dummy, None, None) == lib.ESHAPE
    assert raw.gq8_quantize_per_token(dummy, (1 << 23) + 1, 64, dummy, dummy, None) == lib.ESHAPE
    # routed experts: width above 2^20; T * topk that overflows 32 bits is still rejected
    assert raw.gq8_moe_q8_0_routed(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                   4, 8, 512, (1 << 20) + 32, 512, None, 0, None) == lib.ESHAPE
    assert raw.gq8_moe_q8_0_routed(dummy, dummy, dummy, dummy, dummy, dummy, dummy,
                                   16, 1 << 28, 512, 2048, 512, None, 0, None) == lib.ESHAPE
    assert raw.gq8_moe_plan(dummy, 1 << 16, 1 << 16, 512, dummy, None) == lib.ESHAPE
    assert raw.gq8_moe_route(dummy, (1 << 23) + 1, 512, 8, dummy, dummy, None) == lib.ESHAPE
    # read probe: more than 2^32 - 256 pieces of 16 bytes
    assert raw.gq8_read_probe(dummy, 1 << 40, dummy, None) == lib.ESHAPE
