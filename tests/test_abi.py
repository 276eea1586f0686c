"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp8q.h declares, and rejects invalid arguments on the host before
anything touches a device (the checks that come first in each entry point).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


@pytest.fixture(scope="module")
def L():
    from fp8_weight_quantized_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from fp8_weight_quantized_amd import build
        build.build(verbose=False)
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8q_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 9
    from fp8_weight_quantized_amd import _lib
    assert set(names) == set(_lib.SIGNATURES), "binding signatures must mirror the header"
    for name in names:
        assert hasattr(L, name), name


def test_version_and_strings(L):
    assert L.fp8q_abi_version() == 3
    for s in range(5):
        assert L.fp8q_status_string(s).startswith(b"FP8Q")
    assert L.fp8q_status_string(99) == b"FP8Q: unknown status"


def test_workspace_queries(L):
    # activation pass-1 partials: one word per block, rounded to 256 bytes
    assert L.fp8q_quantize_act_workspace_size(8192, 4096) == 4096
    assert L.fp8q_quantize_act_workspace_size(1, 8) == 256
    assert L.fp8q_quantize_act_workspace_size(0, 8) == 256
    assert L.fp8q_quantize_act_workspace_size(4, 0) == 0
    # the W8A8 GEMM (more than 64 activation rows) needs no scratch; up to 64
    # rows W8A8 runs the decode kernels and their K-split scratch
    assert L.fp8q_linear_workspace_size(1, 8192, 28672, 4096) == 0
    assert L.fp8q_linear_workspace_size(1, 65, 28672, 4096) == 0
    # 65..1024 rows on a narrow weight: the decode kernels (the panel kernel
    # with 64 x 32 tiles up to 512 rows, whole K per workgroup, no scratch;
    # the tile kernel with K split where the panel does not take the shape),
    # or the 16-bit GEMM past 1024 rows
    assert L.fp8q_linear_workspace_size(1, 65, 4096, 4096) == 0
    assert L.fp8q_linear_workspace_size(0, 128, 8192, 4096) == 0
    assert L.fp8q_linear_workspace_size(0, 128, 1024, 4096) == 4 * 128 * 1024 * 4
    assert L.fp8q_linear_workspace_size(0, 1025, 4096, 4096) == 0
    assert L.fp8q_linear_workspace_size(1, 64, 4096, 4096) == 0         # the panel kernel
    assert L.fp8q_linear_workspace_size(1, 64, 1024, 4096) == 4 * 64 * 1024 * 4
    assert L.fp8q_linear_workspace_size(1, 1, 4096, 4096) == 0
    # up to 16 activation rows, K a multiple of 512 from 2048 on: the panel
    # kernel, whole K per workgroup, no scratch (every activation type); E4M3
    # codes with K not a multiple of 512 at 8K <= K < 16K take the tile
    # kernel with K split towards 4 ways (whole 1024-k chunks: 3 here)
    assert L.fp8q_linear_workspace_size(0, 12, 8192, 8192) == 0
    assert L.fp8q_linear_workspace_size(0, 12, 28672, 8192) == 0
    assert L.fp8q_linear_workspace_size(0, 12, 28672, 4096) == 0
    assert L.fp8q_linear_workspace_size(0, 1, 4096, 4096) == 0
    assert L.fp8q_linear_workspace_size(0, 12, 8192, 28672) == 0
    assert L.fp8q_linear_workspace_size(1, 12, 8192, 8192) == 0
    assert L.fp8q_linear_workspace_size(1, 12, 28672, 8192) == 0
    assert L.fp8q_linear_workspace_size(1, 12, 28672, 8208) == 3 * 12 * 28672 * 4
    # a small N on a short K: 64-row tiles, no split (K under two chunks)
    assert L.fp8q_linear_workspace_size(0, 4, 64, 500) == 0
    # 17..64 rows with about one workgroup per CU: the panel kernel, whole K
    # per workgroup, one launch, no scratch
    assert L.fp8q_linear_workspace_size(0, 64, 4096, 4096) == 0
    assert L.fp8q_linear_workspace_size(2, 32, 4096, 4096) == 0
    # otherwise K splits towards 256 workgroups (at least two chunks each),
    # with fp32 partial tiles [splits][m][n rounded up to 4]
    #   M=64, N=1024, K=4096: 16 tiles -> 4 splits of 1024
    assert L.fp8q_linear_workspace_size(0, 64, 1024, 4096) == 4 * 64 * 1024 * 4
    #   a small N on a long K (k/v projections) with K not a multiple of 512:
    #   16-row workgroups, K split in whole ranges of 2048 (4 waves x 512):
    #   N=1022, K=7000 -> 2 splits of 4096, partial rows padded to 1024
    assert L.fp8q_linear_workspace_size(0, 12, 1022, 7000) == 2 * 12 * 1024 * 4
    #   with K a multiple of 1024 the panel kernel spreads the activation rows
    #   4 per workgroup instead: no scratch
    assert L.fp8q_linear_workspace_size(0, 12, 1022, 8192) == 0
    #   E4M3 codes, M=12, N=8192, K=28688 (16-step chunks of 1024): 2 splits
    assert L.fp8q_linear_workspace_size(1, 12, 8192, 28688) == 2 * 12 * 8192 * 4
    #   M=40, N=100, K=3000: 2 tiles, at most 2 splits of whole 512-k chunks
    assert L.fp8q_linear_workspace_size(0, 40, 100, 3000) == 2 * 40 * 100 * 4
    assert L.fp8q_linear_workspace_size(0, 0, 4096, 4096) == 0
    # dynamic W8A8: a 256-byte scale slot, the absmax maxima (rounded to 256
    # bytes), then the decode plan's partial tiles, or the E4M3 codes above 64 rows
    assert L.fp8q_linear_w8a8_dynamic_workspace_size(1, 4096, 4096) == 256 + 256
    # 17..64 rows: the codes [m, k rounded to 16] and the panel GEMM (no scratch)
    assert L.fp8q_linear_w8a8_dynamic_workspace_size(64, 4096, 4096) == 256 + 256 + 64 * 4096
    assert L.fp8q_linear_w8a8_dynamic_workspace_size(12, 1022, 8192) == 256 + 256 + 4 * 12 * 1024 * 4
    assert L.fp8q_linear_w8a8_dynamic_workspace_size(8192, 28672, 4096) == 256 + 4096 + 8192 * 4096
    assert L.fp8q_linear_w8a8_dynamic_workspace_size(100, 300, 13) == 256 + 256 + 100 * 16 + 256 - 100 * 16 % 256
    assert L.fp8q_linear_w8a8_dynamic_workspace_size(0, 4096, 4096) == 0


def test_dynamic_host_validation(L):
    # (m, k, ld_x, n, ld_w, ld_y, ws_bytes) -> status, with NULL pointers: the
    # host checks come first
    cases = [
        ((-1, 64, 64, 16, 64, 16, 0), 1),               # m < 0
        ((1, 0, 64, 16, 64, 16, 0), 1),                 # k < 1
        ((1, 64, 60, 16, 64, 16, 0), 1),                # ld_x < k
        ((1, 64, 68, 16, 64, 16, 0), 1),                # ld_x not a multiple of 8
        ((1, 64, 64, 16, 72, 16, 0), 1),                # ld_w not a multiple of 16
        ((1, 64, 64, 16, 64, 12, 0), 1),                # ld_y not a multiple of 8
        ((0, 64, 64, 16, 64, 16, 0), 0),                # empty M: no-op
        ((4, 64, 64, 0, 64, 16, 0), 0),                 # empty N: no-op
        ((4, 64, 64, 16, 64, 16, 0), 4),                # workspace missing
    ]
    for (m, k, ldx, n, ldw, ldy, wsb), want in cases:
        got = L.fp8q_linear_w8a8_dynamic(NULL, m, k, ldx, NULL, n, ldw, NULL, NULL, ldy, NULL,
                                         NULL, wsb, NULL, NULL)
        assert got == want, ((m, k, ldx, n, ldw, ldy), got, L.fp8q_last_error())
    # the workspace overlapping the output is refused before any device query
    base = 0x20000000
    m, n, k = 8, 256, 1024
    need = L.fp8q_linear_w8a8_dynamic_workspace_size(m, n, k)
    got = L.fp8q_linear_w8a8_dynamic(base, m, k, k, base + (1 << 24), n, k, base + (2 << 24),
                                     base + (3 << 24), n, NULL, base + (3 << 24) + 64, need,
                                     NULL, NULL)
    assert got == 1 and "overlap" in L.fp8q_last_error().decode()


def test_describe(L):
    buf = ctypes.create_string_buffer(256)
    assert L.fp8q_linear_describe(0, 1, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 2, 4, 4>") and b"grid=(256,1)" in buf.value
    assert L.fp8q_linear_describe(0, 64, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<2, 2, 2, 2, 4>") and b"grid=(128,2)" in buf.value
    assert L.fp8q_linear_describe(0, 32, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<2, 1, 2, 3, 4>") and b"grid=(128,2)" in buf.value
    assert L.fp8q_linear_describe(0, 12, 28672, 8192, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<7, 1, 2, 2, 4>") and b"grid=(256,1)" in buf.value
    assert L.fp8q_linear_describe(1, 32, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<2, 1, 4, 3, 4>")
    assert L.fp8q_linear_describe(1, 64, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<2, 2, 4, 2, 4>")
    assert L.fp8q_linear_describe(1, 64, 1024, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_tile<4, 16, 8>")
    assert b"splits=4" in buf.value and b"k_w8a16_reduce" in buf.value
    assert L.fp8q_linear_describe(1, 8192, 28672, 4096, buf, 256) == 0
    assert b"32x112" in buf.value
    # 65..1024 rows: the decode kernels where the GEMM's grid would be one
    # round of a few tiles, the GEMMs otherwise
    # (the panel kernel with 64 x 32 tiles: two chunks in flight where its
    # grid is one round, else one; 16-bit activations on a wider weight only
    # at 3 activation groups)
    for mode, m, n, want in ((1, 128, 4096, b"k_w8a16_panel<4, 2, 2, 2, 4>"),
                             (1, 256, 4096, b"k_w8a16_panel<4, 2, 2, 1, 4>"),
                             (1, 512, 4096, b"k_w8a16_panel<4, 2, 2, 1, 4>"), (1, 768, 4096, b"k_w8a8 "),
                             (1, 65, 28672, b"k_w8a8 "),
                             (1, 128, 8192, b"k_w8a16_panel<4, 2, 2, 1, 4>"),
                             (1, 256, 8192, b"k_w8a16_panel<4, 2, 2, 1, 4>"),
                             (1, 384, 8192, b"k_w8a8 "),
                             (0, 512, 4096, b"k_w8a16_panel<4, 2, 2, 1, 4>"), (0, 1024, 4096, b"k_w8a16_tile<"),
                             (0, 128, 8192, b"k_w8a16_tile<"), (0, 65, 8192, b"k_w8a16_panel<4, 2, 2, 1, 4>"),
                             (0, 1025, 4096, b"k_w8a16_gemm<false>"),
                             (0, 256, 28672, b"k_w8a16_gemm<false>"),
                             (2, 128, 28672, b"k_w8a16_tile<"), (2, 65, 28672, b"k_w8a16_panel<4, 2, 2, 1, 4>"),
                             (2, 256, 28672, b"k_w8a16_gemm<true>"), (0, 128, 1024, b"k_w8a16_tile<")):
        assert L.fp8q_linear_describe(mode, m, n, 4096, buf, 256) == 0
        assert buf.value.startswith(want), (mode, m, n, buf.value)
    assert L.fp8q_linear_w8a8_dynamic_describe(128, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_act_amax + k_act_cast<0> + k_w8a16_panel<4, 2,")
    assert L.fp8q_linear_w8a8_dynamic_describe(128, 28672, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_act_amax + k_act_cast<0> + k_w8a8 ")
    assert L.fp8q_linear_describe(1, 8, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 2, 3, 4>")
    assert L.fp8q_linear_describe(2, 1, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 2, 4, 4>")
    # a weight of under 96 16-row panels (the Llama-3 k/v): 4 activation rows
    # per workgroup
    assert L.fp8q_linear_describe(0, 12, 1024, 8192, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 4, 2, 4>") and b"grid=(64,3)" in buf.value
    assert b"rows_per_workgroup=4" in buf.value
    assert L.fp8q_linear_describe(0, 8, 1024, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 4, 2, 4>") and b"grid=(64,2)" in buf.value
    # on the fly quantized activations keep the split rows kernel there
    assert L.fp8q_linear_w8a8_dynamic_describe(12, 1024, 8192, buf, 256) == 0
    assert b"k_w8a16_rows<1, 1, 8, 4>" in buf.value and b"splits=4" in buf.value
    # up to 32768 activation values on the panel kernel: one launch, the
    # workgroups take the absmax themselves; above, the absmax pass first
    assert L.fp8q_linear_w8a8_dynamic_describe(8, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 2, 3, 4>") and b"absmax and cast in the kernel" in buf.value
    assert L.fp8q_linear_w8a8_dynamic_describe(12, 4096, 4096, buf, 256) == 0
    assert buf.value.startswith(b"k_act_amax + k_w8a16_panel")
    # a K that is not a multiple of 512: the rows kernel
    assert L.fp8q_linear_describe(0, 1, 4096, 4000, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_rows<1, 1, 8, 4>")
    assert L.fp8q_linear_workspace_size(2, 64, 4096, 4096) == L.fp8q_linear_workspace_size(0, 64, 4096, 4096)
    assert L.fp8q_linear_describe(7, 1, 1, 1, buf, 256) == 1


def test_describe_grouped(L):
    buf = ctypes.create_string_buffer(256)
    # fp8_w_fp8_a from 65 to 1024 rows: the decode kernels on a narrow weight,
    # the grouped FP8 GEMM on a wide one or past 1024 rows
    for m, n, g, want in ((128, 4096, 128, b"k_w8a16_tile<"), (512, 4096, 512, b"k_w8a16_tile<"),
                          (1024, 4096, 128, b"k_w8a8<true>"), (128, 28672, 128, b"k_w8a8<true>"),
                          (512, 8192, 128, b"k_w8a8<true>"), (1025, 256, 256, b"k_w8a8<true>")):
        assert L.fp8q_linear_grouped_describe(1, m, n, 4096, g, buf, 256) == 0
        assert buf.value.startswith(want), (m, n, g, buf.value)
    # up to 16 rows on a 4096-row weight: the panel kernel with group scales
    assert L.fp8q_linear_grouped_describe(0, 1, 4096, 4096, 128, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 2, 4, 4, 2>")
    # 28672 rows: 4 weight fragments (7, as per channel, spill with group scales)
    assert L.fp8q_linear_grouped_describe(0, 12, 28672, 8192, 128, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<4, 1, 2, 3, 4, 2>") and b"grid=(448,1)" in buf.value
    # K = 1000 (not a multiple of 512): the rows kernel, wave ranges rounded up
    # to one 512-k round
    assert L.fp8q_linear_grouped_describe(2, 12, 4096, 1000, 64, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_rows<1, 1, 8, 4, 1>") and b"kchunk=512" in buf.value
    # a small N on a long K: 4 activation rows per workgroup, as per channel
    assert L.fp8q_linear_grouped_describe(0, 12, 1024, 8192, 512, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<1, 1, 4, 2, 4, 8>") and b"grid=(64,3)" in buf.value
    # a group that does not divide the waves' K ranges: the rows kernel
    assert L.fp8q_linear_grouped_describe(0, 12, 4096, 2560, 512, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_rows<1, 1, 8, 4, 8>")
    # 64 rows: two 32-row panels for 16-bit activations; the tile kernel for
    # E4M3 codes
    assert L.fp8q_linear_grouped_describe(0, 64, 4096, 4096, 128, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_panel<2, 2, 2, 2, 4, 2>")
    assert L.fp8q_linear_grouped_describe(1, 64, 4096, 4096, 128, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_tile<4, 16, 8, 2>")
    # prefill W8A8: the FP8 GEMM for groups of 128 and up, the tile kernel for 64
    assert L.fp8q_linear_grouped_describe(1, 8192, 28672, 4096, 128, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a8<true>") and b"32x112" in buf.value
    assert L.fp8q_linear_grouped_describe(1, 8192, 28672, 4096, 64, buf, 256) == 0
    assert buf.value.startswith(b"k_w8a16_tile<4, 16, 8, 1>")
    assert L.fp8q_linear_grouped_describe(0, 1, 4096, 4096, 96, buf, 256) == 1
    assert L.fp8q_linear_grouped_describe(7, 1, 1, 1, 128, buf, 256) == 1


NULL = None


def test_linear_host_validation(L):
    # (mode, m, k, ld_x, x_scale, n, ld_w, ld_y, ws_bytes) -> expected status
    fake = ctypes.c_void_p(0x1000)
    cases = [
        ((5, 1, 64, 64, NULL, 16, 64, 16), 1),          # unknown mode
        ((0, 1, 0, 64, NULL, 16, 64, 16), 1),           # k < 1
        ((0, -1, 64, 64, NULL, 16, 64, 16), 1),         # m < 0
        ((0, 1, 64, 32, NULL, 16, 64, 16), 1),          # ld_x < k
        ((0, 1, 64, 68, NULL, 16, 64, 16), 1),          # ld_x not a multiple of 8 (bf16)
        ((1, 1, 64, 72, fake, 16, 64, 16), 1),          # ld_x not a multiple of 16 (fp8)
        ((0, 1, 64, 64, NULL, 16, 72, 16), 1),          # ld_w not a multiple of 16
        ((0, 1, 64, 64, NULL, 16, 64, 12), 1),          # ld_y not a multiple of 8
        ((0, 1, 64, 64, fake, 16, 64, 16), 1),          # x_scale given in W8A16
        ((2, 1, 64, 64, fake, 16, 64, 16), 1),          # x_scale given in W8A16 fp16
        ((2, 1, 64, 68, NULL, 16, 64, 16), 1),          # fp16 ld_x not a multiple of 8
        ((2, 0, 64, 64, NULL, 16, 64, 16), 0),          # fp16, empty M: no-op
        ((1, 1, 64, 64, NULL, 16, 64, 16), 1),          # x_scale missing in W8A8
        ((0, 0, 64, 64, NULL, 16, 64, 16), 0),          # empty M: no-op
        ((1, 4, 64, 64, fake, 0, 64, 16), 0),           # empty N: no-op
        ((0, 1, 64, 1 << 28, NULL, 16, 64, 16), 1),     # ld_x >= 2^28
        ((2, 1, 64, 64, NULL, 16, 1 << 28, 16), 1),     # ld_w >= 2^28
    ]
    for (mode, m, k, ldx, xs, n, ldw, ldy), want in cases:
        got = L.fp8q_linear(mode, NULL, m, k, ldx, xs, NULL, n, ldw, NULL, NULL, ldy, NULL, 0, NULL)
        assert got == want, ((mode, m, k, ldx, n, ldw, ldy), got, L.fp8q_last_error())
        if want:
            assert L.fp8q_last_error()


def test_linear_overlap_rejected_on_host(L):
    """Aliasing is refused from the pointer values alone, before any device
    query: here an activation scale placed inside the K-split workspace, which
    the split GEMM would overwrite before the reduction reads the scale."""
    m, n, k = 12, 1024, 8208          # a K-split decode plan (K not a multiple of 512)
    need = L.fp8q_linear_workspace_size(1, m, n, k)
    assert need > 0
    base = 0x10000000
    x, w, ws, y = base, base + (1 << 24), base + (2 << 24), base + (3 << 24)
    wk = base + (4 << 24)
    args = lambda xs: (1, x, m, k, k, xs, w, n, k, ws, y, n, wk, need, NULL)
    assert L.fp8q_linear(*args(wk + 64)) == 1
    assert "overlap" in L.fp8q_last_error().decode()
    assert L.fp8q_linear(*args(y + 16)) == 1            # scale inside the output
    assert L.fp8q_linear(*args(base + (5 << 24))) != 1 or "overlap" not in L.fp8q_last_error().decode()


def test_quantize_host_validation(L):
    assert L.fp8q_quantize_weight(NULL, 4, 0, 8, NULL, 8, NULL, NULL, NULL) == 1
    assert L.fp8q_quantize_weight(NULL, 4, 8, 4, NULL, 8, NULL, NULL, NULL) == 1
    assert L.fp8q_quantize_weight(NULL, 0, 8, 8, NULL, 8, NULL, NULL, NULL) == 0
    assert L.fp8q_quantize_act(NULL, 4, 8, 8, NULL, 8, NULL, NULL, 0, NULL, NULL) == 4
    assert L.fp8q_quantize_act(NULL, 4, 8, 8, NULL, 8, NULL, ctypes.c_void_p(0x1000), 8, NULL, NULL) == 4
    assert L.fp8q_quantize_act(NULL, -1, 8, 8, NULL, 8, NULL, NULL, 0, NULL, NULL) == 1
    assert L.fp8q_cast_f32_to_e4m3(NULL, -1, NULL, NULL) == 1
    assert L.fp8q_cast_f32_to_e4m3(NULL, 0, NULL, NULL) == 0


def test_act_scale_host_validation(L):
    """Static / EMA entry points reject bad arguments before touching a device."""
    st = L.fp8q_quantize_act_static
    assert st(NULL, 0, 8, 8, NULL, NULL, 8, NULL, NULL) == 0          # empty: no-op
    assert st(NULL, -1, 8, 8, NULL, NULL, 8, NULL, NULL) == 1
    assert st(NULL, 4, 0, 8, NULL, NULL, 8, NULL, NULL) == 1
    assert st(NULL, 4, 8, 4, NULL, NULL, 8, NULL, NULL) == 1           # ld_x < k
    assert st(NULL, 4, 8, 8, NULL, NULL, 7, NULL, NULL) == 1           # ld_q < k
    ema = L.fp8q_quantize_act_ema
    ws = ctypes.c_void_p(0x1000)
    need = L.fp8q_quantize_act_workspace_size(4, 8)

    def call(m=4, k=8, ldx=8, ldq=8, decay=0.9999, temp=0.0, w=ws, nw=need):
        return ema(NULL, m, k, ldx, NULL, ldq, NULL, NULL, decay, temp, 0, w, nw, NULL, NULL)

    for bad in (-0.1, 1.5, float("nan"), float("inf")):
        assert call(decay=bad) == 1, bad
        assert "decay" in L.fp8q_last_error().decode()
    for bad in (-1.0, float("nan"), float("inf")):
        assert call(temp=bad) == 1, bad
        assert "temperature" in L.fp8q_last_error().decode()
    assert call(m=-1) == 1
    assert call(k=0) == 1
    assert call(ldx=7) == 1
    assert call(ldq=7) == 1
    assert call(w=NULL, nw=0) == 4
    assert call(nw=need - 1) == 4


def test_kv_cache_host_validation(L):
    """The KV-cache write rejects bad shapes before touching a device."""
    kv = L.fp8q_kv_cache_write
    ws = ctypes.c_void_p(0x1000)

    def call(t=4, heads=8, hd=128, ld=1024, slots=16, w=ws, nw=None):
        if nw is None:
            nw = L.fp8q_kv_cache_workspace_size(max(t, 0), heads, hd)
        return kv(NULL, NULL, t, heads, hd, ld, NULL, NULL, NULL, slots, NULL, NULL, 1, w, nw,
                  NULL, NULL)

    assert call(t=-1) == 1
    assert call(heads=0) == 1
    assert call(slots=0) == 1
    assert call(hd=0) == 1 and call(hd=12) == 1 and call(hd=4, ld=32) == 1
    assert call(ld=1000) == 1                     # below heads * head_dim
    assert call(ld=1028) == 1                     # not a multiple of 8
    assert call(t=1 << 28) == 1                   # tokens * width / 8 reaches 2^31
    assert call(w=NULL, nw=0) == 4
    assert call(nw=L.fp8q_kv_cache_workspace_size(4, 8, 128) - 1) == 4
    assert L.fp8q_kv_cache_workspace_size(8192, 8, 128) == 2 * 1024 * 4
    assert L.fp8q_kv_cache_workspace_size(12, 8, 128) == 256


def test_grouped_host_validation(L):
    """Per-group entry points: group sizes, shapes and workspace before any device work."""
    for bad in (0, 32, 100, 1024, -128):
        assert L.fp8q_quantize_weight_grouped(NULL, 4, 512, 512, bad, NULL, 512, NULL, NULL,
                                              NULL) == 1, bad
        assert L.fp8q_linear_grouped(0, NULL, 4, 512, 512, NULL, NULL, 8, 512, NULL, bad, NULL, 8,
                                     NULL, 0, NULL) == 1, bad
        assert L.fp8q_linear_grouped_workspace_size(0, 4, 8, 512, bad) == 0
    assert L.fp8q_quantize_weight_grouped(NULL, 0, 512, 512, 128, NULL, 512, NULL, NULL, NULL) == 0
    assert L.fp8q_quantize_weight_grouped(NULL, 4, 0, 512, 128, NULL, 512, NULL, NULL, NULL) == 1
    assert L.fp8q_quantize_weight_grouped(NULL, 4, 512, 500, 128, NULL, 512, NULL, NULL, NULL) == 1
    lg = L.fp8q_linear_grouped
    assert lg(0, NULL, 0, 512, 512, NULL, NULL, 8, 512, NULL, 128, NULL, 8, NULL, 0, NULL) == 0
    assert lg(0, NULL, 4, 512, 500, NULL, NULL, 8, 512, NULL, 128, NULL, 8, NULL, 0, NULL) == 1
    assert lg(1, NULL, 4, 512, 512, NULL, NULL, 8, 512, NULL, 128, NULL, 8, NULL, 0, NULL) == 1
    # a K split at decode: workspace needed, none given
    # 2 tiles of 64 rows, K >= 16K: 1024-k chunks, 14 splits of 2048 k (2
    # chunks each) -> [14][12][128] fp32, as per channel
    assert L.fp8q_linear_grouped_workspace_size(0, 12, 128, 28672, 128) == 14 * 12 * 128 * 4
    assert L.fp8q_linear_workspace_size(0, 12, 128, 28672) == 14 * 12 * 128 * 4
    assert lg(0, NULL, 12, 28672, 28672, NULL, NULL, 128, 28672, NULL, 128, NULL, 128, NULL, 0,
              NULL) == 4
    # up to 16 rows on a 4096-row weight: the panel kernel, unsplit, as per channel
    assert L.fp8q_linear_grouped_workspace_size(0, 1, 4096, 4096, 128) == 0
    # 64 rows of 16-bit activations: two 32-row panels, unsplit
    assert L.fp8q_linear_grouped_workspace_size(0, 64, 4096, 4096, 128) == 0
    # 64 rows of E4M3 codes: 64 tiles, 4 splits of 1024 k
    assert L.fp8q_linear_grouped_workspace_size(1, 64, 4096, 4096, 128) == 4 * 64 * 4096 * 4
    # 448 tiles x 128 row blocks: no split
    assert L.fp8q_linear_grouped_workspace_size(1, 8192, 28672, 4096, 128) == 0


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    from fp8_weight_quantized_amd import _lib
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.lib()
