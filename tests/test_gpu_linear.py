"""GPU parity of the scaled linear layer against the fp64 oracle.

Both FP8 MatMul modes of Llama 3 精读 §3.1 step 3 -- fp8_w_bf16_a (W8A16,
decode) and fp8_w_fp8_a (W8A8, prefill) -- are checked with the same codes
and scales on both sides (the codes come from the oracle, so this file tests
the GEMM alone), to rel. Frobenius <= 5e-3 and per-element <= 1e-2 max|ref|.
Exact cases (one-hot activations) pin every E4M3 code's decode and the MFMA
lane layouts bit for bit.
"""
import numpy as np
import pytest

import workloads
from helpers import assert_gemm_close, dev_bf16, dev_u8, host_bf16_as_f64, rows_every_tile, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_weight_quantized_amd as fq
    fq.library_path()
    return fq


def pad16(a: np.ndarray):
    """Upload codes with a 16-byte-multiple row stride (what the GEMM requires)."""
    rows, cols = a.shape
    ld = (cols + 15) // 16 * 16
    t = torch.zeros((rows, ld), dtype=torch.uint8, device="cuda")
    t[:, :cols] = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t[:, :cols]


def pad8_bf16(bits: np.ndarray):
    rows, cols = bits.shape
    ld = (cols + 7) // 8 * 8
    t = torch.zeros((rows, ld), dtype=torch.bfloat16, device="cuda")
    t[:, :cols] = dev_bf16(bits)
    return t[:, :cols]


def run_w8a16(fq, x_bits, wq, ws):
    y = fq.linear(pad8_bf16(x_bits), pad16(wq), torch.from_numpy(ws).cuda())
    torch.cuda.synchronize()
    return host_bf16_as_f64(y)


def run_w8a8(fq, xq, xs, wq, ws):
    y = fq.linear(pad16(xq), pad16(wq), torch.from_numpy(ws).cuda(),
                  x_scale=torch.tensor([xs], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    return host_bf16_as_f64(y)


def all_codes_weight(n: int, k: int) -> np.ndarray:
    w = ((np.arange(n)[:, None] + np.arange(k)[None, :]) % 256).astype(np.uint8)
    w[(w & 0x7F) == 0x7F] = 0x00           # no NaN codes
    return w


# shapes that take k_w8a16_panel (K a multiple of 512 from 2048 on; 17..64
# rows where that makes about one workgroup per CU), including a ragged last
# panel of weight rows and of activation rows
PANEL_SHAPES = [(40, 4096, 2048), (20, 3200, 3072), (33, 4000, 2048), (64, 4096, 4096),
                (17, 4096, 2048), (64, 3584, 8192),
                # up to 16 rows: 1, 2, 3, 4 or 7 weight fragments per workgroup
                (12, 8192, 2048), (5, 10240, 2048), (16, 28672, 2048), (1, 16384, 3072),
                (7, 9000, 2560), (3, 4096, 2048), (16, 2048, 2560), (8, 1024, 2048),
                (9, 12288, 2048), (4, 1536, 14336),
                # a weight of under 96 16-row panels: 4 activation rows per
                # workgroup (ragged last row group and weight panel)
                (13, 1000, 4096), (16, 1024, 8192)]


@pytest.mark.parametrize("m,n,k", [(16, 256, 64), (1, 256, 64), (64, 272, 64), (12, 256, 64),
                                   (1, 272, 576), (7, 300, 1100), (16, 256, 2048), (40, 320, 1536),
                                   (64, 272, 1600), (5, 4096, 1100), (1, 2304, 640),
                                   (16, 512, 4160), (2, 300, 8200)] + PANEL_SHAPES)
def test_w8a16_exact_every_code(fq, orc, m, n, k):
    """X = one-hot rows: Y[i, j] = dec(W[j, p_i]) exactly, for all 254 finite codes.
    The one-hot positions p_i are spread evenly over K (first to last), so
    with K > 512 they land in different staged chunks, steps, K splits and
    the ragged end of K."""
    wq = all_codes_weight(n, k)
    x = np.zeros((m, k), np.uint16)
    pos = (np.arange(m) * (k - 1)) // max(m - 1, 1)
    x[np.arange(m), pos] = 0x3F80          # 1.0
    ws = np.ones(n, np.float32)
    say("w8a16 exact", m, n, k, fq.describe_linear(0, m, n, k))
    y = run_w8a16(fq, x, wq, ws)
    ref = orc.linear(0, x, wq, ws)
    assert (y == ref).all(), np.argwhere(y != ref)[:5]


def pad8_f16(bits: np.ndarray):
    rows, cols = bits.shape
    ld = (cols + 7) // 8 * 8
    t = torch.zeros((rows, ld), dtype=torch.float16, device="cuda")
    t[:, :cols] = torch.from_numpy(np.ascontiguousarray(bits).view(np.float16)).cuda()
    return t[:, :cols]


def run_w8a16_f16(fq, x_bits, wq, ws):
    y = fq.linear(pad8_f16(x_bits), pad16(wq), torch.from_numpy(ws).cuda())
    torch.cuda.synchronize()
    assert y.dtype == torch.float16
    return host_bf16_as_f64(y)


def f16_act(m: int, k: int, seed: int) -> np.ndarray:
    """fp16 bit patterns of the workload's N(0, 1) activations."""
    return workloads.bf16_bits_to_f32(workloads.normal_act(m, k, seed)).astype(np.float16).view(np.uint16)


@pytest.mark.parametrize("m,n,k", [(16, 256, 64), (1, 272, 576), (64, 272, 1600), (5, 4096, 1100),
                                   (16, 512, 4160), (40, 320, 1536), (33, 4000, 2048)])
def test_w8a16_f16_exact_every_code(fq, orc, m, n, k):
    """fp8_w_fp16_a with one-hot fp16 rows: every E4M3 code widened to fp16 exactly."""
    wq = all_codes_weight(n, k)
    x = np.zeros((m, k), np.uint16)
    pos = (np.arange(m) * (k - 1)) // max(m - 1, 1)
    x[np.arange(m), pos] = 0x3C00          # fp16 1.0
    ws = np.ones(n, np.float32)
    say("w8a16 fp16 exact", m, n, k, fq.describe_linear(2, m, n, k))
    y = run_w8a16_f16(fq, x, wq, ws)
    ref = orc.linear(2, x, wq, ws)
    assert (y == ref).all(), np.argwhere(y != ref)[:5]


@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (8, 4096, 4096), (32, 4096, 4096), (64, 4096, 4096),
                                   (12, 1024, 8192), (3, 100, 1000), (17, 130, 520), (100, 96, 4104),
                                   (5, 300, 5000), (40, 522, 3000), (1, 16, 8), (12, 28672, 512),
                                   (50, 4096, 4096)])
def test_w8a16_f16_ragged(fq, orc, m, n, k):
    w = workloads.heavy_tail_weight(n, k, m + n)
    x = f16_act(m, k, k)
    wq, ws, _ = orc.quantize_weight(w)
    say("w8a16 fp16", m, n, k, fq.describe_linear(2, m, n, k))
    y = run_w8a16_f16(fq, x, wq, ws)
    assert_gemm_close(y, orc.linear(2, x, wq, ws), f"w8a16 fp16 {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(256, 256, 64), (300, 260, 128), (33, 512, 64), (8, 300, 1100),
                                   (64, 272, 1600), (1, 4096, 640), (16, 512, 4160), (520, 300, 640)]
                         + PANEL_SHAPES)
def test_w8a8_exact_every_code(fq, orc, m, n, k):
    """One-hot E4M3 rows (spread over K) pick weight columns exactly; up to 64
    rows this is the decode path, beyond it the FP8 MFMA GEMM."""
    wq = all_codes_weight(n, k)
    xq = np.zeros((m, k), np.uint8)
    xq[np.arange(m), (np.arange(m) * (k - 1)) // max(m - 1, 1)] = 0x38          # 1.0
    ws = np.ones(n, np.float32)
    say("w8a8 exact", m, n, k)
    y = run_w8a8(fq, xq, 1.0, wq, ws)
    ref = orc.linear(1, xq, wq, ws, np.float32(1.0))
    assert (y == ref).all(), np.argwhere(y != ref)[:5]


# the prefill GEMM of the 16-bit activation modes (more than 64 rows): K a
# multiple of its 64-value stage or not (a zero-filled tail stage), ragged M and
# N around the 256 x 256 tile, and more than 8 tile-rows
PREFILL16 = [(65, 300, 640), (256, 256, 64), (513, 257, 200), (300, 520, 1000), (129, 200, 96),
             (777, 64, 2048), (1000, 1000, 1280), (2305, 2048, 640), (100, 96, 4104), (257, 33, 13)]
# From 65 to 1024 rows a narrow weight on a long enough K runs the decode
# kernels instead of a GEMM (the GEMM's grid would be one round of a few
# tiles); these shapes have more than 1024 rows, so the GEMMs take them
# whatever N is.
GEMM_ROWS = [(1089, 300, 640), (1324, 520, 1000), (1801, 64, 2048), (1030, 1000, 1280),
             (1124, 96, 4104)]
PREFILL16_EXACT = [(1089, 300, 640), (256, 256, 64), (513, 257, 200), (1324, 520, 1000),
                   (129, 200, 96), (1801, 64, 2048)]


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("m,n,k", PREFILL16_EXACT)
def test_prefill16_exact_every_code(fq, orc, mode, m, n, k):
    """One-hot 16-bit rows through k_w8a16_gemm: every E4M3 code widened
    exactly, the tile layouts and the zero-filled K tail bit for bit."""
    assert fq.describe_linear(mode, m, n, k).startswith("k_w8a16_gemm")
    wq = all_codes_weight(n, k)
    x = np.zeros((m, k), np.uint16)
    pos = (np.arange(m) * (k - 1)) // max(m - 1, 1)
    x[np.arange(m), pos] = 0x3F80 if mode == 0 else 0x3C00      # 1.0
    ws = np.ones(n, np.float32)
    say("prefill16 exact", mode, m, n, k)
    y = run_w8a16(fq, x, wq, ws) if mode == 0 else run_w8a16_f16(fq, x, wq, ws)
    ref = orc.linear(mode, x, wq, ws)
    assert (y == ref).all(), np.argwhere(y != ref)[:5]


@pytest.mark.parametrize("mode", [0, 2])
@pytest.mark.parametrize("m,n,k", PREFILL16 + GEMM_ROWS)
def test_prefill16_ragged(fq, orc, mode, m, n, k):
    w = workloads.heavy_tail_weight(n, k, m + n + 5)
    wq, ws, _ = orc.quantize_weight(w)
    x = workloads.normal_act(m, k, k + 3) if mode == 0 else f16_act(m, k, k + 3)
    say("prefill16", mode, m, n, k, fq.describe_linear(mode, m, n, k))
    y = run_w8a16(fq, x, wq, ws) if mode == 0 else run_w8a16_f16(fq, x, wq, ws)
    assert_gemm_close(y, orc.linear(mode, x, wq, ws), f"prefill16 mode {mode} {m}x{n}x{k}")


@pytest.mark.parametrize("mode", [2, 0])
def test_prefill16_mlp_full_size_sampled(fq, orc, mode):
    """Llama-3-8B gate+up prefill (M=8192, N=28672, K=4096) with fp16 (the
    write-up's prefill mode) or bf16 activations, as the benchmark launches it:
    seeded rows in every 256-row band x all columns, so every output tile."""
    wl = workloads.WORKLOADS["mlp_prefill"]
    lin = wl.linears[0]
    m = wl.ms[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    xb = workloads.activation(wl, m, lin.k)
    x = xb if mode == 0 else workloads.bf16_bits_to_f32(xb).astype(np.float16).view(np.uint16)
    say("prefill16 full", mode, fq.describe_linear(mode, m, lin.n, lin.k))
    xd = dev_bf16(x) if mode == 0 else torch.from_numpy(np.ascontiguousarray(x).view(np.float16)).cuda()
    y = fq.linear(xd, dev_u8(wq), torch.from_numpy(ws).cuda())
    torch.cuda.synchronize()
    rows = rows_every_tile(m, 13)
    got = y[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    assert_gemm_close(got, orc.linear(mode, x, wq, ws, rows=rows), f"prefill16 full mode {mode}")


def test_tiny(fq, orc):
    wl = workloads.WORKLOADS["tiny"]
    lin = wl.linears[0]
    w = workloads.weight(wl, lin)
    x = workloads.activation(wl, 16, lin.k)
    wq, ws, _ = orc.quantize_weight(w)
    say("tiny w8a16")
    y = run_w8a16(fq, x, wq, ws)
    assert_gemm_close(y, orc.linear(0, x, wq, ws), "tiny")


RAGGED = [(3, 100, 1000), (17, 130, 520), (65, 64, 64), (100, 96, 4104), (1, 16, 8),
          (5, 1, 40), (2, 4096, 4096), (64, 1024, 8192), (33, 77, 13), (129, 200, 96),
          (7, 300, 2048), (13, 63, 1536), (40, 522, 3000), (6, 1, 700),
          (5, 300, 5000), (12, 1022, 8192), (1, 100, 4096), (16, 64, 12288)]


@pytest.mark.parametrize("m,n,k", RAGGED + PANEL_SHAPES)
def test_w8a16_ragged(fq, orc, m, n, k):
    w = workloads.heavy_tail_weight(n, k, m + n)
    x = workloads.normal_act(m, k, k)
    wq, ws, _ = orc.quantize_weight(w)
    say("w8a16 ragged", m, n, k, fq.describe_linear(0, m, n, k))
    y = run_w8a16(fq, x, wq, ws)
    assert_gemm_close(y, orc.linear(0, x, wq, ws), f"w8a16 {m}x{n}x{k}")


# K a multiple of the prefill kernel's 128-byte stage: one stage, two, an odd
# count, with ragged M and N around the 256 x 256 tile
WHOLE_STAGES = [(257, 300, 128), (300, 520, 384), (513, 257, 256), (1000, 1000, 1280), (777, 64, 2048)]
# more than 8 tile-rows, so the XCD-banded tile order has a full band and a
# partial one: 10 x 8 = 80 tiles (a multiple of the 8 XCDs) and 17 x 3 = 51
MANY_TILE_ROWS = [(2305, 2048, 640), (4100, 600, 256)]


@pytest.mark.parametrize("m,n,k", RAGGED + [(300, 520, 1000), (256, 256, 4096), (513, 257, 200)] + WHOLE_STAGES
                         + MANY_TILE_ROWS + PANEL_SHAPES + GEMM_ROWS)
def test_w8a8_ragged(fq, orc, m, n, k):
    w = workloads.heavy_tail_weight(n, k, m + n)
    x = workloads.outlier_act(m, k, k)
    wq, ws, _ = orc.quantize_weight(w)
    xq, xs, _ = orc.quantize_act(x)
    say("w8a8 ragged", m, n, k, fq.describe_linear(1, m, n, k))
    y = run_w8a8(fq, xq, xs, wq, ws)
    assert_gemm_close(y, orc.linear(1, xq, wq, ws, xs), f"w8a8 {m}x{n}x{k}")


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_q_proj_decode_full(fq, orc, m):
    wl = workloads.WORKLOADS["q_proj_decode"]
    lin = wl.linears[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    x = workloads.activation(wl, m, lin.k)
    say("q_proj decode", m, fq.describe_linear(0, m, lin.n, lin.k))
    y = run_w8a16(fq, x, wq, ws)
    assert_gemm_close(y, orc.linear(0, x, wq, ws), f"q_proj M={m}")


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_q_proj_w8a8_decode_full(fq, orc, m):
    """fp8_w_fp8_a at decode sizes (the decode kernels with E4M3 activations)
    on the full q_proj weight, X quantized per tensor by the oracle."""
    wl = workloads.WORKLOADS["q_proj_decode"]
    lin = wl.linears[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    xq, xs, _ = orc.quantize_act(workloads.activation(wl, m, lin.k))
    say("q_proj w8a8 decode", m, fq.describe_linear(1, m, lin.n, lin.k))
    y = run_w8a8(fq, xq, xs, wq, ws)
    assert_gemm_close(y, orc.linear(1, xq, wq, ws, xs), f"q_proj w8a8 M={m}")


@pytest.mark.parametrize("idx", range(7))
def test_layer_decode_70b_full(fq, orc, idx):
    wl = workloads.WORKLOADS["layer_decode_70b"]
    lin = wl.linears[idx]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    x = workloads.activation(wl, 12, lin.k)
    say("70b layer decode", lin.name, fq.describe_linear(0, 12, lin.n, lin.k))
    y = run_w8a16(fq, x, wq, ws)
    assert_gemm_close(y, orc.linear(0, x, wq, ws), lin.name)


@pytest.mark.parametrize("key", ["mlp_prefill", "down_prefill_70b"])
def test_prefill_full_size_sampled(fq, orc, key):
    """Full-size W8A8 GEMM as the benchmark launches it.  Seeded rows, at least
    two in every 256-row band of the GEMM's tiles and at least 64 in all,
    times all N columns, so every 256 x 256 output tile is compared with the
    fp64 oracle."""
    wl = workloads.WORKLOADS[key]
    lin = wl.linears[0]
    m = wl.ms[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    xq, xs, _ = orc.quantize_act(workloads.activation(wl, m, lin.k))
    say("prefill", key, fq.describe_linear(1, m, lin.n, lin.k))
    y = fq.linear(pad16(xq), pad16(wq), torch.from_numpy(ws).cuda(),
                  x_scale=torch.tensor([xs], dtype=torch.float32, device="cuda"))
    torch.cuda.synchronize()
    rows = rows_every_tile(m, 7)
    assert rows.size >= 64 and len(set(rows // 256)) == (m + 255) // 256
    ysel = host_bf16_as_f64(y[torch.from_numpy(rows).cuda()])
    ref = orc.linear(1, xq, wq, ws, xs, rows=rows)
    assert_gemm_close(ysel, ref, key)


def test_pipeline_w8a8_from_gpu_quantizers(fq, orc):
    """quantize_weight + quantize_act + linear, all on the GPU, against the oracle."""
    m, n, k = 384, 512, 1024
    w = workloads.heavy_tail_weight(n, k, 11)
    x = workloads.swiglu_act(m, k, 12)
    say("pipeline w8a8")
    wq, ws = fq.quantize_weight(dev_bf16(w))
    xq, xs = fq.quantize_act(dev_bf16(x))
    y = host_bf16_as_f64(fq.linear(xq, wq, ws, x_scale=xs))
    owq, ows, _ = orc.quantize_weight(w)
    oxq, oxs, _ = orc.quantize_act(x)
    assert_gemm_close(y, orc.linear(1, oxq, owq, ows, oxs), "pipeline")


@pytest.mark.parametrize("shapes", [[(40, 200, 5000), (20, 100, 2100)],
                                    [(64, 1024, 4096), (33, 130, 3000), (64, 1024, 4096)]])
def test_w8a16_split_workspace_reuse(fq, orc, shapes):
    """K-split calls sharing one workspace that starts full of NaN bit patterns:
    every partial a call reads, the same call wrote."""
    from fp8_weight_quantized_amd import _lib
    L = _lib.lib()
    need = max(L.fp8q_linear_workspace_size(0, m, n, k) for m, n, k in shapes)
    assert need > 0
    ws_buf = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    for i, (m, n, k) in enumerate(shapes):
        w = workloads.heavy_tail_weight(n, k, 50 + i)
        x = workloads.normal_act(m, k, 60 + i)
        wq, wsc, _ = orc.quantize_weight(w)
        xd, wd = pad8_bf16(x), pad16(wq)
        wsd = torch.from_numpy(wsc).cuda()
        y = torch.empty((m, (n + 7) // 8 * 8), dtype=torch.bfloat16, device="cuda")[:, :n]
        say("w8a16 workspace reuse", m, n, k, fq.describe_linear(0, m, n, k))
        assert "splits=1 " not in fq.describe_linear(0, m, n, k)
        for rep in range(2):
            st = L.fp8q_linear(0, xd.data_ptr(), m, k, xd.stride(0), None, wd.data_ptr(), n,
                               wd.stride(0), wsd.data_ptr(), y.data_ptr(), y.stride(0),
                               ws_buf.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
            assert st == 0, _lib.last_error()
            torch.cuda.synchronize()
            assert_gemm_close(host_bf16_as_f64(y), orc.linear(0, x, wq, wsc),
                              f"reuse {m}x{n}x{k} call {rep}")


def test_panel_plans_are_taken(fq):
    """The panel shapes above run k_w8a16_panel in every mode (so their parity
    tests cover it)."""
    for m, n, k in PANEL_SHAPES:
        for mode in (0, 1, 2):
            assert fq.describe_linear(mode, m, n, k).startswith("k_w8a16_panel"), (mode, m, n, k)


def test_deterministic(fq, orc):
    w = workloads.heavy_tail_weight(1024, 8192, 3)
    wq, ws = fq.quantize_weight(dev_bf16(w))
    x = dev_bf16(workloads.normal_act(12, 8192, 4))
    say("determinism w8a16 split-K")
    y1 = fq.linear(x, wq, ws)
    y2 = fq.linear(x, wq, ws)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    xq, xs = fq.quantize_act(dev_bf16(workloads.normal_act(512, 8192, 5)))
    say("determinism w8a8")
    z1 = fq.linear(xq, wq, ws, x_scale=xs)
    z2 = fq.linear(xq, wq, ws, x_scale=xs)
    assert torch.equal(z1.view(torch.int16), z2.view(torch.int16))
    wp, wps = fq.quantize_weight(dev_bf16(workloads.heavy_tail_weight(4096, 4096, 6)))
    xp = dev_bf16(workloads.normal_act(64, 4096, 7))
    say("determinism w8a16 panel", fq.describe_linear(0, 64, 4096, 4096))
    p1 = fq.linear(xp, wp, wps)
    p2 = fq.linear(xp, wp, wps)
    assert torch.equal(p1.view(torch.int16), p2.view(torch.int16))


def test_host_pointer_and_device_checks(fq):
    """Boundary errors the library turns into statuses before launching."""
    from fp8_weight_quantized_amd import _lib
    L = _lib.lib()
    stream = torch.cuda.current_stream().cuda_stream
    host = torch.zeros((16, 64), dtype=torch.uint8).pin_memory()
    dev_w = torch.zeros((16, 64), dtype=torch.uint8, device="cuda")
    ws = torch.ones(16, dtype=torch.float32, device="cuda")
    y = torch.empty((4, 16), dtype=torch.bfloat16, device="cuda")
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda")
    # pinned host memory passed where device memory is required
    st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, host.data_ptr(), 16, 64,
                       ws.data_ptr(), y.data_ptr(), 16, None, 0, stream)
    assert st == 1, L.fp8q_last_error()
    # plain host (pageable) memory
    buf = np.zeros(4096, np.uint8)
    st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, buf.ctypes.data, 16, 64,
                       ws.data_ptr(), y.data_ptr(), 16, None, 0, stream)
    assert st == 1, L.fp8q_last_error()
    # null weight pointer
    st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, None, 16, 64,
                       ws.data_ptr(), y.data_ptr(), 16, None, 0, stream)
    assert st == 1
    # misaligned pointer
    st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, dev_w.data_ptr() + 8, 16, 64,
                       ws.data_ptr(), y.data_ptr(), 16, None, 0, stream)
    assert st == 1
    # output overlapping the activation
    st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, dev_w.data_ptr(), 16, 64,
                       ws.data_ptr(), x.data_ptr(), 16, None, 0, stream)
    assert st == 1
    # a valid call still works afterwards
    st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, dev_w.data_ptr(), 16, 64,
                       ws.data_ptr(), y.data_ptr(), 16, None, 0, stream)
    assert st == 0, L.fp8q_last_error()
    torch.cuda.synchronize()
    assert (y.float() == 0).all()
    # the allocations remembered by the valid call admit no host memory
    for hp in (host.data_ptr(), buf.ctypes.data):
        st = L.fp8q_linear(0, x.data_ptr(), 4, 64, 64, None, hp, 16, 64,
                           ws.data_ptr(), y.data_ptr(), 16, None, 0, stream)
        assert st == 1, L.fp8q_last_error()


@pytest.mark.parametrize("mode,m,n,k", [(1, 300, 300, 256), (1, 520, 1000, 384), (1, 300, 300, 200),
                                        (1, 257, 9, 128), (0, 12, 300, 8192), (0, 64, 1000, 4096),
                                        (0, 48, 4000, 2048), (0, 300, 300, 200), (0, 520, 1000, 384)])
def test_output_stride_guard(fq, orc, mode, m, n, k):
    """Y written into a wider buffer (ld_y = n rounded up to 8, plus 24) with
    rows to spare: every element past column n or row m keeps its sentinel,
    and the [m, n] block is in tolerance.  Covers the prefill GEMM's staged
    row stores (ragged last 16-byte chunk) and the decode kernels."""
    from fp8_weight_quantized_amd import _lib
    L = _lib.lib()
    w = workloads.heavy_tail_weight(n, k, 70 + m)
    wq, ws, _ = orc.quantize_weight(w)
    if mode == 1:
        xq, xs, _ = orc.quantize_act(workloads.outlier_act(m, k, 80 + m))
        xd, ref = pad16(xq), orc.linear(1, xq, wq, ws, xs)
        xsd = torch.tensor([xs], dtype=torch.float32, device="cuda")
    else:
        x = workloads.normal_act(m, k, 80 + m)
        xd, ref, xsd = pad8_bf16(x), orc.linear(0, x, wq, ws), None
    wd, wsd = pad16(wq), torch.from_numpy(ws).cuda()
    ld_y = (n + 7) // 8 * 8 + 24
    sentinel = 0x7FC1
    ybuf = torch.full((m + 3, ld_y), sentinel, dtype=torch.int16, device="cuda")
    need = L.fp8q_linear_workspace_size(mode, m, n, k)
    wk = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    say("output stride guard", mode, m, n, k, fq.describe_linear(mode, m, n, k))
    st = L.fp8q_linear(mode, xd.data_ptr(), m, k, xd.stride(0),
                       xsd.data_ptr() if xsd is not None else None, wd.data_ptr(), n, wd.stride(0),
                       wsd.data_ptr(), ybuf.data_ptr(), ld_y, wk.data_ptr(), need,
                       torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.last_error()
    torch.cuda.synchronize()
    yb = ybuf.cpu().numpy()
    assert (yb[:m, n:] == sentinel).all(), "wrote past column n"
    assert (yb[m:, :] == sentinel).all(), "wrote past row m"
    y = host_bf16_as_f64(ybuf[:m, :n].view(torch.bfloat16))
    assert_gemm_close(y, ref, f"stride guard mode {mode} {m}x{n}x{k}")


@pytest.mark.parametrize("mode", [0, 1, 2])
def test_mid_rows_route_by_cost(fq, mode):
    """65..1024 rows: the decode kernels where the GEMM's grid would be one
    round of a few tiles (Llama-3-8B q_proj at 128 rows), the GEMMs on a wide
    weight (gate+up at 512 rows) and past 1024 rows."""
    assert fq.describe_linear(mode, 128, 4096, 4096).startswith("k_w8a16_panel<4, 2,")
    gemm = "k_w8a8 " if mode == 1 else "k_w8a16_gemm<"
    assert fq.describe_linear(mode, 512, 28672, 4096).startswith(gemm)
    assert fq.describe_linear(mode, 1025, 4096, 4096).startswith(gemm)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("m", [65, 128, 200, 256, 512])
def test_mid_rows_q_proj(fq, orc, mode, m):
    """Llama-3-8B q_proj (N = K = 4096) at 65..256 rows, on the decode panel
    kernel with 64 weight rows x 32 activation rows per workgroup (two or one
    chunks in flight per wave), against the oracle."""
    wl = workloads.WORKLOADS["q_proj_decode"]
    lin = wl.linears[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    say("mid rows q_proj", mode, m, fq.describe_linear(mode, m, lin.n, lin.k))
    assert fq.describe_linear(mode, m, lin.n, lin.k).startswith("k_w8a16_panel<4, 2,")
    if mode == 1:
        xq, xs, _ = orc.quantize_act(workloads.activation(wl, m, lin.k))
        y = run_w8a8(fq, xq, xs, wq, ws)
        ref = orc.linear(1, xq, wq, ws, xs)
    elif mode == 0:
        x = workloads.activation(wl, m, lin.k)
        y = run_w8a16(fq, x, wq, ws)
        ref = orc.linear(0, x, wq, ws)
    else:
        x = f16_act(m, lin.k, 77 + m)
        y = run_w8a16_f16(fq, x, wq, ws)
        ref = orc.linear(2, x, wq, ws)
    assert_gemm_close(y, ref, f"mid rows q_proj mode {mode} m={m}")


# 17..64 rows on weights of 6145..16384 rows: 64-row panels in one round of
# workgroups (16-row or 32-row activation groups), where the 32-row panels
# would need more than one round
WIDE_ONE_ROUND = [(17, 6144, 2048, "k_w8a16_panel<4, 1, 2, 3, 4>"),
                  (32, 8192, 4096, "k_w8a16_panel<4, 1, 2, 3, 4>"),
                  (24, 14336, 2048, "k_w8a16_panel<4, 2, 2, 2, 4>"),
                  (48, 8192, 2048, "k_w8a16_panel<4, 2, 2, 2, 4>"),
                  (64, 6000, 2560, "k_w8a16_panel<4, 2, 2, 2, 4>")]


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("m,n,k,kernel", WIDE_ONE_ROUND)
def test_panel_wide_one_round(fq, orc, mode, m, n, k, kernel):
    plan = fq.describe_linear(mode, m, n, k)
    assert plan.startswith(kernel), plan
    w = workloads.heavy_tail_weight(n, k, 60 + m)
    wq, ws, _ = orc.quantize_weight(w)
    say("wide one-round panel", mode, m, n, k, plan)
    if mode == 1:
        xq, xs, _ = orc.quantize_act(workloads.outlier_act(m, k, 61 + m))
        y = run_w8a8(fq, xq, xs, wq, ws)
        ref = orc.linear(1, xq, wq, ws, xs)
    elif mode == 0:
        x = workloads.normal_act(m, k, 62 + m)
        y = run_w8a16(fq, x, wq, ws)
        ref = orc.linear(0, x, wq, ws)
    else:
        x = f16_act(m, k, 63 + m)
        y = run_w8a16_f16(fq, x, wq, ws)
        ref = orc.linear(2, x, wq, ws)
    assert_gemm_close(y, ref, f"wide one-round panel mode {mode} {m}x{n}x{k}")
