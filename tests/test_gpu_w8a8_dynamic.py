"""fp8_w_fp8_a with the dynamic per-tensor activation quantization folded into
the linear layer (fp8q_linear_w8a8_dynamic; "Llama 3 精读" §3.1 step 3 for the
mode, "FP8量化与长上下文实测" §1.2 and §3.1 for the per-tensor scale).

The call must equal the oracle's per-tensor quantization of X followed by its
fp8_w_fp8_a linear layer: the scale bit for bit, the codes bit for bit (shown
exactly through a one-hot weight), and Y within the GEMM tolerance.  Shapes
cover the three decode kernels (rows, tile with a K split, panel) and the
route through the quantizer and the FP8 MFMA GEMM above 64 rows.
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


def padded_bf16(bits: np.ndarray):
    """bf16 rows with a row stride rounded up to 8 elements (as the ABI requires)."""
    rows, cols = bits.shape
    t = torch.zeros((rows, (cols + 7) // 8 * 8), dtype=torch.bfloat16, device="cuda")
    t[:, :cols] = dev_bf16(bits)
    return t[:, :cols]


def padded_u8(a: np.ndarray):
    """Codes with a row stride rounded up to 16 bytes."""
    rows, cols = a.shape
    t = torch.zeros((rows, (cols + 15) // 16 * 16), dtype=torch.uint8, device="cuda")
    t[:, :cols] = dev_u8(a)
    return t[:, :cols]


def run_dynamic(fq, x_bits, wq, ws):
    y, s = fq.linear_w8a8_dynamic(padded_bf16(x_bits), padded_u8(wq), torch.from_numpy(ws).cuda())
    torch.cuda.synchronize()
    return host_bf16_as_f64(y), np.float32(s.cpu().numpy()[0])


# (m, n, k, the GEMM kernel it takes after the absmax pass)
SHAPES = [(1, 4096, 4096, "k_w8a16_panel"), (8, 4096, 4096, "k_w8a16_panel"),
          (12, 1024, 8192, "k_w8a16_rows"), (12, 2048, 4096, "k_w8a16_panel"), (5, 256, 1000, "k_w8a16_tile"),
          (16, 28672, 512, "k_w8a16_tile"), (32, 4096, 4096, "k_act_cast<0> + k_w8a16_panel"),
          (64, 4096, 4096, "k_act_cast<0> + k_w8a16_panel"), (40, 300, 3000, "k_w8a16_tile"),
          (3, 100, 13, "k_w8a16"), (12, 8192, 8192, "k_w8a16_panel"),
          (2, 28672, 2048, "k_w8a16_panel"), (13, 3000, 2560, "k_w8a16_panel"),
          (65, 520, 1000, "k_act_cast<0> + k_w8a16_tile"), (300, 256, 4096, "k_act_cast<0> + k_w8a16_tile"),
          (1100, 520, 1000, "k_act_cast<0> + k_w8a8"), (300, 28672, 1024, "k_act_cast<0> + k_w8a8")]


@pytest.mark.parametrize("m,n,k,kern", SHAPES)
def test_dynamic_matches_quantize_then_linear(fq, orc, m, n, k, kern):
    w = workloads.heavy_tail_weight(n, k, 900 + m)
    x = workloads.outlier_act(m, k, 910 + k)
    wq, ws, _ = orc.quantize_weight(w)
    oxq, oxs, _ = orc.quantize_act(x)
    desc = fq.describe_linear(1, m, n, k, dynamic=True)
    assert kern in desc, desc
    say("w8a8 dynamic", m, n, k, desc)
    y, s = run_dynamic(fq, x, wq, ws)
    assert s.view(np.uint32) == np.float32(oxs).view(np.uint32), (s, oxs)
    assert_gemm_close(y, orc.linear(1, oxq, wq, ws, oxs), f"dynamic {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(4, 512, 512), (12, 1024, 8192), (5, 256, 1024),
                                   (40, 4096, 2048), (20, 3200, 3072), (64, 4096, 4096),
                                   # the panel kernel staging 4, 8 and 16 rows
                                   (3, 4096, 2048), (7, 2048, 2048), (12, 8192, 2048),
                                   (2, 28672, 2048)])
def test_dynamic_codes_exact(fq, orc, m, n, k):
    """One-hot weight rows (code 1.0 at column p_n, scale 1) make
    Y[i, n] = s_x * dec(q(X[i, p_n])); with max|X| = 448 the scale is exactly 1,
    so Y shows every code the kernel formed, bit for bit."""
    rng = np.random.default_rng(m * 7 + n)
    # bf16 patterns of every magnitude below 448 (exponents 2^-14 .. 2^8), both signs
    e = rng.integers(113, 135, size=(m, k)).astype(np.uint32)
    man = rng.integers(0, 128, size=(m, k)).astype(np.uint32)
    sgn = rng.integers(0, 2, size=(m, k)).astype(np.uint32)
    bits = (sgn << 15) | (e << 7) | man
    f = workloads.bf16_bits_to_f32(bits.astype(np.uint16))
    bits[np.abs(f) > 448] = 0x43E0                     # 448.0
    bits[0, 0] = 0xC3E0                                 # -448.0: the maximum
    x = bits.astype(np.uint16)
    p = (np.arange(n) * 37) % k
    wq = np.zeros((n, k), np.uint8)
    wq[np.arange(n), p] = 0x38                          # 1.0
    ws = np.ones(n, np.float32)
    oxq, oxs, _ = orc.quantize_act(x)
    assert oxs == np.float32(1.0)
    say("w8a8 dynamic exact codes", m, n, k, fq.describe_linear(1, m, n, k, dynamic=True))
    y, s = run_dynamic(fq, x, wq, ws)
    assert s == np.float32(1.0)
    want = np.array([orc.e4m3_value(int(c)) for c in range(256)])[oxq[:, p]]
    assert (y == want).all(), np.argwhere(y != want)[:5]


def test_dynamic_mlp_prefill_full_size_sampled(fq, orc):
    """Llama-3-8B gate+up prefill through the dynamic entry point (quantizer +
    FP8 MFMA GEMM): scale bit-exact, every 256 x 256 output tile sampled."""
    wl = workloads.WORKLOADS["mlp_prefill"]
    lin = wl.linears[0]
    m = wl.ms[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    x = workloads.activation(wl, m, lin.k)
    say("w8a8 dynamic mlp prefill")
    y, s = fq.linear_w8a8_dynamic(dev_bf16(x), dev_u8(wq), torch.from_numpy(ws).cuda())
    torch.cuda.synchronize()
    oxq, oxs, _ = orc.quantize_act(x)
    assert np.float32(s.cpu().numpy()[0]).view(np.uint32) == np.float32(oxs).view(np.uint32)
    rows = rows_every_tile(m, 11)
    got = host_bf16_as_f64(y[torch.from_numpy(rows).cuda()])
    assert_gemm_close(got, orc.linear(1, oxq, wq, ws, oxs, rows=rows), "dynamic mlp prefill")


@pytest.mark.parametrize("m", [1, 8, 32, 64])
def test_dynamic_q_proj_decode_full(fq, orc, m):
    wl = workloads.WORKLOADS["q_proj_decode"]
    lin = wl.linears[0]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    x = workloads.activation(wl, m, lin.k)
    oxq, oxs, _ = orc.quantize_act(x)
    say("w8a8 dynamic q_proj", m)
    y, s = run_dynamic(fq, x, wq, ws)
    assert s.view(np.uint32) == np.float32(oxs).view(np.uint32)
    assert_gemm_close(y, orc.linear(1, oxq, wq, ws, oxs), f"dynamic q_proj M={m}")


@pytest.mark.parametrize("idx", range(7))
def test_dynamic_layer_decode_70b(fq, orc, idx):
    wl = workloads.WORKLOADS["layer_decode_70b"]
    lin = wl.linears[idx]
    wq, ws, _ = orc.quantize_weight(workloads.weight(wl, lin))
    x = workloads.activation(wl, 12, lin.k)
    oxq, oxs, _ = orc.quantize_act(x)
    say("w8a8 dynamic 70b layer", lin.name, fq.describe_linear(0, 12, lin.n, lin.k))
    y, s = run_dynamic(fq, x, wq, ws)
    assert s.view(np.uint32) == np.float32(oxs).view(np.uint32)
    assert_gemm_close(y, orc.linear(1, oxq, wq, ws, oxs), lin.name)


def test_dynamic_nonfinite_flag(fq):
    m, n, k = 8, 256, 1024
    x = workloads.normal_act(m, k, 3)
    wq = np.full((n, k), 0x38, np.uint8)
    ws = np.ones(n, np.float32)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("w8a8 dynamic finite input")
    fq.linear_w8a8_dynamic(dev_bf16(x), dev_u8(wq), torch.from_numpy(ws).cuda(), nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    x[3, 100] = 0x7F80                                  # +Inf
    say("w8a8 dynamic non-finite input")
    fq.linear_w8a8_dynamic(dev_bf16(x), dev_u8(wq), torch.from_numpy(ws).cuda(), nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1


def test_dynamic_nonfinite_flag_single_launch(fq, orc):
    """The same flag and scale when the panel kernel's workgroups take the
    absmax themselves (8 x 2048 activations, one launch)."""
    m, n, k = 8, 4096, 2048
    assert "absmax and cast in the kernel" in fq.describe_linear(1, m, n, k, dynamic=True)
    x = workloads.outlier_act(m, k, 4)
    wq, ws, _ = orc.quantize_weight(workloads.heavy_tail_weight(n, k, 5))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    say("w8a8 dynamic single launch, finite input")
    y, s = fq.linear_w8a8_dynamic(padded_bf16(x), padded_u8(wq), torch.from_numpy(ws).cuda(),
                                  nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 0
    oxq, oxs, _ = orc.quantize_act(x)
    assert np.float32(s.cpu().numpy()[0]).view(np.uint32) == np.float32(oxs).view(np.uint32)
    assert_gemm_close(host_bf16_as_f64(y), orc.linear(1, oxq, wq, ws, oxs), "single launch")
    x[5, 2047] = 0xFF80                                  # -Inf
    say("w8a8 dynamic single launch, non-finite input")
    fq.linear_w8a8_dynamic(padded_bf16(x), padded_u8(wq), torch.from_numpy(ws).cuda(),
                           nonfinite_flag=flag)
    torch.cuda.synchronize()
    assert int(flag.item()) == 1


def test_dynamic_workspace_reuse_and_stride_guard(fq, orc):
    """Calls sharing one NaN-filled workspace, Y written into a wider buffer:
    nothing past column n or row m changes, and each call is in tolerance."""
    from fp8_weight_quantized_amd import _lib
    L = _lib.lib()
    shapes = [(12, 1024, 8192), (5, 256, 1000), (64, 4096, 4096), (100, 300, 640)]
    need = max(L.fp8q_linear_w8a8_dynamic_workspace_size(*s) for s in shapes)
    wk = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i, (m, n, k) in enumerate(shapes):
        w = workloads.heavy_tail_weight(n, k, 70 + i)
        x = workloads.normal_act(m, k, 80 + i)
        wq, ws, _ = orc.quantize_weight(w)
        oxq, oxs, _ = orc.quantize_act(x)
        xd, wd, wsd = padded_bf16(x), padded_u8(wq), torch.from_numpy(ws).cuda()
        ld_y = (n + 7) // 8 * 8 + 16
        ybuf = torch.full((m + 2, ld_y), 0x7FC1, dtype=torch.int16, device="cuda")
        say("w8a8 dynamic reuse", m, n, k)
        st = L.fp8q_linear_w8a8_dynamic(xd.data_ptr(), m, k, xd.stride(0), wd.data_ptr(), n,
                                        wd.stride(0), wsd.data_ptr(),
                                        ybuf.data_ptr(), ld_y, None, wk.data_ptr(), need, None,
                                        stream)
        assert st == 0, _lib.last_error()
        torch.cuda.synchronize()
        yb = ybuf.cpu().numpy()
        assert (yb[:m, n:] == 0x7FC1).all() and (yb[m:, :] == 0x7FC1).all()
        y = host_bf16_as_f64(ybuf[:m, :n].view(torch.bfloat16))
        assert_gemm_close(y, orc.linear(1, oxq, wq, ws, oxs), f"reuse {m}x{n}x{k}")
