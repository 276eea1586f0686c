"""GPU parity of per-group weight scales against the oracle.

FP8量化与长上下文实测：Llama 3 70B部署优化指南 §4.3 (per-group granularity): the
grouped quantizer must match the oracle bit for bit (codes and every group
scale), and the grouped linear layer -- all three modes of the "Llama 3 精读"
write-up §3.1 step 3 -- must stay within the GEMM tolerance of the oracle's
fp64 result computed from the same codes and scales, over group sizes,
ragged K (inside a group and inside a 64-k step), ragged N, activation row
counts from 1 to past 64, K splits, and full Llama-3 decode shapes.
"""
import numpy as np
import pytest

import workloads
from helpers import (assert_gemm_close, dev_bf16, dev_u8, host_bf16_as_f64, host_f32, host_u8,
                     rows_every_tile, say)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

GROUPS = (64, 128, 256, 512)


@pytest.fixture(scope="module")
def fq():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp8_weight_quantized_amd as fq
    fq.library_path()
    return fq


def check_quant(fq, orc, w_bits, group, what, w_dev=None):
    say("quantize_weight_grouped", what, w_bits.shape, group)
    q, s = fq.quantize_weight_grouped(dev_bf16(w_bits) if w_dev is None else w_dev, group)
    torch.cuda.synchronize()
    qr, sr, _ = orc.quantize_weight_grouped(w_bits, group)
    sg = host_f32(s)
    assert sg.shape == sr.shape
    bad = np.argwhere(sg.view(np.uint32) != sr.view(np.uint32))
    assert bad.size == 0, (what, bad[:5].tolist())
    bad = np.argwhere(host_u8(q) != qr)
    assert bad.size == 0, (what, bad[:5].tolist())
    return qr, sr


@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("n,k,seed", [(64, 512, 0), (33, 1000, 1), (7, 4096, 2), (300, 8192, 3),
                                      (5, 77, 4), (9, 300, 5), (2, 520, 6), (1, 8, 7)])
def test_quantize_shapes(fq, orc, group, n, k, seed):
    check_quant(fq, orc, workloads.heavy_tail_weight(n, k, seed), group, f"seed {seed}")


@pytest.mark.parametrize("group", GROUPS)
def test_quantize_unaligned_rows(fq, orc, group):
    w = workloads.heavy_tail_weight(11, 700, 8)
    big = np.zeros((11, 703), np.uint16)
    big[:, :700] = w
    check_quant(fq, orc, w, group, "row stride 703", dev_bf16(big)[:, :700])


def test_quantize_special_groups(fq, orc):
    w = workloads.heavy_tail_weight(4, 1024, 9)
    w[0, :] = 0                              # all-zero row: every group at the floor
    w[1, 128:256] = 0x8000                   # a group of -0
    w[2, 5] = workloads.f32_to_bf16_bits(np.array([5e4], np.float32))[0]   # one huge value
    check_quant(fq, orc, w, 128, "special groups")


@pytest.mark.parametrize("key,name", [("q_proj_decode", "q_proj"), ("mlp_prefill", "gate_up")])
def test_quantize_full_weights(fq, orc, key, name):
    wl = workloads.WORKLOADS[key]
    lin = [l for l in wl.linears if l.name == name][0]
    check_quant(fq, orc, workloads.weight(wl, lin), 128, f"{key} {name}")


def make_x(mode, m, k, seed, orc):
    if mode == 1:
        q, s, _ = orc.quantize_act(workloads.outlier_act(m, k, seed))
        return q, np.float32(s)
    x = workloads.outlier_act(m, k, seed)
    if mode == 2:
        x = workloads.bf16_bits_to_f32(x).astype(np.float16).view(np.uint16)
    return x, None


def padded(a: np.ndarray, multiple: int) -> np.ndarray:
    """a copy of the rows with the row stride rounded up (the GEMM's ld rule)"""
    k = a.shape[1]
    out = np.zeros((a.shape[0], -(-k // multiple) * multiple), a.dtype)
    out[:, :k] = a
    return out


def dev_x(mode, x):
    k = x.shape[1]
    if mode == 0:
        return dev_bf16(padded(x, 8))[:, :k]
    if mode == 2:
        return torch.from_numpy(padded(x, 8).view(np.float16)).cuda()[:, :k]
    return dev_u8(padded(x, 16))[:, :k]


def run_grouped(fq, orc, mode, m, n, k, group, seed, what=""):
    w = workloads.heavy_tail_weight(n, k, seed)
    wq, ws, _ = orc.quantize_weight_grouped(w, group)
    x, xs = make_x(mode, m, k, seed + 1, orc)
    say("linear_grouped", what, mode, m, n, k, group)
    xd = dev_x(mode, x)
    y = fq.linear(xd, dev_u8(padded(wq, 16))[:, :k], torch.from_numpy(ws).cuda(),
                  x_scale=None if xs is None else torch.tensor([xs], device="cuda"), group=group)
    torch.cuda.synchronize()
    ref = orc.linear_grouped(mode, x, wq, ws, group, x_scale=xs)
    got = y.float().cpu().numpy().astype(np.float64)
    assert_gemm_close(got, ref, f"grouped {what} mode {mode} m={m} n={n} k={k} g={group}")


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("m,n,k", [(1, 256, 4096), (5, 100, 1000), (16, 1022, 2048), (33, 64, 3000),
                                   (64, 300, 1536), (100, 128, 520)])
def test_linear_shapes(fq, orc, mode, group, m, n, k):
    run_grouped(fq, orc, mode, m, n, k, group, 1000 + m + n + k)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (8, 3000, 4096), (16, 4096, 8192),
                                   (3, 2100, 700), (12, 4096, 1000), (1, 2050, 520),
                                   (16, 8200, 2048), (2, 12000, 1100)])
def test_linear_rows_kernel(fq, orc, mode, group, m, n, k):
    """Up to 16 rows on weights of 2049 to ~16K rows.  K a multiple of 512 (from
    2048): the panel kernel; short or ragged K: the rows kernel with group
    folds at fixed steps of its 512-k rounds (N = 2100 and 2050 give 8-row
    workgroups, 8200 and 12000 32-row ones; K = 520 and 700 leave waves with
    no K range)."""
    run_grouped(fq, orc, mode, m, n, k, group, 4000 + m + n + k, "rows")


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("m,n,k", [(12, 1024, 8192), (1, 1000, 4100), (16, 2048, 16000),
                                   (5, 130, 9000)])
def test_linear_rows_kernel_k_splits(fq, orc, mode, group, m, n, k):
    """A small N on a long K: the rows kernel with K split across workgroups in
    ranges of 2048 k; each split writes its group-scaled partial sums and the
    reduce applies only the activation scale (N = 1000 and 130 leave part of
    a workgroup's rows past N; K = 4100 ends in a partial step).  1024 x 8192
    takes the panel kernel with 4 activation rows per workgroup."""
    run_grouped(fq, orc, mode, m, n, k, group, 5000 + m + n + k, "rows split")


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("m,n,k", [(12, 16448, 12000), (4, 300, 20000), (16, 4160, 17000)])
def test_linear_tile_1024k_chunks(fq, orc, mode, group, m, n, k):
    """The tile kernel with 1024-k chunks (16 steps): a weight of more than 256
    tiles with 8K <= K < 16K (K split 4 ways), or K >= 16K (K = 12000, 20000
    and 17000 leave a ragged tail of steps after the whole chunks)."""
    assert fq.describe_linear(mode, m, n, k, group=group).startswith("k_w8a16_tile<1, ")
    run_grouped(fq, orc, mode, m, n, k, group, 6000 + m + n + k, "tile 1024k")


# ---- decode on the panel kernel: per-group scales folded into the fp32
# accumulators at each group's last 64-k step (the group's scales staged by
# direct loads beside each chunk's weights)

PANEL_GROUPED = [(3, 2048, 2048, "k_w8a16_panel<1, 1,"),     # 1 weight fragment
                 (12, 6100, 2048, "k_w8a16_panel<2, 1,"),    # 2, ragged N
                 (9, 12288, 2048, "k_w8a16_panel<3, 1,"),    # 3
                 (4, 14336, 2048, "k_w8a16_panel<4, 1,"),    # 4
                 (13, 1000, 4096, "k_w8a16_panel<1, 1, 4, 2,"),  # 4 rows per workgroup
                 (5, 3000, 4096, "k_w8a16_panel<1, 1,"),     # ragged N, 1024-k wave ranges
                 (24, 4096, 2048, "k_w8a16_panel<2, 1,"),    # two 16-row activation groups
                 (40, 4096, 2048, "k_w8a16_panel<2, 2,")]    # 32-row activation groups


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", GROUPS)
@pytest.mark.parametrize("m,n,k,kernel", PANEL_GROUPED)
def test_linear_panel(fq, orc, mode, group, m, n, k, kernel):
    plan = fq.describe_linear(mode, m, n, k, group=group)
    if mode == 1 and m > 32:
        # E4M3 codes past 32 rows: the tile kernel (the panel's grouped
        # variant there would spill)
        assert plan.startswith("k_w8a16_tile"), plan
    else:
        assert plan.startswith(kernel), plan
    run_grouped(fq, orc, mode, m, n, k, group, 7000 + m + n + k + group, "panel")


# where a wave's [rows][groups] block of scales does not fit in the LDS the
# rings leave (or for E4M3 codes at 17..32 rows), the scales are staged with
# each chunk instead of preloaded
PANEL_STAGES = [(12, 6100, 16896, 64, 0, "per_chunk"), (12, 6100, 16896, 64, 1, "preloaded"),
                (12, 6100, 16896, 128, 2, "preloaded"),
                (4, 14336, 4608, 64, 2, "per_chunk"), (4, 14336, 4608, 64, 1, "preloaded"),
                (24, 4096, 2048, 128, 1, "per_chunk"), (24, 4096, 2048, 64, 1, "per_chunk"),
                (24, 4096, 2048, 64, 0, "preloaded")]


@pytest.mark.parametrize("m,n,k,group,mode,stage", PANEL_STAGES)
def test_linear_panel_scale_stages(fq, orc, m, n, k, group, mode, stage):
    plan = fq.describe_linear(mode, m, n, k, group=group)
    assert plan.startswith("k_w8a16_panel") and plan.endswith("scales=" + stage), plan
    run_grouped(fq, orc, mode, m, n, k, group, 8000 + m + n + k + group, "panel " + stage)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("m,n,k,group", [(12, 2048, 4096, 128), (13, 1000, 4096, 64),
                                         (40, 4096, 2048, 256)])
def test_linear_panel_strided(fq, orc, mode, m, n, k, group):
    """Activation and weight rows with strides beyond K (views into wider
    buffers, row pitch K + 64 values and K + 128 bytes): the panel kernel's
    per-lane offsets and the preloaded scales' addressing."""
    w = workloads.heavy_tail_weight(n, k, 31 + m)
    wq, ws, _ = orc.quantize_weight_grouped(w, group)
    x, xs = make_x(mode, m, k, 32 + m, orc)
    wbuf = torch.zeros((n, k + 128), dtype=torch.uint8, device="cuda")
    wbuf[:, :k] = dev_u8(wq)
    if mode == 1:
        xbuf = torch.zeros((m, k + 64), dtype=torch.uint8, device="cuda")
        xbuf[:, :k] = dev_u8(x)
    else:
        dt = torch.bfloat16 if mode == 0 else torch.float16
        xbuf = torch.zeros((m, k + 64), dtype=dt, device="cuda")
        xbuf[:, :k] = dev_x(mode, x)
    plan = fq.describe_linear(mode, m, n, k, group=group)
    say("grouped panel strided", mode, m, n, k, group, plan)
    y = fq.linear(xbuf[:, :k], wbuf[:, :k], torch.from_numpy(ws).cuda(),
                  x_scale=None if xs is None else torch.tensor([xs], device="cuda"), group=group)
    torch.cuda.synchronize()
    ref = orc.linear_grouped(mode, x, wq, ws, group, x_scale=xs)
    assert_gemm_close(host_bf16_as_f64(y), ref, f"strided {mode} {m}x{n}x{k} g={group}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("group", (64, 512))
def test_linear_panel_wide_scale_range(fq, orc, mode, group):
    """Adjacent groups whose scales differ by many orders of magnitude on the
    panel kernel: an all-zero group (scale at the 1e-12 floor) next to groups
    scaled up by 1e4 and down by 1e-6."""
    m, n, k = 8, 2048, 4096
    w = workloads.heavy_tail_weight(n, k, 58)
    wf = workloads.bf16_bits_to_f32(w)
    wf[:, group:2 * group] = 0.0
    wf[::3, 3 * group:4 * group] *= np.float32(1e4)
    wf[1::5, :group] *= np.float32(1e-6)
    w = workloads.f32_to_bf16_bits(wf)
    wq, ws, _ = orc.quantize_weight_grouped(w, group)
    assert (ws[:, 1] == np.float32(1e-12)).all()
    x, xs = make_x(mode, m, k, 59, orc)
    assert fq.describe_linear(mode, m, n, k, group=group).startswith("k_w8a16_panel")
    say("grouped panel wide scale range", mode, group)
    y = fq.linear(dev_x(mode, x), dev_u8(wq), torch.from_numpy(ws).cuda(),
                  x_scale=None if xs is None else torch.tensor([xs], device="cuda"), group=group)
    torch.cuda.synchronize()
    ref = orc.linear_grouped(mode, x, wq, ws, group, x_scale=xs)
    assert_gemm_close(host_bf16_as_f64(y), ref, f"panel wide scale range {mode} g={group}")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("m,n,k,group", [(1, 64, 8192, 128), (12, 128, 28672, 128),
                                         (4, 64, 12288, 64), (64, 64, 16384, 512)])
def test_linear_k_splits(fq, orc, mode, m, n, k, group):
    """Small N on long K: the K range is split across workgroups and summed."""
    run_grouped(fq, orc, mode, m, n, k, group, 2000 + k, "split")


def test_linear_agrees_with_per_channel_when_groups_share_scales(fq, orc):
    """Group scales all equal to the row scale: the grouped kernel computes the
    per-channel layer, so the two paths agree closely."""
    n, k, m = 512, 4096, 8
    w = workloads.heavy_tail_weight(n, k, 77)
    wq, ws, _ = orc.quantize_weight(w)
    x = workloads.outlier_act(m, k, 78)
    wsg = np.repeat(ws[:, None], k // 128, axis=1)
    say("grouped vs per-channel")
    y1 = fq.linear(dev_bf16(x), dev_u8(wq), torch.from_numpy(ws).cuda())
    y2 = fq.linear(dev_bf16(x), dev_u8(wq), torch.from_numpy(np.ascontiguousarray(wsg)).cuda(),
                   group=128)
    torch.cuda.synchronize()
    a, b = host_bf16_as_f64(y1), host_bf16_as_f64(y2)
    ref = orc.linear(0, x, wq, ws)
    assert_gemm_close(a, ref, "per-channel")
    assert_gemm_close(b, ref, "grouped, shared scales")


@pytest.mark.parametrize("m", [1, 12, 64])
def test_full_decode_q_proj(fq, orc, m):
    """Llama-3-8B q_proj [4096, 4096], groups of 128, fp8_w_bf16_a."""
    wl = workloads.WORKLOADS["q_proj_decode"]
    lin = wl.linears[0]
    w = workloads.weight(wl, lin)
    q, s = fq.quantize_weight_grouped(dev_bf16(w), 128)
    qr, sr, _ = orc.quantize_weight_grouped(w, 128)
    x = workloads.activation(wl, m, lin.k)
    say("grouped q_proj decode", m)
    y = fq.linear(dev_bf16(x), q, s, group=128)
    torch.cuda.synchronize()
    assert (host_u8(q) == qr).all()
    assert_gemm_close(host_bf16_as_f64(y), orc.linear_grouped(0, x, qr, sr, 128), f"q_proj m={m}")


def test_full_decode_70b_down_proj(fq, orc):
    """Llama-3-70B down_proj [8192, 28672] at decode M = 12, groups of 128."""
    wl = workloads.WORKLOADS["layer_decode_70b"]
    lin = [l for l in wl.linears if l.name == "down_proj"][0]
    w = workloads.weight(wl, lin)
    say("grouped 70b down_proj quantize")
    q, s = fq.quantize_weight_grouped(dev_bf16(w), 128)
    torch.cuda.synchronize()
    qr, sr, _ = orc.quantize_weight_grouped(w, 128)
    assert (host_u8(q) == qr).all()
    assert (host_f32(s).view(np.uint32) == sr.view(np.uint32)).all()
    del w
    x = workloads.activation(wl, 12, lin.k)
    say("grouped 70b down_proj linear")
    y = fq.linear(dev_bf16(x), q, s, group=128)
    torch.cuda.synchronize()
    rows = np.arange(12)
    assert_gemm_close(host_bf16_as_f64(y), orc.linear_grouped(0, x, qr, sr, 128, rows=rows),
                      "70b down_proj")


# ---- fp8_w_fp8_a past the decode rows: the FP8 MFMA GEMM with group scales
# folded at its 128-k stages (groups of 128, 256, 512)

@pytest.mark.parametrize("group", (128, 256, 512))
@pytest.mark.parametrize("m,n,k", [(65, 256, 128), (300, 300, 1000), (513, 1022, 4096),
                                   (130, 64, 640), (257, 100, 100), (70, 520, 1536)])
def test_w8a8_gemm_grouped(fq, orc, group, m, n, k):
    run_grouped(fq, orc, 1, m, n, k, group, 3000 + m + n + k, "gemm")


# more than 8 tile-rows, so the XCD-banded tile order has a full band and a
# partial one (80 and 51 tiles); K = 640 ends in a partial group of 256 or 512
@pytest.mark.parametrize("group", (128, 256, 512))
@pytest.mark.parametrize("m,n,k", [(2305, 2048, 640), (4100, 600, 256)])
def test_w8a8_gemm_grouped_many_tile_rows(fq, orc, group, m, n, k):
    run_grouped(fq, orc, 1, m, n, k, group, 3100 + m + n + k, "gemm, many tile-rows")


@pytest.mark.parametrize("group", (128, 512))
def test_w8a8_gemm_grouped_wide_scale_range(fq, orc, group):
    """Adjacent groups whose scales differ by many orders of magnitude: an
    all-zero group (scale at the 1e-12 floor) between large-valued groups."""
    m, n, k = 200, 256, 2048
    w = workloads.heavy_tail_weight(n, k, 55)
    wf = workloads.bf16_bits_to_f32(w)
    wf[:, group:2 * group] = 0.0                      # group 1 all zero in every row
    wf[::3, 3 * group:4 * group] *= np.float32(1e4)   # group 3 large in a third of the rows
    wf[1::5, :group] *= np.float32(1e-6)              # group 0 tiny in a fifth of the rows
    w = workloads.f32_to_bf16_bits(wf)
    wq, ws, _ = orc.quantize_weight_grouped(w, group)
    assert (ws[:, 1] == np.float32(1e-12)).all()
    xq, xs, _ = orc.quantize_act(workloads.outlier_act(m, k, 56))
    say("grouped gemm wide scale range", group)
    y = fq.linear(dev_u8(xq), dev_u8(wq), torch.from_numpy(ws).cuda(),
                  x_scale=torch.tensor([np.float32(xs)], device="cuda"), group=group)
    torch.cuda.synchronize()
    ref = orc.linear_grouped(1, xq, wq, ws, group, x_scale=xs)
    assert_gemm_close(host_bf16_as_f64(y), ref, f"wide scale range g={group}")


def test_w8a8_gemm_grouped_equals_per_channel_on_shared_scales(fq, orc):
    """Every group scale equal to the row scale: the grouped GEMM computes the
    per-channel layer (the ratios are all 1)."""
    m, n, k = 300, 512, 4096
    wq, ws, _ = orc.quantize_weight(workloads.heavy_tail_weight(n, k, 57))
    xq, xs, _ = orc.quantize_act(workloads.outlier_act(m, k, 58))
    wsg = np.ascontiguousarray(np.repeat(ws[:, None], k // 128, axis=1))
    say("grouped gemm vs per-channel gemm")
    xs_d = torch.tensor([np.float32(xs)], device="cuda")
    y1 = fq.linear(dev_u8(xq), dev_u8(wq), torch.from_numpy(ws).cuda(), x_scale=xs_d)
    y2 = fq.linear(dev_u8(xq), dev_u8(wq), torch.from_numpy(wsg).cuda(), x_scale=xs_d, group=128)
    torch.cuda.synchronize()
    ref = orc.linear(1, xq, wq, ws, xs)
    assert_gemm_close(host_bf16_as_f64(y1), ref, "per-channel gemm")
    assert_gemm_close(host_bf16_as_f64(y2), ref, "grouped gemm, shared scales")


def test_w8a8_gemm_grouped_full_mlp_prefill_sampled(fq, orc):
    """Llama-3-8B gate+up prefill, W[28672, 4096], X[8192, 4096], groups of 128:
    codes and scales bit-exact, GEMM checked on sampled rows."""
    wl = workloads.WORKLOADS["mlp_prefill"]
    lin = wl.linears[0]
    m = wl.ms[0]
    w = workloads.weight(wl, lin)
    x = workloads.activation(wl, m, lin.k)
    say("grouped mlp prefill quantize")
    q, s = fq.quantize_weight_grouped(dev_bf16(w), 128)
    xq, xs = fq.quantize_act(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr, _ = orc.quantize_weight_grouped(w, 128)
    assert (host_u8(q) == qr).all()
    assert (host_f32(s).view(np.uint32) == sr.view(np.uint32)).all()
    del w
    say("grouped mlp prefill gemm")
    y = fq.linear(xq, q, s, x_scale=xs, group=128)
    torch.cuda.synchronize()
    xqr, xsr, _ = orc.quantize_act(x)
    rows = rows_every_tile(m, 9)
    assert rows.size >= 64 and len(set(rows // 256)) == (m + 255) // 256
    ref = orc.linear_grouped(1, xqr, qr, sr, 128, x_scale=xsr, rows=rows)
    got = host_bf16_as_f64(y[torch.from_numpy(rows).cuda()])
    assert_gemm_close(got, ref, "grouped mlp prefill sampled rows")


@pytest.mark.parametrize("mode,m,n,k,group", [(1, 300, 300, 512, 128), (1, 257, 9, 256, 256),
                                              (0, 12, 300, 4096, 128)])
def test_grouped_output_stride_guard(fq, orc, mode, m, n, k, group):
    """Grouped linear written into a wider, sentinel-filled buffer: nothing
    past column n or row m changes, and the [m, n] block is in tolerance."""
    from fp8_weight_quantized_amd import _lib
    L = _lib.lib()
    w = workloads.heavy_tail_weight(n, k, 4100 + m)
    wq, ws, _ = orc.quantize_weight_grouped(w, group)
    x, xs = make_x(mode, m, k, 4200 + m, orc)
    xd = dev_x(mode, x)
    wd = dev_u8(padded(wq, 16))[:, :k]
    wsd = torch.from_numpy(ws).cuda()
    xsd = None if xs is None else torch.tensor([xs], dtype=torch.float32, device="cuda")
    ld_y = (n + 7) // 8 * 8 + 24
    sentinel = 0x7FC1
    ybuf = torch.full((m + 3, ld_y), sentinel, dtype=torch.int16, device="cuda")
    need = L.fp8q_linear_grouped_workspace_size(mode, m, n, k, group)
    wk = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    say("grouped output stride guard", mode, m, n, k, group)
    st = L.fp8q_linear_grouped(mode, xd.data_ptr(), m, k, xd.stride(0),
                               xsd.data_ptr() if xsd is not None else None, wd.data_ptr(), n,
                               wd.stride(0), wsd.data_ptr(), group, ybuf.data_ptr(), ld_y,
                               wk.data_ptr(), need, torch.cuda.current_stream().cuda_stream)
    assert st == 0, _lib.last_error()
    torch.cuda.synchronize()
    yb = ybuf.cpu().numpy()
    assert (yb[:m, n:] == sentinel).all(), "wrote past column n"
    assert (yb[m:, :] == sentinel).all(), "wrote past row m"
    got = ybuf[:m, :n].view(torch.bfloat16).float().cpu().numpy().astype(np.float64)
    ref = orc.linear_grouped(mode, x, wq, ws, group, x_scale=xs)
    assert_gemm_close(got, ref, f"grouped stride guard mode {mode} {m}x{n}x{k} g={group}")


def test_w8a8_gemm_grouped_full_down_prefill_sampled(fq, orc):
    """Llama-3-70B down_proj prefill, W[8192, 28672], X[4096, 28672], groups
    of 128: 224 groups per row, so every wave pair of the GEMM passes through
    224 rescales; codes and scales bit-exact, GEMM checked on sampled rows of
    every 256-row tile band."""
    wl = workloads.WORKLOADS["down_prefill_70b"]
    lin = wl.linears[0]
    m = wl.ms[0]
    w = workloads.weight(wl, lin)
    x = workloads.activation(wl, m, lin.k)
    say("grouped down prefill quantize")
    q, s = fq.quantize_weight_grouped(dev_bf16(w), 128)
    xq, xs = fq.quantize_act(dev_bf16(x))
    torch.cuda.synchronize()
    qr, sr, _ = orc.quantize_weight_grouped(w, 128)
    assert (host_u8(q) == qr).all()
    assert (host_f32(s).view(np.uint32) == sr.view(np.uint32)).all()
    del w
    say("grouped down prefill gemm")
    y = fq.linear(xq, q, s, x_scale=xs, group=128)
    torch.cuda.synchronize()
    xqr, xsr, _ = orc.quantize_act(x)
    rows = rows_every_tile(m, 10)
    assert rows.size >= 64 and len(set(rows // 256)) == (m + 255) // 256
    ref = orc.linear_grouped(1, xqr, qr, sr, 128, x_scale=xsr, rows=rows)
    got = host_bf16_as_f64(y[torch.from_numpy(rows).cuda()])
    assert_gemm_close(got, ref, "grouped down prefill sampled rows")
