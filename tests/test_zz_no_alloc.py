"""fp8q_linear_noalloc: the allocation-free variant of fp8q_linear, called
through the C ABI.  Its output must equal fp8q_linear's (same kernels, the
K-split partial tiles in the library's device scratch instead of a caller
workspace) and lie within the GEMM tolerance of the fp64 oracle, on two calls
in a row, the second with a smaller input; a shape whose K-split scratch
exceeds the 8 MiB maximum is refused before anything is launched.
"""
import numpy as np
import pytest

import workloads
from helpers import assert_gemm_close, dev_bf16, dev_u8, host_bf16_as_f64, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 8 << 20


@pytest.fixture(scope="module")
def L():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from fp8_weight_quantized_amd import _lib
    return _lib.lib()


def _padded(a: np.ndarray, align: int, dtype):
    """Rows with a stride rounded up to `align` elements (as the ABI requires)."""
    rows, cols = a.shape
    t = torch.zeros((rows, (cols + align - 1) // align * align), dtype=dtype, device="cuda")
    src = dev_bf16(a) if dtype == torch.bfloat16 else dev_u8(a)
    t[:, :cols] = src
    return t[:, :cols]


def _inputs(orc, mode, m, n, k, seed):
    wq, ws, _ = orc.quantize_weight(workloads.heavy_tail_weight(n, k, seed))
    if mode == 1:
        xq, xs, _ = orc.quantize_act(workloads.outlier_act(m, k, seed + 1))
        return _padded(xq, 16, torch.uint8), torch.tensor([xs], dtype=torch.float32, device="cuda"), \
            wq, ws, orc.linear(1, xq, wq, ws, xs)
    x = workloads.normal_act(m, k, seed + 1)
    return _padded(x, 8, torch.bfloat16), None, wq, ws, orc.linear(0, x, wq, ws)


def _out(m, n, fill):
    ld = (n + 7) // 8 * 8
    return torch.full((m, ld), fill, dtype=torch.bfloat16, device="cuda")[:, :n]


def _call(L, fn, mode, xd, xsd, m, k, wd, n, wsd, y, extra):
    st = fn(mode, xd.data_ptr(), m, k, xd.stride(0), xsd.data_ptr() if xsd is not None else None,
            wd.data_ptr(), n, wd.stride(0), wsd.data_ptr(), y.data_ptr(), y.stride(0), *extra,
            torch.cuda.current_stream().cuda_stream)
    return st


# (mode, m, n, k): the first call of each pair is the larger one; every shape
# splits K (so the scratch carries partial tiles between two kernels)
PAIRS = [[(1, 12, 28672, 8208), (0, 12, 1022, 7000)],
         [(1, 64, 1024, 4096), (1, 24, 1024, 8192)],
         [(0, 40, 300, 3000), (0, 12, 1000, 6000)],
         # more than 64 rows on a narrow weight: the decode kernels with K split
         [(1, 128, 1024, 4096), (0, 100, 700, 4096)]]


@pytest.mark.parametrize("pair", PAIRS)
def test_noalloc_matches_linear(L, orc, pair):
    from fp8_weight_quantized_amd import _lib
    for i, (mode, m, n, k) in enumerate(pair):
        need = L.fp8q_linear_workspace_size(mode, m, n, k)
        assert 0 < need <= SCRATCH_BYTES, (mode, m, n, k, need)
        xd, xsd, wq, ws, ref = _inputs(orc, mode, m, n, k, 100 + 10 * i + m)
        wd, wsd = _padded(wq, 16, torch.uint8), torch.from_numpy(ws).cuda()
        y_ref = _out(m, n, 0.0)
        y_na = _out(m, n, float("nan"))
        wk = torch.empty(need, dtype=torch.uint8, device="cuda")
        say("noalloc vs linear", i, mode, m, n, k)
        assert _call(L, L.fp8q_linear, mode, xd, xsd, m, k, wd, n, wsd, y_ref,
                     (wk.data_ptr(), need)) == 0, _lib.last_error()
        assert _call(L, L.fp8q_linear_noalloc, mode, xd, xsd, m, k, wd, n, wsd, y_na, ()) == 0, \
            _lib.last_error()
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ref.view(torch.int16)), (mode, m, n, k)
        assert_gemm_close(host_bf16_as_f64(y_na), ref, f"noalloc {mode} {m}x{n}x{k}")


def test_noalloc_without_split_and_refusal(L, orc):
    from fp8_weight_quantized_amd import _lib
    # no K split: no scratch needed, same result as fp8q_linear
    mode, m, n, k = 0, 1, 4096, 4096
    assert L.fp8q_linear_workspace_size(mode, m, n, k) == 0
    xd, xsd, wq, ws, ref = _inputs(orc, mode, m, n, k, 7)
    wd, wsd = _padded(wq, 16, torch.uint8), torch.from_numpy(ws).cuda()
    y = _out(m, n, 0.0)
    say("noalloc no split")
    assert _call(L, L.fp8q_linear_noalloc, mode, xd, xsd, m, k, wd, n, wsd, y, ()) == 0, \
        _lib.last_error()
    torch.cuda.synchronize()
    assert_gemm_close(host_bf16_as_f64(y), ref, "noalloc no split")
    # a K-split scratch above the maximum: refused, nothing launched (the
    # output keeps its sentinel).  16 rows of E4M3 codes on a 57344-row weight
    # (the Llama-3-70B fused gate_up) with K = 8208 (not a multiple of 512, so
    # the tile kernel) split K 3 ways: 3 * 16 * 57344 * 4 bytes.  Every buffer
    # has its full size, so nothing could be read out of bounds.
    mode, m, n, k = 1, 16, 57344, 8208
    need = L.fp8q_linear_workspace_size(mode, m, n, k)
    assert need == 3 * 16 * 57344 * 4 > SCRATCH_BYTES
    xb = torch.zeros((m, k), dtype=torch.uint8, device="cuda")
    xs1 = torch.ones(1, dtype=torch.float32, device="cuda")
    w8 = torch.zeros((n, k), dtype=torch.uint8, device="cuda")
    ws1 = torch.ones(n, dtype=torch.float32, device="cuda")
    ysent = torch.full((m, n), 0x7FC1, dtype=torch.int16, device="cuda")
    say("noalloc refusal")
    st = L.fp8q_linear_noalloc(mode, xb.data_ptr(), m, k, k, xs1.data_ptr(), w8.data_ptr(), n, k,
                               ws1.data_ptr(), ysent.data_ptr(), n,
                               torch.cuda.current_stream().cuda_stream)
    assert st == 4, st
    assert str(SCRATCH_BYTES) in _lib.last_error()
    torch.cuda.synchronize()
    assert (ysent.cpu().numpy() == 0x7FC1).all()
