"""The dense FP8 projection family (wq_a, wkv, wq_b, wo_b, main_proj) through moe_fp8_linear, against the
oracle's fp8_linear: QDQ'd x and exact sums rounded once to bf16.

Bars: outputs within max|err| <= 2e-2 * max|ref| and relative L2 <= 5e-3 (fp32 accumulation order is the
only difference from the oracle); the fp32 output mode rounds to the bf16 mode bit for bit.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import formats as F
from oracle import moe as O

from gpu_helpers import assert_within, bf16_host, dev_tensor

pytestmark = pytest.mark.gpu


def m():
    import mxfp4_routed_expert_moe_amd as lib
    return lib


def _run(N, K, M, seed=7, rows=None):
    inp = synth.make_dense_inputs(N, K, M, seed=seed)
    x, w, s = dev_tensor(inp["x"]), dev_tensor(inp["w"]), dev_tensor(inp["s"])
    y = torch.empty((M, N), dtype=torch.int16, device="cuda")
    y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    m().moe_fp8_linear(x, w, s, y=y)
    m().moe_fp8_linear(x, w, s, y_f32=y32)
    torch.cuda.synchronize()
    rows = np.arange(M) if rows is None else rows
    ref = O.fp8_linear(inp["x"][rows], inp["w"], inp["s"])
    return y, y32, ref, rows


@pytest.mark.parametrize("name", list(synth.DENSE_SHAPES))
@pytest.mark.parametrize("M", [1, 8])
def test_dense_family_at_decode_widths(name, M):
    N, K = synth.DENSE_SHAPES[name]
    y, y32, ref, rows = _run(N, K, M)
    got = bf16_host(y)
    mx, l2 = assert_within(got, ref["y"], f"{name} M={M}")
    print(f"{name} M={M}: max-err ratio {mx:.3g}, rel-L2 {l2:.3g}")
    # fp32 mode: unrounded sums that round to the bf16 mode exactly
    b = F.bf16_bits(F.bf16_rne(y32.cpu().numpy().astype(np.float64)))
    assert np.array_equal(b, y.cpu().numpy().view(np.uint16))
    assert_within(y32.cpu().numpy().astype(np.float64), ref["acc"], f"{name} fp32 M={M}")


@pytest.mark.parametrize("M", [5, 37, 64])
def test_dense_ragged_token_groups(M):
    """M not a multiple of the 16-token MFMA groups, and the largest decode width."""
    y, y32, ref, rows = _run(1280, 5120, M, seed=M)
    assert_within(bf16_host(y), ref["y"], f"wq_a M={M}")


@pytest.mark.parametrize("M", [5, 20])
def test_dense_single_run_wide_shape(M):
    """16384 output rows (a block per CU already): the whole K in one run and no reduce launch, with a
    partial 16-token group."""
    y, y32, ref, rows = _run(16384, 1280, M, seed=100 + M)
    assert_within(bf16_host(y), ref["y"], f"wq_b M={M}")
    b = F.bf16_bits(F.bf16_rne(y32.cpu().numpy().astype(np.float64)))
    assert np.array_equal(b, y.cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("M", [65, 300])
def test_dense_prefill_width(M):
    """Above 64 rows: the block-scaled grouped GEMM as one expert."""
    y, y32, ref, rows = _run(1280, 5120, M, seed=M)
    assert_within(bf16_host(y), ref["y"], f"wq_a M={M}")
    b = F.bf16_bits(F.bf16_rne(y32.cpu().numpy().astype(np.float64)))
    assert np.array_equal(b, y.cpu().numpy().view(np.uint16))


def test_dense_small_shapes_and_refusals():
    y, y32, ref, rows = _run(128, 128, 3)
    assert_within(bf16_host(y), ref["y"], "128x128")
    x = torch.zeros((2, 200), dtype=torch.int16, device="cuda")
    w = torch.zeros((128, 200), dtype=torch.uint8, device="cuda")
    s = torch.zeros((4, 7), dtype=torch.uint8, device="cuda")
    with pytest.raises(m().MoeError):
        m().moe_fp8_linear(x, w, s, y=torch.empty((2, 128), dtype=torch.int16, device="cuda"),
                           ws=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))


def test_prepare_fp8_weights_layout():
    """The fragment-order copy: out[f][q][l][b] = w[16 f + l % 16][64 q + 16 (l / 16) + b]."""
    N, K = 256, 640
    g = torch.Generator().manual_seed(3)
    w_host = torch.randint(0, 256, (N, K), dtype=torch.uint8, generator=g)
    t = m().moe_prepare_fp8_weights(w_host.cuda())
    torch.cuda.synchronize()
    want = w_host.numpy().reshape(N // 16, 16, K // 64, 4, 16).transpose(0, 2, 3, 1, 4).reshape(-1)
    assert np.array_equal(t.cpu().numpy(), want)


@pytest.mark.parametrize("name", list(synth.DENSE_SHAPES))
@pytest.mark.parametrize("M", [1, 8, 37])
def test_dense_tiled_weights_are_identical(name, M):
    """moe_fp8_linear_tiled on the prepared copy equals moe_fp8_linear on the row-major codes bit for bit
    (bf16 and fp32 outputs), at the split-K and single-run plans and a ragged 16-token group."""
    N, K = synth.DENSE_SHAPES[name]
    inp = synth.make_dense_inputs(N, K, M, seed=200 + M)
    x, w, s = dev_tensor(inp["x"]), dev_tensor(inp["w"]), dev_tensor(inp["s"])
    wt = m().moe_prepare_fp8_weights(w)
    outs = {}
    for tag in ("rows", "tiled"):
        y = torch.empty((M, N), dtype=torch.int16, device="cuda")
        y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        if tag == "rows":
            m().moe_fp8_linear(x, w, s, y=y)
            m().moe_fp8_linear(x, w, s, y_f32=y32)
        else:
            m().moe_fp8_linear_tiled(x, wt, N, s, y=y)
            m().moe_fp8_linear_tiled(x, wt, N, s, y_f32=y32)
        torch.cuda.synchronize()
        outs[tag] = (y.cpu().numpy(), y32.cpu().numpy().view(np.uint32))
    assert np.array_equal(outs["rows"][0], outs["tiled"][0]), name
    assert np.array_equal(outs["rows"][1], outs["tiled"][1]), name
