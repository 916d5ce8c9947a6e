"""GPU parity of the NVFP4 weight quantizer through the C-ABI against the
oracle, on the same seeded bf16 weights: small ragged shapes, a whole expert
matrix and edge cases (all-zero blocks, an all-zero tensor, negative zeros).

* The per-tensor scale g: bit-exact in both modes.
* Max-based block scales and codes: bit-exact.
* MSE search: the oracle minimises the exact squared error; the kernel
  evaluates the same objective in fp32, so where two scale bytes' errors
  are closer than its evaluation error it may take the other one.  Checked
  by validity: the GPU's byte has an exact error at most EPS_MSE * sum(w^2)
  of the block above the exact minimum (bound derived in the design notes:
  twice the fp32 evaluation error), all-zero blocks take byte 0, and the
  codes are bit for bit the nearest-even codes under the GPU's own byte."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host

pytestmark = pytest.mark.gpu


def run_wq(w_bits, mse):
    rows, cols = w_bits.shape
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    g.q4moe_quantize_weights(dev(w_bits), codes, scales, gs, mode=g.WQ_MSE if mse else g.WQ_MAX)
    torch.cuda.synchronize()
    return host(codes), host(scales), np.float32(host(gs)[0])


EPS_MSE = 2.0 ** -14


def check(w_bits, mse):
    c, s, gs = run_wq(w_bits, mse)
    co, so, go = oracle.quant_weights_nvfp4(w_bits, mse=mse)
    assert gs.view(np.uint32) == go.view(np.uint32), (gs, go)
    if not mse:
        assert np.array_equal(s, so), f"{int((s != so).sum())} scale bytes differ"
        assert np.array_equal(c, co), f"{int((c != co).sum())} code bytes differ"
        return
    rows, cols = w_bits.shape
    wf = (w_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(rows, cols // 16, 16)
    energy = (wf ** 2).sum(-1)
    zero = np.abs(wf).max(-1) == 0
    assert np.all(s[zero] == 0) and np.all(so[zero] == 0)
    cg, excess = oracle.wq_codes_excess(w_bits, gs, s)
    assert np.array_equal(c, cg), f"{int((c != cg).sum())} code bytes differ from the codes under the GPU's bytes"
    assert np.all(s[~zero] >= 1) and np.all(s[~zero] <= 0x7E)
    bad = excess > EPS_MSE * energy
    assert not bad.any(), f"{int(bad.sum())} blocks exceed the MSE bound (worst {(excess / np.maximum(energy, 1e-300)).max():.3g})"
    diff = int((s != so).sum())
    print(f"MSE {rows}x{cols}: {diff} of {s.size} blocks chose another byte than the exact minimum "
          f"(largest excess / block energy {(excess / np.maximum(energy, 1e-300)).max():.3g})")


@pytest.mark.parametrize("mse", [False, True])
@pytest.mark.parametrize("rows,cols", [(1, 16), (3, 48), (37, 160), (130, 2688)])
def test_wquant_small(rows, cols, mse):
    w = synth.bf16_normal(synth.key(5, 4, rows, cols), rows * cols).reshape(rows, cols)
    check(w, mse)


@pytest.mark.parametrize("mse", [False, True])
def test_wquant_expert_matrix(mse):
    # one expert's up_proj shape, weights ~N(0, 0.02^2) as a trained layer's
    w = synth.bf16_normal(synth.key(6, 4, 0, 0), 1856 * 2688, 0.0, 0.02).reshape(1856, 2688)
    check(w, mse)


@pytest.mark.parametrize("mse", [False, True])
def test_wquant_edge_cases(mse):
    w = synth.bf16_normal(synth.key(7, 4, 0, 0), 8 * 64).reshape(8, 64)
    w[2, :16] = 0            # an all-zero block
    w[3, 16:32] = 0x8000     # a block of negative zeros
    w[4, 5] = 0x8000
    check(w, mse)
    check(np.zeros((4, 32), np.uint16), mse)  # all-zero tensor: g = 1, scales 0
