"""GPU parity of the INT4 weight-only linear layer (pkv_int4_linear) against
the float64 oracle (oracle.int4.linear) on the counter-based inputs,
element by element within |gpu - ref| <= 2e-3 + 1e-2 |ref| (the output is
bf16; accumulation fp32)."""
import numpy as np
import pytest
import torch

import decode_attention_fp8_amd as pkv
import workloads as W
from oracle import int4
from tests.gpu_state import assert_close

pytestmark = pytest.mark.gpu
dev = "cuda"


def _gpu(lay, codes=None, scales=None, workspace=True):
    x = lay.x(dev)
    w = lay.codes(dev) if codes is None else codes.to(dev)
    s = lay.scales(dev) if scales is None else scales.to(dev)
    y = torch.full((lay.batch, lay.n), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = None
    need = pkv.pkv_int4_linear_workspace(lay.batch, lay.n, lay.k)
    if workspace and need:
        # stale partials from an earlier use must not leak into y
        ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    pkv.pkv_int4_linear(x, w, s, y, ws)
    torch.cuda.synchronize()
    return y.float().cpu().numpy()


def _ref(lay, rows, codes=None, scales=None):
    x = lay.x().float().numpy().astype(np.float64)
    packed = (lay.codes(rows=rows) if codes is None else codes[rows]).numpy()
    s = (lay.scales() if scales is None else scales).float().numpy().astype(np.float64)
    return int4.linear(x, packed, s[:, rows])


@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8, 9, 16, 17, 33, 64])
@pytest.mark.parametrize("n,k", [(64, 1024), (96, 2048), (32, 4096)])
def test_small_layers_every_output(batch, n, k):
    """One to eight groups per wave, one to four token tiles, ragged batches;
    up to 8 tokens with k a multiple of 2048 take the direct-to-LDS kernel
    (x rings of 2, 4 and 8 tokens), the rest the register kernel."""
    lay = W.int4_custom(f"i4_{n}_{k}_{batch}", 40 + batch, n, k, batch)
    y = _gpu(lay)
    assert_close(y, _ref(lay, np.arange(n)), f"{lay.name}")


@pytest.mark.parametrize("batch", [9, 16, 17, 33, 64])
@pytest.mark.parametrize("n,k", [(128, 2048), (256, 1024), (384, 4096)])
@pytest.mark.parametrize("workspace", [True, False])
def test_split_inputs_every_output(batch, n, k, workspace):
    """Above 8 tokens with rows in blocks of 128: inputs split over 4 or 8
    workgroups per block (1, 2 or 8 tiles each) through the workspace, and
    the same calls without one (the register kernel)."""
    lay = W.int4_custom(f"i4s_{n}_{k}_{batch}", 70 + batch, n, k, batch)
    y = _gpu(lay, workspace=workspace)
    assert_close(y, _ref(lay, np.arange(n)), f"{lay.name} workspace={workspace}")


def test_workspace_reused_across_calls_and_shapes():
    """One workspace through successive calls of different batches and
    shapes: nothing carries over from one call to the next."""
    ws = pkv.int4_workspace(64, 384, 4096, dev)
    for i, (n, k, batch) in enumerate([(384, 4096, 64), (128, 2048, 9), (384, 4096, 33),
                                       (256, 1024, 64), (384, 4096, 64)]):
        lay = W.int4_custom(f"i4r_{i}", 110 + i, n, k, batch)
        y = torch.full((batch, n), float("nan"), dtype=torch.bfloat16, device=dev)
        pkv.pkv_int4_linear(lay.x(dev), lay.codes(dev), lay.scales(dev), y, ws)
        torch.cuda.synchronize()
        assert_close(y.float().cpu().numpy(), _ref(lay, np.arange(n)), f"call {i} {lay.name}")


@pytest.mark.parametrize("batch", [12, 64])
def test_split_kernel_unsplit_rows_sampled(batch):
    """24576 rows fill the chip: one input slice, y written directly, no
    workspace wanted. Every token of 40 sampled rows."""
    lay = W.int4_custom(f"i4u_{batch}", 90 + batch, 24576, 1024, batch)
    assert pkv.pkv_int4_linear_workspace(batch, 24576, 1024) == 0
    y = _gpu(lay)
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 127, 128, 24575], rng.integers(0, lay.n, 36)]))
    assert_close(y[:, rows], _ref(lay, rows), f"{lay.name} sampled rows")


@pytest.mark.parametrize("batch", [1, 8, 16, 64])
def test_full_size_sampled_rows(batch):
    """The benchmark's 8192 x 8192 layer: every token of 48 sampled rows
    (first and last rows of workgroups, random others)."""
    lay = W.int4_layer(batch)
    y = _gpu(lay)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, 31, 32, 8191], rng.integers(0, lay.n, 44)]))
    assert_close(y[:, rows], _ref(lay, rows), f"{lay.name} sampled rows")


@pytest.mark.parametrize("byte", [0x88, 0x77, 0x0F, 0xF0])
@pytest.mark.parametrize("k,batch", [(1024, 16), (2048, 4)])
def test_extreme_and_mixed_sign_codes(byte, k, batch):
    """All codes -8, all 7, and alternating 0 / -1 patterns, through both
    kernels."""
    lay = W.int4_custom("i4x", 50, 64, k, batch)
    codes = torch.full((64, k // 2), byte, dtype=torch.uint8)
    y = _gpu(lay, codes=codes)
    assert_close(y, _ref(lay, np.arange(64), codes=codes), f"codes 0x{byte:02x}")


def test_bad_arguments_raise():
    lay = W.int4_custom("i4b", 51, 32, 1024, 2)
    x, w, s = lay.x(dev), lay.codes(dev), lay.scales(dev)
    y = torch.empty((2, 32), dtype=torch.bfloat16, device=dev)
    with pytest.raises(ValueError):
        pkv.pkv_int4_linear(x, w[:, :256], s, y)
    with pytest.raises(ValueError):
        pkv.pkv_int4_linear(x.float(), w, s, y)
    big = W.int4_custom("i4c", 52, 32, 1024, 65)
    with pytest.raises(pkv.PkvError):
        pkv.pkv_int4_linear(big.x(dev), w, s, torch.empty((65, 32), dtype=torch.bfloat16,
                                                          device=dev))


@pytest.mark.parametrize("batch", [2, 20])
def test_codes_above_4gib_sampled_rows(batch):
    """A 32768 x 262144 layer holds 4 GiB of codes, past the 32-bit byte
    offsets of the direct-to-LDS kernels, so the register kernel (64-bit
    offsets) runs at every batch. Every token of 24 sampled rows."""
    n, k = 32768, 262144
    assert n * k // 2 > 0xFFFFFFFF
    assert pkv.pkv_int4_linear_workspace(batch, n, k) == 0
    lay = W.int4_custom(f"i4big_{batch}", 130 + batch, n, k, batch)
    y = _gpu(lay)
    torch.cuda.empty_cache()
    rng = np.random.default_rng(13)
    rows = np.unique(np.concatenate([[0, 31, 16384, n - 1], rng.integers(0, n, 20)]))
    assert_close(y[:, rows], _ref(lay, rows), f"{lay.name} sampled rows")
