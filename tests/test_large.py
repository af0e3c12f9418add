"""Tensors larger than 4 GiB (row offsets beyond 2^32 bytes), in the vectorized forward, the
pair kernel and the backward: inputs are drawn on the device from a seeded torch generator
(plain torch, not this library), and the outputs are checked against the oracle on sampled
rows (forward, dx) and sampled columns (dgamma, dbeta), including rows that start beyond
the 4 GiB boundary. The backward's statistics are computed with plain torch in fp32 and
given to both sides."""

import numpy as np
import pytest
import torch

import oracle
import row_wise_normalization_fp32_amd as rn
from _compare import check_colsum, check_dx, check_mean, check_rstd, check_y

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
BF16 = torch.bfloat16
EPS = 1e-5


def _inputs(rows, N, seed, dtype=BF16):
    gen = torch.Generator(device=DEV).manual_seed(seed)
    x = torch.empty(rows, N, dtype=dtype, device=DEV)
    step = max(1, (1 << 28) // N)
    for r0 in range(0, rows, step):  # in slices: no fp32 copy of the whole tensor
        r1 = min(rows, r0 + step)
        x[r0:r1] = (torch.randn(r1 - r0, N, generator=gen, device=DEV) * 3 + 5).to(dtype)
    gamma = (torch.rand(N, generator=gen, device=DEV) + 0.5).to(dtype)
    beta = (0.1 * torch.randn(N, generator=gen, device=DEV)).to(dtype)
    return x, gamma, beta


def _rows_to_check(rows, N, s=2):
    first_beyond = (1 << 32) // (N * s) + 1  # the first row starting past 2^32 bytes
    assert first_beyond < rows
    return sorted({0, 1, rows // 2, first_beyond - 1, first_beyond, rows - 2, rows - 1})


def _forward_case(rows, N, seed, expect, variant="auto"):
    x, gamma, beta = _inputs(rows, N, seed)
    assert x.numel() * 2 > (1 << 32)
    st, info = rn.plan("ln", rows, N, BF16, ptrs={"x": x.data_ptr(), "gamma": gamma.data_ptr(),
                                                  "beta": beta.data_ptr()}, variant=variant)
    assert st == 0 and info["persistent"], info
    assert (info["variant"], info["pairs"], info["ragged"]) == expect, info
    y, mean, rstd = rn.ln_forward(x, gamma, beta, EPS, return_stats=True, variant=variant)
    torch.cuda.synchronize()
    idx = torch.tensor(_rows_to_check(rows, N), device=DEV)
    ref = oracle.layer_norm(x[idx].cpu(), gamma.cpu(), beta.cpu(), EPS)
    check_y(y[idx], ref["y"], op="ln")
    check_mean(mean[idx], ref["mean"], ref["rstd"], EPS)
    check_rstd(rstd[idx], ref["rstd"])


def test_layer_norm_beyond_4gib_vectorized():
    _forward_case(131075, 16384, 7001, ("workgroup", False, False))  # 4.3 GB per tensor


def test_layer_norm_beyond_4gib_ragged():
    # ragged rows, 4.3 GB per tensor: the byte-addressed vectorized kernel
    _forward_case(524420, 4095, 7002, ("workgroup", False, True))


def test_layer_norm_beyond_4gib_pairs():
    _forward_case(524420, 4095, 7003, ("element", True, False), variant="element")  # the pair kernel


def test_split_rows_beyond_4gib():
    # fp32 rows of 65536 elements (256 KiB): two launches through a workspace
    rows, N = 16400, 65536
    x, gamma, beta = _inputs(rows, N, 7005, torch.float32)
    ws = rn.forward_workspace_bytes("ln", rows, N, torch.float32)
    assert rn.plan("ln", rows, N, torch.float32, workspace_bytes=ws)[1]["variant"] == "wide"
    y, mean, rstd = rn.ln_forward(x, gamma, beta, EPS, return_stats=True)
    torch.cuda.synchronize()
    idx = torch.tensor(_rows_to_check(rows, N, 4), device=DEV)
    ref = oracle.layer_norm(x[idx].cpu(), gamma.cpu(), beta.cpu(), EPS)
    check_y(y[idx], ref["y"], op="ln")
    check_mean(mean[idx], ref["mean"], ref["rstd"], EPS)
    check_rstd(rstd[idx], ref["rstd"])


def test_layer_norm_backward_beyond_4gib():
    rows, N = 131075, 16384
    x, gamma, _ = _inputs(rows, N, 7003)
    dy, _, _ = _inputs(rows, N, 7004)
    mean = torch.empty(rows, device=DEV)
    rstd = torch.empty(rows, device=DEV)
    for r0 in range(0, rows, 16384):
        xf = x[r0:r0 + 16384].float()
        mean[r0:r0 + 16384] = xf.mean(1)
        rstd[r0:r0 + 16384] = torch.rsqrt(xf.var(1, unbiased=False) + EPS)
    dx, dg, db = rn.ln_backward(dy, x, mean, rstd, gamma)
    torch.cuda.synchronize()
    idx = torch.tensor(_rows_to_check(rows, N), device=DEV)
    m_s, r_s = mean[idx].cpu().numpy(), rstd[idx].cpu().numpy()
    ref = oracle.layer_norm_backward(dy[idx].cpu(), x[idx].cpu(), gamma.cpu(), mean=m_s, rstd=r_s, eps=EPS)
    xs, dys = x[idx].cpu().double().numpy(), dy[idx].cpu().double().numpy()
    xh = (xs - m_s.astype(np.float64)[:, None]) * r_s.astype(np.float64)[:, None]
    g = dys * gamma.cpu().double().numpy()[None, :]
    row = r_s.astype(np.float64) * np.abs(g).max(axis=1) * np.maximum(1.0, np.abs(xh).max(axis=1)) ** 2
    check_dx(dx[idx], ref["dx"], row)
    # parameter gradients on sampled columns: the oracle's column sums over all rows
    cols = torch.tensor([0, 1, 4097, 8191, 12345, 16383], device=DEV)
    xc, dyc = x[:, cols].cpu(), dy[:, cols].cpu()
    refc = oracle.layer_norm_backward(dyc, xc, gamma[cols].cpu(), mean=mean.cpu().numpy(),
                                      rstd=rstd.cpu().numpy(), eps=EPS)
    xhc = (xc.double().numpy() - mean.cpu().double().numpy()[:, None]) * rstd.cpu().double().numpy()[:, None]
    st, info = rn.plan_backward("ln", rows, N, BF16, ptrs={"workspace": 1 << 46})
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    depth = -(-rows // min(info["grid_blocks"], cus)) + info["rows_per_block"] + info["grid_blocks"] / 16 + 16
    check_colsum(dg[cols], refc["dgamma"], np.abs(dyc.double().numpy() * xhc).sum(axis=0), depth, "dgamma")
    check_colsum(db[cols], refc["dbeta"], np.abs(dyc.double().numpy()).sum(axis=0), depth, "dbeta")
