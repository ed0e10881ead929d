"""The allocation-free inference product (quip_qmatvec_rht_noalloc, for callers
that cannot allocate: code under graph capture, tight serving loops) against the
workspace entry point quip_qmatvec_rht, through the C ABI: the same kernels on
the same inputs, so the outputs must agree bit for bit. Two calls in a row, the
second smaller, so the second reuses the scratch the first left behind."""
import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_quip_amd as Q
import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(seed, m, n, bits):
    r = np.random.default_rng(seed)
    codes = r.integers(0, 1 << bits, (m, n)).astype(np.uint8)
    scales = r.uniform(0.5, 1.5, m).astype(np.float32)
    sl = np.where(r.random(m) < 0.5, -1.0, 1.0).astype(np.float32)
    sr = np.where(r.random(n) < 0.5, -1.0, 1.0).astype(np.float32)
    x = wl.gaussian_rows(seed, 1, n)[0]
    return codes, scales, sl, sr, x


def _run(seed, m, n, bits):
    codes, scales, sl, sr, x = _case(seed, m, n, bits)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    packed = torch.empty((m, Q.quip_packed_row_bytes(n, bits)), dtype=torch.uint8, device=DEV)
    Q.quip_pack_codes(d(codes), bits, packed)
    args = (packed, n, bits, d(scales), d(sl), d(sr), d(x))
    y_ws = torch.full((m,), float("nan"), device=DEV)
    Q.quip_qmatvec_rht(*args, y_ws)
    y_na = torch.full((m,), float("nan"), device=DEV)
    Q.quip_qmatvec_rht_noalloc(*args, y_na)
    torch.cuda.synchronize()
    return y_ws.cpu().numpy(), y_na.cpu().numpy(), (codes, scales, sl, sr, x)


def test_noalloc_product_equals_the_workspace_product_on_two_calls():
    print("noalloc: 4096 x 4096, 2 bits", flush=True)
    y_ws, y_na, _ = _run(11, 4096, 4096, 2)
    assert np.array_equal(y_ws, y_na)
    print("noalloc: 512 x 2048, 4 bits (smaller, second call)", flush=True)
    y_ws, y_na, (codes, scales, sl, sr, x) = _run(12, 512, 2048, 4)
    assert np.array_equal(y_ws, y_na)
    ref = O.qmatvec_rht(codes, scales, 16, sl, sr, x)
    assert np.linalg.norm(y_na - ref) <= 1e-5 * np.linalg.norm(ref)


def test_noalloc_product_rejects_unsupported_shapes():
    codes, scales, sl, sr, x = _case(13, 64, 1024, 2)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)  # noqa: E731
    packed = torch.zeros((64, 512), dtype=torch.uint8, device=DEV)
    y = torch.empty(64, device=DEV)
    with pytest.raises(Q.QuipError):
        Q.quip_qmatvec_rht_noalloc(packed, 1000, 2, d(scales), d(sl), d(sr), d(x), y)
    with pytest.raises(Q.QuipError):
        Q.quip_qmatvec_rht_noalloc(packed, 1024, 9, d(scales), d(sl), d(sr), d(x), y)
