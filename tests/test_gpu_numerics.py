"""The kernels' per-element arithmetic over complete domains, against the
oracle: every (x, amax) pair of BF16 values through both tile paths' element
functions, and the saturating E4M3 cast of every fp32 bit pattern. Marked gpu."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from gpu_util import WORKERS, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wt():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from bf16_fp8_weight_amd import wt as _wt
    return _wt


X = np.arange(65536, dtype=np.uint32)
X_NAN = ((X & 0x7F80) == 0x7F80) & ((X & 0x7F) != 0)   # BF16 NaN patterns (out of contract)


def _oracle_domain(amax):
    parts = np.array_split(amax, WORKERS)
    with ThreadPoolExecutor(WORKERS) as ex:
        res = list(ex.map(oracle.quantize_domain, parts))
    return np.concatenate(res)


@pytest.mark.parametrize("path", [0, 1])
def test_quantize_domain_exhaustive(wt, path):
    # amax over 0 and every positive finite BF16 value; x over all 65,536 patterns
    amax_all = np.arange(0, 0x7F80, dtype=np.uint16)
    step = 2048
    out = torch.empty((step, 65536), dtype=torch.uint8, device="cuda")
    n_bad = 0
    n_out = 0
    for a in range(0, amax_all.size, step):
        am = amax_all[a:a + step]
        am_dev = torch.from_numpy(am.view(np.int16)).to("cuda")
        wt.wt_quantize_domain(am_dev.data_ptr(), am.size, path, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got = out[:am.size].cpu().numpy()
        want = _oracle_domain(am)
        # in contract: x is an element of a tile whose amax is am[i], so |x| <= amax
        inside = ((X[None, :] & 0x7FFF) <= am[:, None].astype(np.uint32)) & ~X_NAN[None, :]
        n_out += int(((got != want) & ~inside & ~X_NAN[None, :]).sum())
        diff = (got != want) & inside
        if diff.any():
            i, j = np.argwhere(diff)[0]
            n_bad += int(diff.sum())
            log(f"  path {path}: amax {am[i]:#06x} x {j:#06x}: got {got[i, j]:#04x} want {want[i, j]:#04x}")
    log(f"  path {path}: {amax_all.size} amax x 65536 x: {n_bad} mismatches for |x| <= amax; "
        f"{n_out} outside the contract (|x| > amax)")
    assert n_bad == 0


def test_cast_every_fp32_pattern(wt):
    step = 1 << 28
    out = torch.empty(step, dtype=torch.uint8, device="cuda")
    mism_nan = 0
    for first in range(0, 1 << 32, step):
        wt.wt_cast_f32_range(first, step, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
        got = out.cpu().numpy()
        sub = step // WORKERS
        with ThreadPoolExecutor(WORKERS) as ex:
            want = np.concatenate(list(ex.map(lambda k: oracle.cast_f32_range(first + k * sub, sub), range(WORKERS))))
        bits = np.arange(step, dtype=np.uint32) + np.uint32(first)
        is_nan = (bits & 0x7F800000) == 0x7F800000
        is_nan &= (bits & 0x7FFFFF) != 0
        d = got != want
        mism_nan += int((d & is_nan).sum())
        d &= ~is_nan
        if d.any():
            i = np.nonzero(d)[0][0]
            raise AssertionError(f"fp32 {bits[i]:#010x}: got {got[i]:#04x} want {want[i]:#04x}")
    log(f"  all 2^32 fp32 patterns: non-NaN inputs identical; NaN inputs differing: {mism_nan}")
