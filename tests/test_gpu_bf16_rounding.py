"""bf16 outputs are rounded to nearest, ties to even, and a NaN stays a quiet
NaN: an elementwise plan i -> i (join ident, fp32 in, bf16 out) over float
bit patterns that cover every exponent, rounding ties of both parities, the
values next to them, subnormals, zeros, infinities and NaNs, compared bit by
bit with the rounding written out in integer arithmetic.

The pages do not fix the dtype's rounding; round-to-nearest-even is the
reading every bf16 result in the oracle's tolerances assumes.
"""
import numpy as np
import pytest
import torch

import tensor_relational_algebra_amd as tra
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu


def _patterns() -> np.ndarray:
    rng = np.random.default_rng(2026)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16            # every sign / exponent / top-7 mantissa
    low = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    grid = (hi[:, None] | low[None, :]).reshape(-1)           # ties of both parities and their neighbours
    rand = rng.integers(0, 1 << 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([grid, rand])


def _rne(u: np.ndarray) -> np.ndarray:
    u = u.astype(np.uint64)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF
    quiet = ((u >> 16) | 0x40) & 0xFFFF
    return np.where(nan, quiet, rounded).astype(np.uint16)


def test_bf16_output_rounds_to_nearest_even_bit_exact():
    u = _patterns()
    n = u.size
    p = tra.tra_plan("i->i", {"i": n}, {"i": 1}, "ident", "none", "f32", "bf16")
    x = torch.from_numpy(u.view(np.float32)).to(DEV)
    z = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    tra.tra_execute(p, x, None, z)
    torch.cuda.synchronize()
    got = z.cpu().view(torch.int16).numpy().view(np.uint16)
    want = _rne(u)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(u[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]
