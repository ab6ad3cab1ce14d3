"""Double quantisation of several weights' scales in one call, bit for bit against the oracle and
against one nf4_double_quant call per weight: ragged last groups, empty tensors, a single scale,
and more tensors than one launch carries (64)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, log

pytestmark = pytest.mark.gpu


def _scales(rng, n, zero_group=False):
    c = (np.abs(rng.standard_normal(n)).astype(np.float32) * np.float32(0.05)).astype(np.float32)
    if zero_group and n >= 512:
        c[256:512] = 0.0
    return c


@pytest.mark.parametrize("sizes", [
    [256, 257, 1, 0, 512 + 3, 917504],                 # ragged ends, an empty tensor, one scale, a full weight
    [300 + 7 * i for i in range(70)],                  # 70 tensors: two launches
])
def test_double_quant_many_matches_oracle_and_single_calls(sizes):
    import bit_nf4_quantised_amd as q
    log(f"[dq_many] {len(sizes)} tensors, {sum(sizes)} scales")
    rng = np.random.default_rng(len(sizes))
    host = [_scales(rng, n, zero_group=(i == 5)) for i, n in enumerate(sizes)]
    absmax = [torch.from_numpy(h).to(dev()) for h in host]
    codes = [torch.full((n,), 0xAB, dtype=torch.uint8, device=dev()) for n in sizes]
    c2 = [torch.full(((n + 255) // 256,), -1.0, dtype=torch.float32, device=dev()) for n in sizes]
    q.nf4_double_quant_many(absmax, codes, c2)
    torch.cuda.synchronize()
    for i, (h, cd, g) in enumerate(zip(host, codes, c2)):
        rc, rg = oracle.double_quant(h)
        assert np.array_equal(cd.cpu().numpy(), rc), f"codes of tensor {i}"
        assert np.array_equal(g.cpu().numpy().view(np.uint32), rg.astype(np.float32).view(np.uint32)), \
            f"c2 of tensor {i}"
        if sizes[i]:
            one_c = torch.empty_like(cd)
            one_g = torch.empty_like(g)
            q.nf4_double_quant(absmax[i], one_c, one_g)
            torch.cuda.synchronize()
            assert torch.equal(one_c, cd) and torch.equal(one_g, g)
