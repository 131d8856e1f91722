"""GPU parity at the size limits of the boundary.

The kernels address one head's rows through 32-bit byte offsets, so a
request must keep N * row_stride * 2 bytes below 2^31 (`bsa_plan_create`
refuses larger ones, checked on the host in test_host_lib).  In the
token-major layout (NHD, rows of H*d elements) the benchmark sizes stay far
below that bound; this test runs a request just under it: 60 heads x 131,072
tokens x d = 128 (a 2.01e9-byte row range), i.i.d. blocks of 128 x 128 at 1%
plus the diagonal (Tessera paper, section 4.4: the layout is a tensor
property of the request; section 2.2: the output is the masked attention of
every row), with the table's plan and with a forced split-K plan.  Checks:
the whole output is written and finite and bounded by max|V|, and sampled
rows of the first and last head (first, last and 64 random rows) match the
fp64 oracle.
"""

import numpy as np
import pytest
import torch

import dynamic_block_sparse_bsa_amd as bsa
from oracle import attention as oatt
from workloads import gen

from bsa_testutil import MAX_ERR, MEAN_ERR

pytestmark = pytest.mark.gpu


def test_offsets_near_the_32bit_limit():
    H, N, d, block = 60, 131072, 128, (128, 128)
    assert 1.8 * 2**30 < N * H * d * 2 < 2**31
    dev = torch.device("cuda")
    M = gen.mask_iid_diag(H, N, *block, p=0.01, seed=3131)
    Md = torch.from_numpy(M).to(dev)
    q, k, v = gen.qkv_device((N, H, d), (3132, 3133, 3134), dev)  # NHD: [N][H][d]
    heads = [0, H - 1]
    rng = np.random.default_rng(3135)
    rows = {i: np.unique(np.concatenate([rng.integers(0, N, 64), [0, N - 1]])) for i in range(len(heads))}
    qh, kh, vh = (t[:, heads, :].permute(1, 0, 2).contiguous().cpu() for t in (q, k, v))
    ref = oatt.attention_rows(qh, kh, vh, M[heads], *block, rows)
    vmax = float(v.abs().amax())
    for fs in (-1, 12):  # the table's plan, and split-K partitions of 12 entries
        p = bsa.plan(Md, block, H, N, d, force_split=fs, layout="NHD")
        label = f"plan {p.info['plan_id']} split {fs}"
        out = torch.full((N, H, d), float("nan"), dtype=torch.bfloat16, device=dev)
        bsa.run(p, q, k, v, out)
        torch.cuda.synchronize()
        p.destroy()
        assert bool(torch.isfinite(out).all()), f"{label}: unwritten or non-finite output"
        assert float(out.abs().amax()) <= vmax, f"{label}: |o| above max|v|"
        for i, h in enumerate(heads):
            o = out[torch.as_tensor(rows[i], device=dev), h].float().cpu().numpy().astype(np.float64)
            err = np.abs(o - ref[i])
            assert err.max() <= MAX_ERR and err.mean() <= MEAN_ERR, \
                f"{label} head {h}: max {err.max():.3e} mean {err.mean():.3e}"
        del out
