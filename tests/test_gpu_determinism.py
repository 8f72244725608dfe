"""Every configuration gives the same bits on every call (N(0,1) data, where
rounding would expose any change of summation order between calls): the K
order of each element is fixed by the kernel, never by timing -- the 256-row
tiles (256 and 224 wide), the 128 x 128 kernel with either ring, the skinny-K
kernel, split-K (in-order reduction) and the ragged-round plans, fp16 and
fp8; two calls of each, with other launches in between.
"""
import numpy as np
import pytest
import torch

import dense_gemm_tn_amd as dg
from dense_gemm_tn_amd import inputs
from test_gpu_parity import DEV

pytestmark = pytest.mark.gpu

CASES = [  # kind, M, N, K, forced tile (None: the library's choice), splits
    ("f16", 1000, 1100, 2000, "256", 1),
    ("f16", 1000, 1100, 2000, "224", 1),
    ("f16", 1000, 1100, 2000, "128", 1),      # 64 blocks of 32 steps: the four-stage ring
    ("f16", 3000, 3000, 1000, "128", 1),      # 576 blocks: the two-stage ring
    ("f16", 4096, 4096, 128, None, 1),        # skinny-K
    ("f16", 512, 512, 32768, None, 16),       # split-K
    ("f16", 4096, 4608, 1024, None, 1),       # a ragged-round plan
    ("f8", 1000, 1100, 4000, "256", 1),
    ("f8", 1000, 1100, 4000, "128", 1),
    ("f8", 4096, 4096, 256, None, 1),
    ("f8", 512, 512, 32768, None, 8),
]


@pytest.mark.parametrize("kind,M,N,K,tile,splits", CASES)
def test_same_bits_every_call(monkeypatch, kind, M, N, K, tile, splits):
    monkeypatch.delenv("DG_GEMM_TILE", raising=False)
    if tile:
        monkeypatch.setenv("DG_GEMM_TILE", tile)
    print("determinism %s %dx%dx%d tile %s splits %d" % (kind, M, N, K, tile, splits), flush=True)
    x = inputs.make_shape(kind, M, N, K, dist="normal", seed=M + K)
    a = torch.from_numpy(x["A"].view(np.int16) if kind == "f16" else x["A"]).to(DEV)
    b = torch.from_numpy(x["B"].view(np.int16) if kind == "f16" else x["B"]).to(DEV)
    ws = torch.empty(max(dg.lib().gemm_splitk_workspace_bytes(M, N, splits), 16) // 4,
                     dtype=torch.float32, device=DEV)

    def call():
        c = torch.empty((N, M), dtype=torch.int16, device=DEV)
        if splits > 1:
            if kind == "f16":
                dg.gemm_f16_tn_splitk(a, b, c, M, N, K, K, K, M, splits, ws, ws.numel() * 4)
            else:
                dg.gemm_f8_tn_splitk(a, b, c, M, N, K, K, K, M, x["scale_a"], x["scale_b"], splits,
                                     ws, ws.numel() * 4)
        elif kind == "f16":
            dg.gemm_f16_tn(a, b, c, M, N, K, K, K, M)
        else:
            dg.gemm_f8_tn(a, b, c, M, N, K, K, K, M, x["scale_a"], x["scale_b"])
        return c

    first = call()
    # Other work in between: a different product on the same stream.
    other = torch.randn(2048, 2048, device=DEV).half()
    torch.mm(other, other)
    second = call()
    torch.cuda.synchronize()
    assert torch.equal(first, second)
    assert bool(torch.isfinite(first.view(torch.float16 if kind == "f16" else torch.bfloat16)).all())
