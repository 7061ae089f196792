"""The bf16 grouped GEMMs' addressing, on the host (tests/gemm_address_model.py):
for the small parity layers and the seeded random shapes the GPU tests run,
every copy, store and exponent index of both launches is in bounds and every
output piece is written exactly once."""
import numpy as np
import pytest

import moe_inputs as mi
import oracle as o
from gemm_address_model import check, configs
from helpers import random_shapes

def _bf16_token_path(c):
    """Shapes that run the bf16 grouped GEMMs (not the fp32 kernels, not the decode path)."""
    decode = c["T"] <= 16 and c["H"] % 2048 == 0 and c["Im"] % 256 == 0
    return c.get("dtype", mi.BF16) == mi.BF16 and not decode


SHAPES = [c for c in random_shapes() if _bf16_token_path(c)] + [
    dict(name="denoise", T=4096, H=4096, E=64, k=8, Im=1536, micro=1),
    dict(name="h448_im160_two_micro", T=200, H=448, E=6, k=3, Im=160, micro=2),
    dict(name="h64_im32", T=100, H=64, E=4, k=2, Im=32, micro=1),
    dict(name="one_token_all_experts", T=1, H=256, E=64, k=64, Im=128, micro=1, Is=640),
]


@pytest.mark.parametrize("c", SHAPES, ids=[c["name"] for c in SHAPES])
def test_gemm_addresses_in_bounds(c):
    T, H, E, k, Im, mu, Is = c["T"], c["H"], c["E"], c["k"], c["Im"], c["micro"], c.get("Is", 0)
    rng = np.random.default_rng(T * 7 + H)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)])
    counts = o.expert_counts(ids, E)
    offsets = o.expert_offsets(counts)
    perm, _ = o.route_permutation(ids)
    w13, down = configs(Im, Is)
    check(w13, T, H, E, k, Im, mu, perm, offsets, Is)
    check(down, T, H, E, k, Im, mu, perm, offsets, Is)
