"""moe_permute_noalloc (the permutation without a workspace argument, for
callers that cannot allocate) against moe_permute with a caller workspace and
against the oracle: bit-exact on two calls in a row, the second on a smaller
batch, both large enough to use the chunk histograms in the library's own
buffer."""

import numpy as np
import pytest
import torch

from oracle import permute as OP

from .parity import assert_equal
from .test_gpu_kernels import dev, host

pytestmark = pytest.mark.gpu


def _ids(T, E, topk, seed):
    """Distinct ids per token (a routing result), a few outside [0, E) to drop."""
    g = np.random.default_rng(seed)
    ids = np.argsort(g.random((T, E)), axis=1)[:, :topk].astype(np.int32)
    ids[::97, 0] = E + 3
    return ids


def _outputs(lib, T, topk, E, n_shared, block_m):
    k = topk + n_shared
    mt = lib.moe_permute_max_tiles(T, topk, E, n_shared, block_m)

    def filled(shape):
        return torch.full(shape, -7, dtype=torch.int32, device="cuda")

    return dict(expert_offsets=filled((E + n_shared + 1,)), sorted_pairs=filled((T * k,)),
                pair_pos=filled((T * k,)), tiles=filled((max(mt, 1), 2)), n_tiles=filled((1,)),
                n_dropped=filled((1,)))


def test_noalloc_permute_matches_workspace_variant(gpu_lib):
    lib = gpu_lib.load()
    E, n_shared, topk, block_m = 384, 1, 8, 192
    assert lib.moe_permute_noalloc_max_workspace() == 4 << 20
    for T, seed in ((16384, 1), (300, 2)):      # the second call is the smaller one
        assert lib.moe_permute_workspace(T, topk, E, n_shared, block_m) > 0
        ids_np = _ids(T, E, topk, seed)
        ids = dev(ids_np)
        ref = gpu_lib.moe_permute(ids, E, n_shared, block_m)
        out = _outputs(lib, T, topk, E, n_shared, block_m)
        gpu_lib.moe_permute_noalloc(ids, E, n_shared, block_m, out)
        torch.cuda.synchronize()
        for key in ("expert_offsets", "sorted_pairs", "pair_pos", "n_tiles", "n_dropped"):
            assert_equal(host(out[key]), host(ref[key]), f"T={T} {key}")
        nt = int(host(ref["n_tiles"])[0])
        assert_equal(host(out["tiles"])[:nt], host(ref["tiles"])[:nt], f"T={T} tiles")
        want = OP.moe_permute(ids_np, E, n_shared, block_m)
        assert_equal(host(out["sorted_pairs"]), want["sorted_pairs"], f"T={T} sorted_pairs (oracle)")
        assert_equal(host(out["pair_pos"]), want["pair_pos"], f"T={T} pair_pos (oracle)")
        assert_equal(host(out["expert_offsets"]), want["expert_offsets"],
                     f"T={T} expert_offsets (oracle)")
