"""Context-parallel localisation of the bounds on the GPU (fm_localize_bounds)
against the oracle's count of local rows below each bound, bit for bit.

FlashMask-3 paper summary, abstract: a rank's mask comes from the global
boundary vectors by a clip-shift-max that needs no communication."""
import numpy as np
import pytest

import oracle
from column_sparse_masked_amd import masks as M
from _parity import say

pytestmark = pytest.mark.gpu


def _gpu_localize(gb, starts, lens):
    import torch
    from column_sparse_masked_amd.api import localize_bounds, to_device_bounds
    out = localize_bounds(to_device_bounds(gb), starts, lens)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def test_context_parallel_share_all_ranks():
    """The context-parallel workload's global causal-document bounds
    (S = 65536, 16 chunks of 4096), localised for each of the 8 ranks (chunks
    r and 15 - r): equal to the oracle and to the bounds the workload
    generator builds on the host."""
    world, S = 8, 65536
    base = M.cp_rank_share(H=16, S=S, D=128, world=world, rank=0, seed=5)
    gb = base.structure["global_bounds"][None, None]
    C = S // (2 * world)
    for r in range(world):
        starts, lens = [r * C, (2 * world - 1 - r) * C], [C, C]
        got = _gpu_localize(gb, starts, lens)
        ref = oracle.localize_bounds(gb, starts, lens)
        assert np.array_equal(got, ref), f"rank {r}: localised bounds differ from the oracle"
        host = M.cp_rank_share(H=16, S=S, D=128, world=world, rank=r, seed=5).bounds
        assert np.array_equal(got, host), f"rank {r}: differs from the generator's bounds"
        say(f"[localize] rank {r}: {gb.shape[2]} columns bit-exact")


@pytest.mark.parametrize("seed", range(8))
def test_random_bounds_and_chunks(seed):
    """Random int32 bounds (including INT32_MIN / INT32_MAX and values just
    around the chunk edges), batch 2 with 3 mask heads, 1..9 chunks with
    random (also empty) lengths."""
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(1, 5000))
    Sk = int(rng.integers(0, 3000))
    gb = rng.integers(-2 ** 31, 2 ** 31 - 1, size=(2, 3, Sk, 4), dtype=np.int64)
    near = rng.integers(-50, S + 50, size=(2, 3, Sk, 4))
    gb = np.where(rng.random(gb.shape) < 0.7, near, gb)
    if Sk:
        gb[:, :, ::17] = [-2 ** 31, 2 ** 31 - 1, 2 ** 31 - 1, -2 ** 31]
    gb = gb.astype(np.int32)
    n = int(rng.integers(1, 10))
    cuts = np.sort(rng.integers(0, S + 1, size=2 * n))
    starts, lens = cuts[0::2].tolist(), (cuts[1::2] - cuts[0::2]).tolist()
    got = _gpu_localize(gb, starts, lens)
    assert np.array_equal(got, oracle.localize_bounds(gb, starts, lens)), (S, Sk, starts, lens)
    say(f"[localize] seed {seed}: S={S} Sk={Sk} {n} chunks bit-exact")


def test_bad_chunks_rejected():
    import torch
    from column_sparse_masked_amd import _lib
    from column_sparse_masked_amd.api import localize_bounds
    gb = torch.zeros((1, 1, 8, 4), dtype=torch.int32, device="cuda")
    for starts, lens in (([10, 5], [2, 2]), ([0, 3], [5, 1]), ([-1], [3]), ([0], [-2]), ([], [])):
        with pytest.raises((_lib.FmError, ValueError)):
            localize_bounds(gb, starts, lens)
