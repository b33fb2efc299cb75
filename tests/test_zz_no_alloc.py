"""moe_permute_noalloc, the allocation-free variant of moe_permute, against
moe_permute itself: every grouping output and the row copy bit-equal, on two calls
in a row (the second with a smaller input, so stale scratch from the first call
would show), and sizes beyond its scratch rejected before anything is enqueued.
Called through the C ABI (the binding only marshals arguments)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    import mixture_experts_transformer_amd as m
    return m


def _outputs(n, R, E):
    i32 = dict(dtype=torch.int32, device=DEV)
    return dict(slot_row=torch.full((n,), -7, **i32), row_src=torch.full((max(R, 1),), -7, **i32),
                counts=torch.full((E,), -7, **i32), offsets=torch.full((E + 1,), -7, **i32),
                n_dropped=torch.full((1,), -7, dtype=torch.int64, device=DEV))


def _ids(n, E, seed, pad=0.0, skew=1.0):
    rng = np.random.default_rng(seed)
    p = 1.0 / np.arange(1, E + 1) ** skew
    ids = rng.choice(E, size=n, p=p / p.sum()).astype(np.int32)
    if pad:
        ids[rng.random(n) < pad] = -1
    return torch.from_numpy(ids).to(DEV)


def _compare(M, ids, E, capacity, src, src_div, R):
    n = ids.numel()
    width = src.shape[1]
    dst_ref = torch.zeros((R, width), dtype=src.dtype, device=DEV)
    ref = M.moe_permute(ids, E, capacity=capacity, src=src, src_div=src_div, dst=dst_ref,
                        R_phys=R)
    out = _outputs(n, R, E)
    dst = torch.zeros((R, width), dtype=src.dtype, device=DEV)
    M.moe_permute_noalloc(ids, E, out, capacity=capacity, src=src, src_div=src_div, dst=dst,
                          R_phys=R)
    torch.cuda.synchronize()
    for key in ["slot_row", "counts", "offsets", "n_dropped"]:
        assert torch.equal(out[key][:ref[key].numel()], ref[key]), key
    assert torch.equal(out["row_src"][:R], ref["row_src"]), "row_src"
    kept = int(ref["offsets"][E])
    assert torch.equal(dst[:kept], dst_ref[:kept]), "copied rows"
    return ref


def test_noalloc_permute_equals_permute_on_two_calls(M):
    # 1. the 535B layer's grouping: 8,192 tokens x top-8 of 384 experts, rows copied
    #    (a scatter of shared token rows), capacity 1.10 x the mean
    E, T, k, w = 384, 8192, 8, 3072
    g = torch.Generator(device=DEV).manual_seed(1)
    x = torch.randn((T, w), generator=g, device=DEV).to(torch.bfloat16)
    cap = (110 * T * k + 100 * E - 1) // (100 * E)
    ref = _compare(M, _ids(T * k, E, 1, skew=0.7), E, cap, x, k, T * k)
    assert int(ref["n_dropped"][0]) > 0
    # 2. smaller and of another kind: a padded pool of 9,000 rows over 6 experts,
    #    float32 rows gathered one per assignment, dropless
    P, E2 = 9000, 6
    xp = torch.randn((P, 256), generator=g, device=DEV)
    _compare(M, _ids(P, E2, 2, pad=0.1), E2, -1, xp, 1, P)


def test_noalloc_permute_rejects_sizes_beyond_its_scratch(M):
    E = 1024
    n = 1 << 21          # 8 MiB of ranks + 16 MiB of segment counts: over the 16 MiB
    assert M.moe_permute_workspace_size(n, E) > M.MOE_PERMUTE_NOALLOC_SCRATCH_BYTES
    ids = torch.zeros(n, dtype=torch.int32, device=DEV)
    out = _outputs(n, n, E)
    with pytest.raises(M.MoeError) as err:
        M.moe_permute_noalloc(ids, E, out)
    assert err.value.status == M.MOE_EWORKSPACE
    torch.cuda.synchronize()
    assert int(out["counts"][0]) == -7, "nothing may be written"
