"""The group boundaries are fenced: a grouped GEMM never reads the offsets of an
earlier grouping.

The pages' hang came from a consumer decoding the expert boundaries (cu_seqlens)
before the producer's writes were visible, and it took about 100,000 launches
to surface (Marin 535B-A23B article, section "21% to 27% MFU without stopping the
run"; Marin weekly summary of September 14, hero-run section).  Here moe_permute
writes the offsets and moe_grouped_ffn reads them on the same stream.  This test
runs that pair 10,000 times (about 100,000 kernel launches), with each call's
expert sizes drawn afresh (from near-uniform to a single expert, with empty
experts), and before every call it clears the offsets and the GEMM's tile prefix
to zero.  A consumer reading the cleared values would see empty groups and leave
its output rows as the NaN poison written before the call.  The poison is zeros,
so a stale read cannot go out of bounds; it can only show up as a mismatch.

Every call's offsets are checked against the oracle's grouping of that call's
ids, and every output row against the same token through the same expert
computed once up front.  A row's output depends only on its input row and its
expert's weights, with a fixed reduction order, so the two must be bit-equal.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def M():
    import mixture_experts_transformer_amd as m
    return m


def test_boundaries_fenced_over_10000_changing_groupings(M):
    n_iter, T, k, E, d, H = 10_000, 96, 2, 16, 64, 64
    n = T * k
    rng = np.random.default_rng(2024)
    g = torch.Generator(device=DEV).manual_seed(5)
    x = (torch.randn((T, d), generator=g, device=DEV)).to(torch.bfloat16)
    W_gu = (torch.randn((E, 2 * H, d), generator=g, device=DEV) / 8).to(torch.bfloat16)
    W_d = (torch.randn((E, d, H), generator=g, device=DEV) / 8).to(torch.bfloat16)

    # every (token, expert) output, from one grouping that sends each token to
    # every expert (expert-major rows)
    full_ids = torch.arange(E, dtype=torch.int32, device=DEV).repeat(T, 1)
    X_all = torch.empty((T * E, d), dtype=torch.bfloat16, device=DEV)
    ga = M.moe_permute(full_ids, E, src=x, src_div=E, dst=X_all)
    F = M.moe_grouped_ffn(X_all, ga["offsets"], W_gu, W_d)
    torch.cuda.synchronize()
    assert np.array_equal(ga["offsets"].cpu().numpy(), np.arange(E + 1) * T)
    F = F.view(E, T, d)                         # F[e, t] = expert e on token t

    # each call's ids: a fresh Dirichlet spread over the experts (concentration
    # from 0.02, nearly one expert, to 50, nearly uniform), k distinct per token
    ids_all = np.empty((n_iter, n), np.int32)
    exp_off = np.empty((n_iter, E + 1), np.int32)
    exp_tok = np.empty((n_iter, n), np.int64)
    exp_e = np.empty((n_iter, n), np.int64)
    for i in range(n_iter):
        p = rng.dirichlet(np.full(E, 10.0 ** rng.uniform(-1.7, 1.7)))
        p = np.maximum(p, 1e-12)
        keys = np.log(rng.random((T, E))) / p         # k distinct experts weighted by p
        ids = np.argsort(-keys, axis=1)[:, :k].astype(np.int32).ravel()
        ids_all[i] = ids
        ref = O.permute(ids, E)
        exp_off[i] = ref["offsets"]
        src = ref["row_src"]
        exp_tok[i] = src // k
        exp_e[i] = ids[src]
    ids_dev = torch.from_numpy(ids_all).to(DEV)
    exp_tok_d = torch.from_numpy(exp_tok).to(DEV)
    exp_e_d = torch.from_numpy(exp_e).to(DEV)

    out = dict(slot_row=torch.empty(n, dtype=torch.int32, device=DEV),
               row_src=torch.empty(n, dtype=torch.int32, device=DEV),
               counts=torch.empty(E, dtype=torch.int32, device=DEV),
               offsets=torch.empty(E + 1, dtype=torch.int32, device=DEV),
               n_dropped=torch.empty(1, dtype=torch.int64, device=DEV))
    ws_p = torch.empty(M.moe_permute_workspace_size(n, E), dtype=torch.uint8, device=DEV)
    ws_g = torch.empty(M.moe_grouped_ffn_workspace_size(E, n, H, torch.bfloat16),
                       dtype=torch.uint8, device=DEV)
    tile_prefix = ws_g[:(E + 1) * 4].view(torch.int32)
    X_perm = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    Y = torch.empty((n, d), dtype=torch.bfloat16, device=DEV)
    off_log = torch.empty((n_iter, E + 1), dtype=torch.int32, device=DEV)
    bad_rows = torch.empty(n_iter, dtype=torch.int32, device=DEV)
    for i in range(n_iter):
        out["offsets"].zero_()
        tile_prefix.zero_()
        Y.fill_(float("nan"))
        M.moe_permute(ids_dev[i], E, src=x, src_div=k, dst=X_perm, ws=ws_p, out=out)
        M.moe_grouped_ffn(X_perm, out["offsets"], W_gu, W_d, Y=Y, ws=ws_g)
        off_log[i].copy_(out["offsets"])
        want = F[exp_e_d[i], exp_tok_d[i]]
        bad_rows[i] = (Y.view(torch.int16) != want.view(torch.int16)).any(dim=1).sum()
        if (i + 1) % 2000 == 0:
            torch.cuda.synchronize()
            print(f"{i + 1} groupings run", flush=True)
    torch.cuda.synchronize()
    offs = off_log.cpu().numpy()
    bad = bad_rows.cpu().numpy()
    wrong_off = np.flatnonzero(np.any(offs != exp_off, axis=1))
    assert wrong_off.size == 0, f"offsets differ first at call {wrong_off[0]}"
    wrong = np.flatnonzero(bad)
    assert wrong.size == 0, f"call {wrong[0]}: {bad[wrong[0]]} output rows differ"
    sizes = np.diff(exp_off, axis=1)
    print(f"{n_iter} calls; largest group {sizes.max()} of {n} rows, "
          f"{int((sizes == 0).sum())} empty groups in all")
