"""The hot path captured into a HIP graph: every replay must equal the eager run.

Replays are interleaved with eager work and host synchronisations, and every
replay is checked (not only the first)."""

import pytest
import torch

import oracle
from scale_wise_attention_amd.inputs import WORKLOADS, make_qkv, pruned_index

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    assert torch.cuda.is_available()
    from scale_wise_attention_amd import api
    wl = WORKLOADS["var512"]
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(wl, 0, device=dev)
    off = oracle.offsets(wl.h, wl.w)
    K = wl.num_scales
    s = K - 1
    qs = q[:, :, off[s]:]
    sel = torch.from_numpy(pruned_index(1024, 0.4, 0)).to(dev)
    mp = api.mask_params(64, 64, 3, 3, 2, 2)
    n_qt, n_kt = api.var_tile_mask_dims((wl.h, wl.w), s, s + 1, mp, sel.numel())
    rp = torch.empty(n_qt + 1, dtype=torch.int32, device=dev)
    ci = torch.empty(n_qt * n_kt, dtype=torch.int32, device=dev)
    dense = torch.empty(2, 30, 1024, 64, dtype=torch.bfloat16, device=dev)
    prev = torch.empty(2, 30, 576, 64, dtype=torch.bfloat16, device=dev)
    upd = torch.empty(2, 30, sel.numel(), 64, dtype=torch.bfloat16, device=dev)
    out = torch.empty(2, 30, 1024, 64, dtype=torch.bfloat16, device=dev)
    out1 = torch.empty(2, 30, 1024, 64, dtype=torch.bfloat16, device=dev)   # one-launch reconstruction

    def run():
        api.var_attn_dense((wl.h, wl.w), qs, k, v, s, s + 1, out=dense)
        api.var_attn_dense((wl.h, wl.w), q[:, :, off[s - 1]:off[s]], k, v, s - 1, s, out=prev)
        api.var_build_tile_mask((wl.h, wl.w), s, s + 1, mp, q_index=sel, row_ptr=rp, col_idx=ci)
        api.var_attn_block_sparse((wl.h, wl.w), qs, k, v, s, s + 1, rp, ci, out=upd, q_index=sel)
        api.var_scatter_restore(prev, 24, 24, upd, sel, 32, 32, out=out)
        api.var_attn_block_sparse_restore((wl.h, wl.w), qs, k, v, s, rp, ci, sel, prev, 24, 24, out=out1)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (dense, rp, ci[: int(rp[-1].item())], upd, out, out1)]
    assert torch.equal(out, out1), "one-launch reconstruction against attention + scatter"

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(4):
        for t in (dense, rp, ci, upd, out, out1):
            t.fill_(0) if t.dtype != torch.int32 else t.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (dense, rp, ci[: int(rp[-1].item())], upd, out, out1)
        for a, b in zip(eager, got):
            assert torch.equal(a, b), f"replay {rep}"
        # eager work between replays
        _ = (q[:, :, :100].float() * 2).sum().item()


def test_graph_replays_match_eager_e4m3():
    """Key quantisation (a growing cache: only the step's new tiles) and the e4m3 dense and sparse calls."""
    assert torch.cuda.is_available()
    from scale_wise_attention_amd import api
    from scale_wise_attention_amd.inputs import custom_workload
    wl = custom_workload((1, 2, 4, 6, 8, 12, 16, 20), 2, 2, 128, sink_offset_scales=3)
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(wl, 1, device=dev)
    off = oracle.offsets(wl.h, wl.w)
    s = wl.num_scales - 1
    qs = q[:, :, off[s]:off[s + 1]]
    k8 = torch.zeros(k.shape, dtype=torch.uint8, device=dev)
    sk = torch.zeros((2, 2, -(-k.shape[2] // 64)), dtype=torch.float32, device=dev)
    api.var_quantize_e4m3(k[:, :, :off[s]], codes=k8[:, :, :off[s]], scale=sk)   # the cache before the step
    mp = api.mask_params(64, 64, 2, 3, 1, 1)
    rp, ci = api.var_build_tile_mask((wl.h, wl.w), s, s + 1, mp)
    n = off[s + 1] - off[s]
    dense = torch.empty(2, 2, n, 128, dtype=torch.bfloat16, device=dev)
    sparse = torch.empty(2, 2, n, 128, dtype=torch.float32, device=dev)

    def run():
        api.var_quantize_e4m3(k[:, :, :off[s + 1]], codes=k8[:, :, :off[s + 1]], scale=sk, first_token=off[s])
        api.var_attn_dense_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, out=dense)
        api.var_attn_block_sparse_e4m3((wl.h, wl.w), qs, k8, sk, v, s, s + 1, rp, ci, out=sparse)

    run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in (k8, sk, dense, sparse)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    t0 = off[s] // 64 * 64
    for rep in range(4):
        k8[:, :, t0:].fill_(0)
        sk[:, :, t0 // 64:].fill_(0)
        dense.fill_(0)
        sparse.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eager, (k8, sk, dense, sparse)):
            assert torch.equal(a, b), f"replay {rep}"
        _ = (q[:, :, :100].float() * 2).sum().item()
