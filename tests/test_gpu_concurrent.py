"""One-launch forms under concurrency (GPU).

kvs_score, kvs_delta_pages and wide-row kvs_topk run their workgroup exchanges inside one
launch when the device holds the whole grid at once.  Calls enqueued on several streams at
the same time overlap on the device, so no call's grid is guaranteed to be resident: a
workgroup that waits in vain computes what is missing itself after the wait bound.  Every
call here runs on its own stream with its own workspace, all enqueued before any is waited
for, and must give exactly the bits the same call gives alone.
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _score_call(kvs, seed):
    ly = synth.gaussian_layer(seed, L=8200, W=32, d_k=128, H_q=32, H_kv=8)
    Q, K = kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K)
    a = kvs.score_args(L=ly.L, W=ly.W, d_k=128, H_q=32, H_kv=8, q_pos0=ly.q_pos0)
    ws = torch.empty(kvs.kvs_score_workspace(a), dtype=torch.uint8, device="cuda")
    S = torch.empty(8, ly.L, dtype=torch.float32, device="cuda")
    return lambda stream: kvs.kvs_score(Q, K, a, S=S, ws=ws, stream=stream), S


def _delta_call(kvs, seed):
    lens = [4096, 3000, 4096, 1234]
    Ks, Qs = [], []
    for b, L in enumerate(lens):
        ly = synth.gaussian_layer(seed + b, L=L, W=1, d_k=128, H_q=32, H_kv=8, q_pos0=L - 1)
        Ks.append(kvs.bf16_from_bits(ly.K))
        Qs.append(ly.Q[:, 0, :])
    Q = kvs.bf16_from_bits(np.stack(Qs))
    ptrs = torch.tensor([k.data_ptr() for k in Ks], dtype=torch.int64, device="cuda")
    Lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    a = kvs.delta_args(B=len(lens), d_k=128, H_q=32, H_kv=8, L_max=max(lens), P=16, K_pages=32,
                       L_recent=4)
    S = torch.empty(len(lens), (max(lens) + 15) // 16, dtype=torch.float32, device="cuda")
    rho = torch.empty(len(lens), 32, dtype=torch.int32, device="cuda")
    ws = torch.empty(kvs.kvs_delta_workspace(a), dtype=torch.uint8, device="cuda")
    return (lambda stream: kvs.kvs_delta_pages(Q, ptrs, Lt, a, page_scores=S, rho=rho, ws=ws,
                                               stream=stream), (S, rho, Ks))


def _topk_call(kvs, seed):
    x = torch.from_numpy(synth.score_array(seed, 4, 60000, levels=5)).cuda()
    idx = torch.empty(4, 15000, dtype=torch.int32, device="cuda")
    ws = torch.empty(kvs.library().kvs_topk_workspace(4, 60000, 15000), dtype=torch.uint8,
                     device="cuda")
    return lambda stream: kvs.kvs_topk(x, 60000, 15000, idx=idx, ws=ws, stream=stream), idx


def test_one_launch_forms_on_concurrent_streams(kvs):
    calls = [_score_call(kvs, 11), _score_call(kvs, 12), _delta_call(kvs, 40), _topk_call(kvs, 70)]
    # alone, one after the other
    alone = []
    for run, out in calls:
        run(torch.cuda.current_stream())
        torch.cuda.synchronize()
        alone.append(_snapshot(out))
    # all four enqueued at once on streams of their own, three rounds
    streams = [torch.cuda.Stream() for _ in calls]
    for _ in range(3):
        for (run, out), st in zip(calls, streams):
            run(st)
        torch.cuda.synchronize()
        for (run, out), want in zip(calls, alone):
            for g, w in zip(_snapshot(out), want):
                assert np.array_equal(g.view(np.uint32) if g.dtype == np.float32 else g,
                                      w.view(np.uint32) if w.dtype == np.float32 else w)


def _snapshot(out):
    if isinstance(out, tuple):
        return [out[0].cpu().numpy(), out[1].cpu().numpy()]
    return [out.cpu().numpy()]
