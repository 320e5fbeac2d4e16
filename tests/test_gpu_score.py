"""GPU parity of kvs_score against the fp64 oracle (element by element).

Tolerance: |gpu - oracle| <= 2e-3 |oracle| + 2e-3 * 1e-3 * R / L (fp32
accumulation of bf16 products and exp2 vs fp64); total mass within 1e-4 R.
Sizes span several 32-key tiles, several key splits and a ragged tail; the
full-size cases run the shapes of the Llama-3.1-8B (32K) and Mistral-7B (128K)
layers in the launch configuration the bench times.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_mass, assert_scores_close

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _run(kvs, ly, heads, q_pos0=None, **kw):
    q_pos0 = ly.q_pos0 if q_pos0 is None else q_pos0
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    a = kvs.score_args(L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv, q_pos0=q_pos0,
                       heads=heads, **kw)
    S = kvs.kvs_score(Q, K, a)
    torch.cuda.synchronize()
    return S.cpu().numpy()


CASES = [
    # (name, L, W, d_k, H_q, H_kv, q_pos0 offset from L - W)
    ("tiny", 512, 16, 64, 4, 1, 0),
    ("ragged", 1000, 7, 128, 8, 2, 0),
    ("ragged64", 777, 13, 64, 6, 3, 0),
    ("gqa_w32", 4113, 32, 128, 32, 8, 0),
    ("decode_w1", 2000, 1, 128, 32, 8, 0),
    ("claa_w8", 3000, 8, 128, 32, 8, 0),
    ("lookahead", 1500, 32, 128, 8, 2, 40),     # queries after the prompt: all keys visible
    ("mha", 640, 32, 64, 4, 4, 0),
    ("w64", 900, 64, 64, 4, 2, 0),
    ("one_key", 1, 1, 64, 2, 1, 0),
    ("short", 20, 20, 128, 4, 1, 0),            # window is the whole prompt
    ("g3_w32", 2500, 32, 128, 6, 2, 0),         # 96 padded rows: three row tiles
    ("g6_w16_64", 1200, 16, 64, 12, 2, 0),      # 96 padded rows at d_k = 64
    # more than 128 padded rows per KV head: two row groups
    ("r160_g8_w20", 3001, 20, 128, 64, 8, 0),   # R = 160 (heads padded to 32 rows)
    ("r160_g4_w40", 2100, 40, 128, 16, 4, 0),   # R = 160 (heads padded to 64 rows)
    ("r192_g8_w24", 1500, 24, 64, 16, 2, 0),    # R = 192
    ("r192_g6_w32", 2500, 32, 128, 12, 2, 0),   # R = 192: groups of 4 heads and 2 heads
    ("r192_g2_w96", 1000, 96, 128, 4, 2, 0),    # one head per group (96 rows each)
    ("r256_g8_w32", 4113, 32, 128, 64, 8, 0),   # R = 256: Llama shape with G = 8
    ("r256_g4_w64", 2000, 64, 64, 8, 2, 0),     # R = 256
    ("r200_g1_w200", 1200, 200, 128, 2, 2, 0),  # one head of 200 rows, split at row 128
]


@pytest.mark.parametrize("name,L,W,d_k,H_q,H_kv,off", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("heads", [1, 0, 2], ids=["group_sum", "none", "group_max"])
def test_score_parity(kvs, name, L, W, d_k, H_q, H_kv, off, heads):
    print(f"case {name} heads={heads}", flush=True)
    ly = synth.gaussian_layer(100 + L, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    q_pos0 = L - W + off
    got = _run(kvs, ly, heads, q_pos0=q_pos0)
    want = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0, heads=heads)
    G = H_q // H_kv
    R = W * G if heads == 1 else W
    assert_scores_close(got, want, R, L, name)
    if heads != 2:
        assert_mass(got, R)


def test_accumulate_and_strides(kvs):
    """accumulate=1 adds into S; sequence-major K via strides; padded S rows."""
    L, W, d_k, H_q, H_kv = 1100, 16, 128, 16, 4
    ly = synth.gaussian_layer(7, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    want = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0)
    Q = kvs.bf16_from_bits(ly.Q)
    Kseq = kvs.bf16_from_bits(np.ascontiguousarray(ly.K.transpose(1, 0, 2)))  # [L][H_kv][d]
    s_ld = 1152
    S = torch.full((H_kv, s_ld), 0.5, dtype=torch.float32, device="cuda")
    a = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, accumulate=True,
                       k_head_stride=d_k, k_tok_stride=H_kv * d_k, s_ld=s_ld)
    kvs.kvs_score(Q, Kseq, a, S=S)
    torch.cuda.synchronize()
    got = S.cpu().numpy()
    assert_scores_close(got[:, :L] - 0.5, want, W * H_q // H_kv, L, "accumulate")
    assert np.all(got[:, L:] == 0.5), "wrote past L"


def test_deterministic(kvs):
    ly = synth.gaussian_layer(3, L=5000, W=32, d_k=128, H_q=32, H_kv=8)
    a = _run(kvs, ly, 1)
    b = _run(kvs, ly, 1)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_identical_keys_closed_form(kvs):
    """All keys equal: prefix columns equal G * sum_j 1/(q_pos0 + j + 1)."""
    L, W, G = 3000, 32, 4
    ly = synth.gaussian_layer(9, L=L, W=W, d_k=128, H_q=G, H_kv=1)
    ly.K = np.repeat(ly.K[:, :1, :], L, axis=1)
    got = _run(kvs, ly, 1)[0]
    q_pos0 = L - W
    inv = np.array([1.0 / (q_pos0 + j + 1) for j in range(W)])
    np.testing.assert_allclose(got[:q_pos0], G * inv.sum(), rtol=2e-3)
    for i in range(W):
        np.testing.assert_allclose(got[q_pos0 + i], G * inv[i:].sum(), rtol=2e-3)


@pytest.mark.slow
@pytest.mark.parametrize("which", ["llama32k", "mistral128k"])
def test_full_size_parity(kvs, which):
    """Full layer shapes (Llama-3.1-8B at 32K, Mistral-7B at 128K), all heads, every column
    (the oracle takes a few seconds)."""
    print(f"full-size {which}", flush=True)
    ly = synth.llama_layer() if which == "llama32k" else synth.mistral_layer()
    got = _run(kvs, ly, 1)
    want = oracle.score(ly.Q, ly.K, L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                        q_pos0=ly.q_pos0)
    R = ly.W * ly.G
    assert_scores_close(got, want, R, ly.L, which)
    assert_mass(got, R)


@pytest.mark.parametrize("heads", [1, 0, 2], ids=["group_sum", "none", "group_max"])
def test_two_row_groups_accumulate_and_phases(kvs, heads):
    """R = 256 (G = 8, W = 32): accumulate = 1 adds the score once, and the phase-1 /
    phase-2 calls equal one call bit for bit."""
    L, W, d_k, H_q, H_kv = 3000, 32, 128, 32, 4
    ly = synth.gaussian_layer(41, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    shape = dict(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, heads=heads)
    rows = H_q if heads == 0 else H_kv
    one = kvs.kvs_score(Q, K, kvs.score_args(**shape))
    ws = torch.empty(kvs.kvs_score_workspace(kvs.score_args(**shape)), dtype=torch.uint8,
                     device="cuda")
    S = torch.full((rows, L), float("nan"), dtype=torch.float32, device="cuda")
    kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=1), S=S, ws=ws)
    kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=2), S=S, ws=ws)
    acc = torch.full((rows, L), 0.25, dtype=torch.float32, device="cuda")
    kvs.kvs_score(Q, K, kvs.score_args(**shape, accumulate=True), S=acc)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int32), S.view(torch.int32))
    want = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0,
                        heads=heads)
    R = W * (H_q // H_kv) if heads == 1 else W
    assert_scores_close(acc.cpu().numpy() - 0.25, want, R, L, "accumulate")


@pytest.mark.parametrize("which", ["ragged", pytest.param("mistral128k", marks=pytest.mark.slow)])
def test_phase_split_matches_one_call(kvs, which):
    """phase 1 (row statistics into ws) then phase 2 (column sums from that ws), as the bench
    times the 128K layer, equals a single phase-0 call bit for bit."""
    print(f"phase split {which}", flush=True)
    if which == "ragged":
        ly = synth.gaussian_layer(4113, L=4113, W=32, d_k=128, H_q=32, H_kv=8)
    else:
        ly = synth.mistral_layer()
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    shape = dict(L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv, q_pos0=ly.q_pos0)
    one = kvs.kvs_score(Q, K, kvs.score_args(**shape))
    ws = torch.empty(kvs.kvs_score_workspace(kvs.score_args(**shape)), dtype=torch.uint8,
                     device="cuda")
    S = torch.full_like(one, float("nan"))
    kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=1), S=S, ws=ws)
    kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=2), S=S, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(one.view(torch.int32), S.view(torch.int32))


@pytest.mark.parametrize("heads", [1, 0, 2, 3], ids=["group_sum", "none", "group_max", "all_sum"])
@pytest.mark.parametrize("name,L,W,d_k,H_q,H_kv", [
    ("gqa_w32", 4113, 32, 128, 32, 8),     # 26 splits x 8 KV heads in one launch
    ("tiny", 512, 16, 64, 4, 1),
    ("g3_w32", 2500, 32, 128, 6, 2),
], ids=["gqa_w32", "tiny", "g3_w32"])
def test_one_launch_late_split_path(kvs, name, L, W, d_k, H_q, H_kv, heads):
    """With the wait bound at 0, every workgroup of the one-launch form that finds its KV head
    incomplete computes the missing splits' statistics itself.  The scores must equal the
    two-phase calls bit for bit and the oracle within tolerance; the flags and statistics
    left in the workspace (garbage on entry, then an earlier call's) change nothing."""
    print(f"late-split path {name} heads={heads}", flush=True)
    ly = synth.gaussian_layer(L + 17 * H_kv, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    shape = dict(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0, heads=heads)
    ws = torch.empty(kvs.kvs_score_workspace(kvs.score_args(**shape)), dtype=torch.uint8,
                     device="cuda")
    two = kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=1), ws=ws)
    two = kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=2), S=two, ws=ws)
    ws.fill_(0xA5)
    prev = kvs.kvs_wait_limit(0)
    try:
        late = [kvs.kvs_score(Q, K, kvs.score_args(**shape), ws=ws) for _ in range(2)]
    finally:
        assert kvs.kvs_wait_limit(prev) == 0
    ws.fill_(0xFF)
    fast = kvs.kvs_score(Q, K, kvs.score_args(**shape), ws=ws)
    torch.cuda.synchronize()
    for got in late + [fast]:
        assert torch.equal(two.view(torch.int32), got.view(torch.int32))
    So = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0,
                      heads=heads)
    R = W * (H_q // H_kv) if heads == 1 else W * H_q if heads == 3 else W
    assert_scores_close(fast.cpu().numpy(), So, R, L, "one launch")


ALL_SUM_CASES = [
    # (name, L, W, d_k, H_q, H_kv): the CLAA layer score, summed over every head
    ("claa_w8", 3000, 8, 128, 32, 8),
    ("tiny", 512, 16, 64, 4, 1),
    ("ragged64", 777, 13, 64, 6, 3),
    ("two_groups", 2100, 32, 128, 64, 8),
]


@pytest.mark.parametrize("name,L,W,d_k,H_q,H_kv", ALL_SUM_CASES, ids=[c[0] for c in ALL_SUM_CASES])
def test_all_heads_sum(kvs, name, L, W, d_k, H_q, H_kv):
    """ALL_SUM: one row per layer summed over every query head, written into a row of a
    longer buffer (s_ld > L) and accumulated on a second call."""
    print(f"all-heads sum {name}", flush=True)
    ly = synth.gaussian_layer(300 + L, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    s_ld = L + 64
    ring = torch.full((3, s_ld), -5.0, dtype=torch.float32, device="cuda")
    a = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0,
                       heads=kvs.HEADS_ALL_SUM, s_ld=s_ld)
    kvs.kvs_score(Q, K, a, S=ring[1:2])
    b = kvs.score_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0,
                       heads=kvs.HEADS_ALL_SUM, s_ld=s_ld, accumulate=True)
    kvs.kvs_score(Q, K, b, S=ring[2:3])
    torch.cuda.synchronize()
    got = ring.cpu().numpy()
    want = oracle.score(ly.Q, ly.K, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=ly.q_pos0,
                        heads=oracle.HEADS_ALL_SUM)
    R = W * H_q
    assert_scores_close(got[1:2, :L], want, R, L, name)
    assert_mass(got[1:2, :L], R)
    assert_scores_close(got[2:3, :L] + 5.0, want, R, L, name + " accumulate")
    assert (got[0] == -5.0).all() and (got[1:, L:] == -5.0).all(), "wrote outside the slot"
