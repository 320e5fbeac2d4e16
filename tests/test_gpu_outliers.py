"""GPU parity against the fp64 oracle with outlier logits (attention-sink-like keys).

The score statistics pass sums exp2 against a running maximum taken from each
wave's first key tile.  A later logit far above that maximum either leaves the
sums dominated by huge but representable terms (86 log2 units above it:
terms near 2^86), or pushes a sum past 2^100 or out of the float range, and
then the wave redoes its tiles with the exact online update (202 and 606
log2 units).  Seeded N(0,1)
inputs reach neither; these cases plant keys whose logit exceeds every
ordinary logit of some rows by about 60, 140 and 420 (about 86, 202 and 606
in log2 units), in later tiles of several waves
and key splits, in a wave's first tile, inside the causal window and in the
ragged last tile.  Every head mode, the split statistics/column-sum calls, the
DELTA decode page scores and the raw-logit scores are checked against the
oracle with the usual bars.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_mass, assert_scores_close, assert_topk_parity

pytestmark = pytest.mark.gpu

LIFTS = (60.0, 140.0, 420.0)   # logit units above the row's ordinary logits


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


def _tiles_per_split(L, H_kv):
    """Key tiles (32 keys) per split in the score launch: one 4-wave workgroup per
    CU (256 in all, shared by the KV heads), at least one tile per wave."""
    n_tiles = (L + 31) // 32
    per_head = (256 + H_kv - 1) // H_kv
    ns = max(1, min(per_head, max(n_tiles // 4, 1)))
    return (n_tiles + ns - 1) // ns


def _later_tile(t, L, H_kv):
    """True when key t sits in a tile that is not its wave's first tile."""
    tps = _tiles_per_split(L, H_kv)
    tile = t // 32
    return tile - (tile // tps) * tps >= 4


def _outlier_layer(seed, L, W, d_k, H_q, H_kv, positions):
    """positions: per KV head, a list of keys; head slot i of the group takes
    lift LIFTS[i % 3] for its keys (slot = position index mod min(G, 3))."""
    G = H_q // H_kv
    ly = synth.gaussian_layer(seed, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    out = []
    for g, ts in enumerate(positions):
        for i, t in enumerate(ts):
            hs = i % min(G, 3)
            out.append((g, hs, t, LIFTS[hs]))
    return synth.plant_outliers(ly, seed + 77, out)


def _score(kvs, ly, heads, phase_split=False):
    Q = kvs.bf16_from_bits(ly.Q)
    K = kvs.bf16_from_bits(ly.K)
    shape = dict(L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv, q_pos0=ly.q_pos0,
                 heads=heads)
    if not phase_split:
        S = kvs.kvs_score(Q, K, kvs.score_args(**shape))
    else:
        ws = torch.empty(kvs.kvs_score_workspace(kvs.score_args(**shape)), dtype=torch.uint8,
                         device="cuda")
        rows = ly.H_q if heads == 0 else ly.H_kv
        S = torch.full((rows, ly.L), float("nan"), dtype=torch.float32, device="cuda")
        kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=1), S=S, ws=ws)
        kvs.kvs_score(Q, K, kvs.score_args(**shape, phase=2), S=S, ws=ws)
    torch.cuda.synchronize()
    return S.cpu().numpy()


def _check(got, ly, heads, what):
    want = oracle.score(ly.Q, ly.K, L=ly.L, W=ly.W, d_k=ly.d_k, H_q=ly.H_q, H_kv=ly.H_kv,
                        q_pos0=ly.q_pos0, heads=heads)
    R = ly.W * ly.G if heads == 1 else ly.W
    assert np.isfinite(got).all(), f"{what}: non-finite scores"
    assert_scores_close(got, want, R, ly.L, what)
    if heads != 2:
        assert_mass(got, R)


def _spread(L, H_kv, count, seed, first_tile=True):
    """Per KV head: `count` keys in later tiles of their waves (different waves and
    splits for different heads), plus one in a wave's first tile and one in the
    ragged last tile."""
    tps = _tiles_per_split(L, H_kv)
    rng = np.random.default_rng(seed)
    out = []
    for g in range(H_kv):
        ts = []
        while len(ts) < count:
            t = int(rng.integers(0, L - 64))
            if _later_tile(t, L, H_kv):
                ts.append(t)
        if first_tile:
            split = int(rng.integers(0, max(1, (L // 32) // tps)))
            ts.append(split * tps * 32 + 32 * (g % 4) + 5)     # first tile of wave g % 4
        ts.append(L - 1 - (g % 3))                           # causal window / ragged tail
        out.append(ts)
    return out


CASES = [
    # name, L, W, d_k, H_q, H_kv, later-tile outliers per KV head
    ("tiny", 512, 16, 64, 4, 1, 0),            # one tile per wave: first-tile outliers only
    ("ragged4k", 4113, 32, 128, 32, 8, 3),
    ("l16k", 16384, 32, 128, 32, 8, 4),
    ("g3_ragged", 2500, 32, 128, 6, 2, 3),
]


@pytest.mark.parametrize("name,L,W,d_k,H_q,H_kv,count", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("heads", [1, 0, 2], ids=["group_sum", "none", "group_max"])
def test_score_outliers(kvs, name, L, W, d_k, H_q, H_kv, count, heads):
    print(f"outlier case {name} heads={heads}", flush=True)
    if name == "tiny":
        pos = [[100, 300, 450, 500, 511]]   # 500 and 511 sit inside the causal window
    else:
        pos = _spread(L, H_kv, count, seed=L)
        assert any(_later_tile(t, L, H_kv) for ts in pos for t in ts), "case misses the redo path"
    ly = _outlier_layer(200 + L, L, W, d_k, H_q, H_kv, pos)
    _check(_score(kvs, ly, heads), ly, heads, name)


def test_score_outliers_phase_split(kvs):
    L, H_kv = 4113, 8
    ly = _outlier_layer(31, L, 32, 128, 32, H_kv, _spread(L, H_kv, 3, seed=5))
    one = _score(kvs, ly, 1)
    two = _score(kvs, ly, 1, phase_split=True)
    assert np.array_equal(one.view(np.uint32), two.view(np.uint32))
    _check(two, ly, 1, "phase split")


@pytest.mark.slow
@pytest.mark.parametrize("heads", [1, 0, 2], ids=["group_sum", "none", "group_max"])
def test_score_outliers_full_size(kvs, heads):
    """The Mistral-7B layer at 128K (planted spans) with outlier keys added."""
    print(f"outliers at 128K heads={heads}", flush=True)
    base = synth.mistral_layer()
    pos = _spread(base.L, base.H_kv, 6, seed=11)
    out = []
    for g, ts in enumerate(pos):
        for i, t in enumerate(ts):
            out.append((g, i % 3, t, LIFTS[i % 3]))
    ly = synth.plant_outliers(base, 123, out)
    _check(_score(kvs, ly, heads), ly, heads, "mistral128k outliers")


def test_delta_outliers(kvs):
    """DELTA decode page scores and sets with outlier keys in some sequences."""
    lens, H_q, H_kv, d_k, P, K_pages, L_recent = [3000, 1500, 777], 32, 8, 128, 16, 16, 4
    layers, Ks = [], []
    for b, L in enumerate(lens):
        ly = synth.gaussian_layer(400 + b, L=L, W=1, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L - 1)
        rng = np.random.default_rng(b)
        out = [(g, i % 3, int(rng.integers(0, L)), LIFTS[i % 3]) for g in range(H_kv)
               for i in range(3)]
        ly = synth.plant_outliers(ly, 500 + b, out)
        layers.append(ly)
        Ks.append(kvs.bf16_from_bits(ly.K))
    Q = kvs.bf16_from_bits(np.stack([ly.Q[:, 0, :] for ly in layers]))
    ptrs = torch.tensor([k.data_ptr() for k in Ks], dtype=torch.int64, device="cuda")
    a = kvs.delta_args(B=len(lens), d_k=d_k, H_q=H_q, H_kv=H_kv, L_max=max(lens), P=P,
                       K_pages=K_pages, L_recent=L_recent)
    n_pages_max = (max(lens) + P - 1) // P
    S = torch.full((len(lens), n_pages_max), -7.0, dtype=torch.float32, device="cuda")
    rho = kvs.kvs_delta_pages(Q, ptrs, torch.tensor(lens, dtype=torch.int32, device="cuda"), a,
                              page_scores=S).cpu().numpy()
    S = S.cpu().numpy()
    for b, L in enumerate(lens):
        ly = layers[b]
        want_rho, z = oracle.delta_pages(ly.Q[:, 0, :], ly.K, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv,
                                         P=P, K_pages=K_pages, L_recent=L_recent)
        n_pages = len(z)
        assert np.isfinite(S[b, :n_pages]).all()
        np.testing.assert_allclose(S[b, :n_pages], z, rtol=1e-4, atol=1e-9)
        n_recent = min(L_recent, n_pages)
        keep = min(K_pages - L_recent, n_pages - n_recent)
        np.testing.assert_array_equal(rho[b, keep:keep + n_recent],
                                      np.arange(n_pages - n_recent, n_pages))
        assert_topk_parity(rho[b][None, :keep], z[None, :n_pages - n_recent], keep, rel=1e-4)


@pytest.mark.parametrize("reduce", [1, 2], ids=["sum", "max"])
def test_raw_outliers(kvs, reduce):
    """Raw logits with outlier keys: the same fp32 error bound as ordinary inputs."""
    L, W, d_k, H_q, H_kv = 4113, 8, 128, 32, 8
    ly = synth.gaussian_layer(61, L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L)
    rng = np.random.default_rng(7)
    out = [(g, i % 3, int(rng.integers(0, L)), LIFTS[i % 3]) for g in range(H_kv) for i in range(4)]
    ly = synth.plant_outliers(ly, 62, out)
    a = kvs.raw_args(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=L, reduce=reduce)
    got = kvs.kvs_score_raw(kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K), a)
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    kw = dict(L=L, W=W, d_k=d_k, H_q=H_q, H_kv=H_kv)
    want = oracle.score_raw(ly.Q, ly.K, reduce=reduce, **kw)
    absb = lambda b: (np.asarray(b, np.uint16) & np.uint16(0x7FFF)).astype(np.uint16)
    bound = oracle.score_raw(absb(ly.Q), absb(ly.K), reduce=1, **kw)
    assert np.all(np.abs(got - want) <= 2.0 ** -16 * bound + 1e-30)
