"""Block selection against the oracle on unplanted inputs (GPU).

Gaussian queries and keys give flat block softmaxes: the 0.9-mass crossing
falls among many blocks of nearly equal probability, which exercises the
select's long-list path (more radix digits over the crossing bin) rather than
the one-wave finish that planted inputs reach.  Also small and full masses.
The parity rule is the one of the chunked-prefill workload: a block whose
preceding mass is more than 2e-3 (relative) away from p_mass is classified
exactly as the oracle does.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu
REL = 2e-3


@pytest.fixture(scope="module")
def kvs():
    import prompt_token_importance_amd as k
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    return k


@pytest.mark.parametrize("L,Lq,block,H_q,H_kv,d_k,p_mass", [
    (3000, 512, 64, 8, 2, 64, 0.9),
    (3000, 512, 64, 8, 2, 64, 0.5),
    (3000, 512, 64, 8, 2, 64, 0.02),     # the crossing at the first block
    (3000, 512, 64, 8, 2, 64, 1.0),      # every visible block
    (9000, 1000, 32, 4, 4, 128, 0.9),    # ragged last query block, 282 key blocks
    (70000, 256, 64, 4, 1, 128, 0.9),    # 1094 key blocks: four per thread and more
])
def test_block_select_flat(kvs, L, Lq, block, H_q, H_kv, d_k, p_mass):
    print(f"block select L={L} Lq={Lq} block={block} p={p_mass}", flush=True)
    q_pos0 = L - Lq
    ly = synth.gaussian_layer(31 + L + Lq, L=L, W=Lq, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0)
    a = kvs.block_select_args(Lq=Lq, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv, q_pos0=q_pos0, block=block,
                              p_mass=p_mass)
    M = kvs.kvs_block_select(kvs.bf16_from_bits(ly.Q), kvs.bf16_from_bits(ly.K), a)
    torch.cuda.synchronize()
    Mo, before = oracle.block_select(ly.Q, ly.K, Lq=Lq, L=L, d_k=d_k, H_q=H_q, H_kv=H_kv,
                                     q_pos0=q_pos0, block=block, p_mass=p_mass,
                                     return_before=True)
    Mg = M.cpu().numpy()
    assert Mg.shape == Mo.shape
    decidable = np.abs(before - p_mass) > REL * p_mass
    assert np.array_equal(Mg[decidable], Mo[decidable].astype(Mg.dtype))
    visible = np.isfinite(before)
    assert not Mg[~visible].any(), "a block after the query block's end was kept"
    # the kept set of every (head, query block) holds at least the crossing block
    assert Mg.any(axis=2).all()
