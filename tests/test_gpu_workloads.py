"""Full-size parity of the three large owner-share workloads.

Each test runs ONE grouped mfsdp_muon_step over the whole workload, exactly as
bench.py launches it, then checks against the float64 oracle:

* oracle matrices: the full Muon step (O, M', W', per tensor and per 256 x 256
  tile) of every distinct shape of the Llama-3-8B and 32B-class shares -- the
  square, the short-K 1024-row, the tall and the wide long-K matrices, which
  carry most of the Newton-Schulz work -- and of all 512 many-small
  matrices;
* every matrix: M' = beta*M + G on sampled elements (computable one by one);
* grouping does not change results: a matrix run alone gives bitwise the same
  W' as inside the grouped call (one matrix of a later block).

The d=2048 block is checked matrix by matrix in test_gpu_parity.py.
"""

import numpy as np
import pytest
import torch

import matrix_optimizer_step_owner_amd as mf
from matrix_optimizer_step_owner_amd import workloads as wlm

from gpu_helpers import (GpuStep, check_matrix, f64, muon_hparams, oracle_matrix, say)

pytestmark = [pytest.mark.gpu, pytest.mark.slow, pytest.mark.timeout(1200)]


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def sampled_momentum_check(inp, st, hp, n_samples=4096, seed=0):
    rng = np.random.default_rng(seed)
    beta = hp["beta"]
    for i, (G, M0) in enumerate(zip(inp.grads, inp.momenta)):
        r, c = G.shape
        rows = rng.integers(0, r, n_samples)
        cols = rng.integers(0, c, n_samples)
        g = G[rows, cols].double().numpy()
        m0 = M0[rows, cols].double().numpy()
        want = beta * m0 + g
        got = st.M[i][torch.from_numpy(rows).to(st.M[i].device),
                      torch.from_numpy(cols).to(st.M[i].device)].double().cpu().numpy()
        # bf16 storage of M': each element within half an ulp (plus fp32 slack)
        tol = np.abs(want) * 2.0 ** -8 + 1e-30
        assert np.all(np.abs(got - want) <= tol), f"matrix {i}: M' off at sampled elements"


def run_workload(key, check_idx, alone_idx):
    say(f"== workload {key}: generating")
    inp = wlm.generate(key, seed=0)
    wl = inp.workload
    hp = muon_hparams(wl)
    n = len(inp.weights)
    W0 = {i: f64(inp.weights[i]) for i in check_idx}
    mask = [i in set(check_idx) for i in range(n)]
    say(f"== workload {key}: {n} matrices, one grouped call")
    st = GpuStep(inp.weights, inp.grads, inp.momenta, update_mask=mask)
    st.run(**hp)
    for i in check_idx:
        ref = oracle_matrix(inp.weights[i], inp.grads[i], inp.momenta[i], hp)
        check_matrix(i, W0.pop(i), f64(inp.grads[i]), f64(inp.momenta[i]), f64(st.W[i]),
                     f64(st.M[i]), f64(st.U[i]), ref, wl.dtype, hp["beta"], label=key)
        st.U[i] = None
        del ref
    sampled_momentum_check(inp, st, hp)
    for i in alone_idx:
        one = GpuStep([inp.weights[i]], [inp.grads[i]], [inp.momenta[i]],
                      update_mask=[False])
        one.run(**hp)
        assert torch.equal(one.W[0], st.W[i]), f"{key}: matrix {i} alone != grouped"
        assert torch.equal(one.M[0], st.M[i])
        say(f"{key}: matrix {i} {tuple(inp.weights[i].shape)} alone == grouped (bitwise)")
        del one
    del st
    torch.cuda.empty_cache()


def test_llama3_8b_4blocks_full():
    # oracle: block 0 Wq (4096 x 4096), Wk and Wv (1024 x 4096), gate
    # (14336 x 4096, tall) and down (4096 x 14336, wide);
    # alone == grouped: block 1 gate and block 3 down
    run_workload("llama3_8b_4blocks", check_idx=[0, 2, 3, 4, 6], alone_idx=[11, 27])


def test_many_small_full():
    # 512 matrices in one call, every one against the oracle
    run_workload("many_small", check_idx=list(range(512)), alone_idx=[3, 260])


def test_d5120_2blocks_full():
    # oracle: block 0 Wq (5120 x 5120), Wk (1024 x 5120), gate (27648 x 5120,
    # tall) and down (5120 x 27648, wide);
    # alone == grouped: block 1 gate and down
    run_workload("d5120_2blocks", check_idx=[0, 2, 4, 6], alone_idx=[11, 13])
