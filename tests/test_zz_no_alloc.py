"""The step without a caller workspace (mfsdp_muon_step_noalloc) against the
step with one (mfsdp_muon_step), through the C ABI on cuda:0.

Two calls in a row share the library's static scratch; the second has a
smaller list, so it runs over what the first left there.  Each must give
bitwise the results of mfsdp_muon_step on the same inputs (the no-alloc call
keeps every Newton-Schulz group on the caller's stream, and results do not
depend on the grouping), and both are checked against the float64 oracle.
"""

import numpy as np
import pytest
import torch

import matrix_optimizer_step_owner_amd as mf
from matrix_optimizer_step_owner_amd import workloads as wlm

from gpu_helpers import GpuStep, check_matrix, f64, muon_hparams, oracle_matrix, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare(shapes, dtype, seed, label):
    Ws, Gs, Ms = wlm.random_matrix_inputs(shapes, dtype, seed=seed)
    hp = muon_hparams()
    need = mf.muon_workspace_size(shapes, dtype)
    assert need <= mf.NOALLOC_SCRATCH_BYTES
    ref = GpuStep(Ws, Gs, Ms)
    ref.run(**hp)
    got = GpuStep(Ws, Gs, Ms)
    mf.muon_step_noalloc(got.W, got.G, got.M, update_out=got.U, **hp)
    torch.cuda.synchronize()
    for i in range(len(shapes)):
        assert torch.equal(got.W[i], ref.W[i]), (label, i)
        assert torch.equal(got.M[i], ref.M[i]), (label, i)
        assert torch.equal(got.U[i], ref.U[i]), (label, i)
        r = oracle_matrix(Ws[i], Gs[i], Ms[i], hp)
        check_matrix(i, f64(Ws[i]), f64(Gs[i]), f64(Ms[i]), f64(got.W[i]), f64(got.M[i]),
                     f64(got.U[i]), r, dtype, hp["beta"], label=label)
    say(f"{label}: {len(shapes)} matrices, workspace {need} bytes, bitwise equal to "
        f"mfsdp_muon_step")


def test_noalloc_step_twice_then_smaller():
    # first call: five matrices (46 MB of workspace), two stream groups in
    # mfsdp_muon_step; second call: two smaller matrices over the leftovers
    _compare([(512, 512), (1536, 512), (512, 1536), (300, 700), (2048, 2048)],
             torch.bfloat16, 21, "noalloc call 1")
    _compare([(256, 512), (130, 77)], torch.bfloat16, 22, "noalloc call 2 (smaller)")
    _compare([(64, 200), (96, 96)], torch.float32, 23, "noalloc call 3 (fp32)")


def test_noalloc_refuses_oversize_list_on_gpu():
    dev = torch.device("cuda:0")
    W = torch.zeros(8192, 8192, dtype=torch.bfloat16, device=dev)
    G, M = torch.zeros_like(W), torch.zeros_like(W)
    with pytest.raises(mf.MfsdpError) as err:
        mf.muon_step_noalloc([W], [G], [M], lr=0.02)
    assert err.value.status == 3
    torch.cuda.synchronize()
    assert not W.any().item()
