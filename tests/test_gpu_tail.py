"""Packed-tail gather/scatter on the GPU against the plain reference
(oracle.planner_ref.tail_pack): bit-exact, zero gaps, > 64 tensors (several
launches), large tensors (several workgroups), unaligned sources (scalar
path), and AdamW on the packed tail unpacked back per tensor."""

import numpy as np
import pytest
import torch

import matrix_optimizer_step_owner_amd as mf
import oracle

from gpu_helpers import ADAMW_TOL, f64, rel, say

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tensors(seed, unaligned=True):
    gen = torch.Generator().manual_seed(seed)
    shapes = [(4096,), (7,), (0,), (3, 5), (2, 3, 4), (1,), (50001,), (64, 65)]
    shapes += [(int(k),) for k in np.random.default_rng(seed).integers(1, 300, 70)]
    host = [torch.randn(s, generator=gen) for s in shapes]
    dev = [h.to("cuda") for h in host]
    if unaligned:   # views 4 bytes into their storage: not 16-byte aligned
        for i in (1, 3, 9, 20):
            base = torch.randn(host[i].numel() + 1, generator=gen)
            host[i] = base[1:].reshape(host[i].shape)
            dev[i] = base.to("cuda")[1:].reshape(host[i].shape)
    return host, dev


def test_pack_unpack_bit_exact():
    host, dev = _tensors(0)
    say(f"{len(dev)} tensors, {sum(t.numel() for t in dev)} elements")
    packed, offs = mf.tail_pack(dev)
    torch.cuda.synchronize()
    want, want_offs = oracle.planner_ref.tail_pack([h.numpy() for h in host])
    assert offs == want_offs
    assert np.array_equal(packed.cpu().numpy(), want)
    out = [torch.full_like(t, float("nan")) for t in dev]
    mf.tail_unpack(packed, out, offs)
    torch.cuda.synchronize()
    for o, h in zip(out, host):
        assert torch.equal(o.cpu(), h)


def test_pack_leaves_outside_elements():
    host, dev = _tensors(1, unaligned=False)
    offs, total = mf.tail_layout([t.numel() for t in dev])
    # spread the segments out: 8 extra elements before each
    offs = [o + 8 * (i + 1) for i, o in enumerate(offs)]
    packed = torch.full((total + 8 * (len(dev) + 1),), 7.0, device="cuda")
    mf.tail_pack(dev, packed=packed, offsets=offs)
    torch.cuda.synchronize()
    p = packed.cpu().numpy()
    covered = np.zeros(p.size, dtype=bool)
    for t, o in zip(host, offs):
        span = (t.numel() + 3) // 4 * 4
        covered[o:o + span] = True
        assert np.array_equal(p[o:o + t.numel()], t.numpy().ravel())
        assert np.all(p[o + t.numel():o + span] == 0.0)
    assert np.all(p[~covered] == 7.0)


def test_adamw_on_packed_tail_then_unpack():
    host, dev = _tensors(2)
    gen = torch.Generator().manual_seed(9)
    grads_h = [torch.randn(h.shape, generator=gen) * 1e-3 for h in host]
    packed_p, offs = mf.tail_pack(dev)
    packed_g, _ = mf.tail_pack([g.to("cuda") for g in grads_h])
    m = torch.zeros_like(packed_p)
    v = torch.zeros_like(packed_p)
    hp = dict(lr=0.02, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.01)
    mf.adamw_tail(packed_p, packed_g, m, v, step=1, **hp)
    out = [torch.empty_like(t) for t in dev]
    mf.tail_unpack(packed_p, out, offs)
    torch.cuda.synchronize()
    for o, h, g in zip(out, host, grads_h):
        z = np.zeros(h.numel())
        want, _, _ = oracle.adamw_tail(f64(h).ravel(), f64(g).ravel(), z, z, step=1, **hp)
        assert rel(f64(o).ravel(), want) <= ADAMW_TOL
    # the padding gaps stay zero under AdamW
    p = packed_p.cpu().numpy()
    for h, o in zip(host, offs):
        span = (h.numel() + 3) // 4 * 4
        assert np.all(p[o + h.numel():o + span] == 0.0)
