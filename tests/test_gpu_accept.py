"""GPU parity of MTP draft verification (moe_mtp_accept) with the CPU oracle,
through the C ABI.

Kept-draft counts and emitted tokens are integers decided in fp64 on both
sides; the GPU sums its softmax normalisers and draw masses per 4096-token
chunk in a fixed order, the oracle sequentially, so the two could differ
only where a sampled decision lies within rounding of its boundary.  The
oracle reports each sequence's smallest relative decision margin: at the
seeds used here every margin exceeds 1e-10 (asserted), far above the
~1e-15 relative rounding of either side, so every sequence must match the
oracle exactly.  Greedy decisions compare fp32 logits and are exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu

V_FULL = 320000   # the order of the pages' 320k-merge BPE vocabulary


@pytest.fixture(scope="module")
def m(dev):
    from quantized_moe_noaux_amd import moe
    return moe


def run(m, dev, draft, p, q, tau, u):
    B, D1, V = p.shape
    D = D1 - 1
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a, dtype=dt)).to(dev)
    dr = t(np.asarray(draft).reshape(B, D), np.int32)
    pt = t(p, np.float32)
    qt = t(np.asarray(q).reshape(B, D, V), np.float32) if D else torch.empty(0, device=dev)
    ut = t(np.asarray(u).reshape(B, D + 1), np.float64)
    n = torch.full((B,), -7, dtype=torch.int32, device=dev)
    nx = torch.full((B,), -7, dtype=torch.int32, device=dev)
    ws = m.workspace(m.moe_mtp_accept_workspace_bytes(B, D, V), dev)
    m.moe_mtp_accept(dr, pt, qt if D else None, tau, ut, n, nx, ws)
    torch.cuda.synchronize()
    return n.cpu().numpy(), nx.cpu().numpy()


def check(m, dev, draft, p, q, tau, u, what=""):
    print("mtp accept parity: %s B=%d D=%d V=%d tau=%g" % (what, p.shape[0], p.shape[1] - 1, p.shape[2], tau),
          flush=True)
    n, nx = run(m, dev, draft, p, q, tau, u)
    n_ref, nx_ref, mg = oracle.mtp_accept(draft, p, q, tau, u)
    if tau > 0:
        low = np.flatnonzero(mg <= 1e-10)
        assert low.size == 0, "sequences %s decide within 1e-10 of a boundary (margins %s)" % (low, mg[low])
    assert np.array_equal(n, n_ref), (n, n_ref)
    assert np.array_equal(nx, nx_ref), (nx, nx_ref)
    return n, nx


@pytest.mark.parametrize("tau", [0.7, 1.0, 0.0])
def test_full_vocabulary(dev, m, tau):
    d, p, q, u = synth.mtp_inputs(11, 8, 4, V_FULL, tau)
    n, _ = check(m, dev, d, p, q, tau, u, "full vocabulary")
    if tau > 0:
        assert 0 < n.mean() < 4        # some drafts kept, some refused


@pytest.mark.parametrize("V", [3, 1000, 4096, 4097, 9999, 65536 + 12])
def test_ragged_vocabularies(dev, m, V):
    # one chunk, exactly one chunk, one token past a chunk, V % 4 != 0 (scalar
    # loads), several chunks
    for tau in (0.7, 0.0):
        d, p, q, u = synth.mtp_inputs(V, 16, 3, V, tau, sigma_p=1.5, sigma_n=0.7)
        check(m, dev, d, p, q, tau, u, "ragged")


@pytest.mark.parametrize("D", [0, 1, 2, 5, 16])
def test_draft_depths(dev, m, D):
    d, p, q, u = synth.mtp_inputs(100 + D, 12, D, 50000, 0.7, sigma_p=2.0, sigma_n=0.6)
    check(m, dev, d, p, q, 0.7, u, "depth")


def test_many_sequences(dev, m):
    d, p, q, u = synth.mtp_inputs(5, 64, 3, 20000, 0.9)
    check(m, dev, d, p, q, 0.9, u, "batch")


def test_equal_draft_and_target_keep_everything(dev, m):
    d, p, q, u = synth.mtp_inputs(6, 8, 4, 30000, 0.7)
    n, _ = check(m, dev, d, p, p[:, :4], 0.7, u, "q = p")
    assert (n == 4).all()


def test_greedy_ties_and_full_acceptance(dev, m):
    rng = np.random.default_rng(9)
    B, D, V = 32, 4, 5000
    p = rng.integers(-2, 3, (B, D + 1, V)).astype(np.float32)      # many exact ties
    am = np.argmax(p, axis=2)
    draft = am[:, :D].copy()
    draft[::3, 2] = (draft[::3, 2] + 1) % V
    q = rng.normal(0, 1, (B, D, V)).astype(np.float32)
    u = rng.random((B, D + 1))
    n, nx = check(m, dev, draft, p, q, 0.0, u, "greedy ties")
    assert (n[1::3] == D).all() and (nx[1::3] == am[1::3, D]).all()


def test_peaked_and_flat_distributions(dev, m):
    # very peaked rows (most tokens underflow to zero probability) and flat ones
    for sp, sn in ((40.0, 5.0), (0.05, 0.05)):
        d, p, q, u = synth.mtp_inputs(int(sp * 100), 16, 3, 12000, 0.7, sigma_p=sp, sigma_n=sn)
        check(m, dev, d, p, q, 0.7, u, "sigma_p=%g" % sp)


def test_small_residual(dev, m):
    # q = p except for the draft token's logit, raised a hair: the draft is
    # refused (u near 1) and max(0, p - q) keeps only ~1e-3 of p's mass, a
    # difference of nearly equal numbers on both sides
    d, p, q, u = synth.mtp_inputs(8, 16, 1, 4096, 1.0)
    q = p[:, :1].copy()
    for b in range(16):
        q[b, 0, d[b, 0]] += 1e-3
    u[:, 0] = 0.9999999
    check(m, dev, d, p, q, 1.0, u, "tiny residual")


def test_deterministic(dev, m):
    d, p, q, u = synth.mtp_inputs(12, 8, 4, 100000, 0.7)
    a = run(m, dev, d, p, q, 0.7, u)
    b = run(m, dev, d, p, q, 0.7, u)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_out_of_range_draft_is_refused(dev, m):
    d, p, q, u = synth.mtp_inputs(13, 4, 3, 8192, 0.7)
    d[:, 1] = -1
    d[2, 1] = 8192
    u[:, 0] = 0.0                     # the first draft is always kept
    n, nx = run(m, dev, d, p, q, 0.7, u)
    assert (n == 1).all() and ((0 <= nx) & (nx < 8192)).all()
