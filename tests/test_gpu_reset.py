"""GPU parity of ReSET's step-aware temperature (nvfp4_reset_temperature)
against the oracle (oracle/reset.py).

* Token entropy: within a bound derived from the binary32 arithmetic, at
  the Qwen3 vocabulary size (151936) and ragged sizes, for Gaussian logits
  of several spreads, uniform rows (log V), a dominant logit, and masked
  (-inf) logits (compared with the oracle on the unmasked entries).
* The temperature rule and the step statistics (parity unpinned: their
  formula is this library's reading): the decision H < tau0 and the rule
  are evaluated by the oracle on the GPU's own binary32 entropies, in the
  kernel's precision; the step state is followed over a sequence of calls.
* The scaled logits: bit-exact binary32 divisions by the row temperature,
  written to a separate buffer or in place.
* Run-to-run bit stability and graph replay."""

import numpy as np
import pytest

from gpu_util import note
from oracle import reset

pytestmark = pytest.mark.gpu

U = 2.0 ** -24
V_QWEN3 = 151936


@pytest.fixture(scope="module")
def nv():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import nvfp4_decode_linear_amd as nv
    return nv


def _params(nv, t_low=0.1, tau0=0.5505, t_base=0.6, t_max=1.5):
    return nv.ResetParams(t_low, tau0, t_base, t_max)


def _bound(z):
    """|H - H_ref| bound per row: every exponential and the shift z - max
    carry a relative error of at most (|z - max| + 2) u, every addition u
    along a chain of 16 (per thread) + 6 (wave tree) + 3 (waves) + the
    number of 4096-logit groups (their combination); the entropy
    log S - T / S amplifies relative errors of S and T by 1 + 2 |T / S|."""
    z = np.asarray(z, np.float64)
    fin = np.isfinite(z)
    m = np.max(np.where(fin, z, -np.inf), axis=1, keepdims=True)
    d = np.where(fin, m - z, 0.0)
    groups = -(-z.shape[1] // 4096)
    chain = 16 + 6 + 3 + groups + 4
    # T / S = mean of (z - m) under softmax
    e = np.where(fin, np.exp(-d), 0.0)
    ts = np.sum(e * d, axis=1) / np.sum(e, axis=1)
    href = reset.token_entropy(np.where(fin, z, -1e300))
    return U * (chain + np.max(d, axis=1) + 2) * (1 + 2 * ts) + 4 * U * np.abs(href) + 1e-7


def _run(nv, z_np, state=None, step_end=None, out=None, params=None):
    import torch
    M, V = z_np.shape
    ld = -(-V // 4) * 4                      # the row stride must be a multiple of 4
    buf = np.full((M, ld), np.nan, np.float32)
    buf[:, :V] = z_np
    z = torch.from_numpy(buf).cuda()[:, :V]
    st = torch.zeros((M, 2), dtype=torch.float32, device="cuda") if state is None else state
    se = None if step_end is None else torch.tensor(step_end, dtype=torch.int32, device="cuda")
    h, t, o = nv.reset_temperature(z, params or _params(nv), st, se, out=out)
    torch.cuda.synchronize()
    return z, st, h.cpu().numpy(), t.cpu().numpy(), o


def _check_entropy(h, z_np):
    z = np.asarray(z_np, np.float64)
    fin = np.isfinite(z)
    # masked entries have probability 0: the oracle on the finite entries of each row
    ref = np.array([reset.token_entropy(z[r:r + 1, fin[r]])[0] for r in range(z.shape[0])])
    b = _bound(z)
    err = np.abs(h.astype(np.float64) - ref)
    assert np.all(err <= b), f"max err/bound {np.max(err / b)} (err {np.max(err)})"
    return ref


@pytest.mark.parametrize("M", [1, 2, 8])
@pytest.mark.parametrize("sigma", [1.0, 4.0, 12.0])
def test_entropy_qwen3_vocab(nv, M, sigma):
    note(f"reset entropy M={M} V={V_QWEN3} sigma={sigma}")
    rng = np.random.default_rng([26, M, int(sigma)])
    z = (rng.standard_normal((M, V_QWEN3)) * sigma).astype(np.float32)
    _, _, h, _, _ = _run(nv, z)
    _check_entropy(h, z)


@pytest.mark.parametrize("V", [1, 5, 100, 4095, 4096, 4097, 12289, V_QWEN3 + 3, 1 << 20])
def test_entropy_ragged_vocab(nv, V):
    note(f"reset entropy ragged V={V}")
    rng = np.random.default_rng(V)
    z = (rng.standard_normal((3, V)) * 3.0).astype(np.float32)
    _, _, h, _, _ = _run(nv, z)
    _check_entropy(h, z)
    if V == 1:
        assert np.all(h == 0.0)


def test_entropy_special_rows(nv):
    note("reset entropy special rows")
    V = V_QWEN3
    z = np.zeros((4, V), np.float32)
    z[0] = 2.5                                            # uniform: log V
    z[1, 123456] = 80.0                                   # one dominant logit: ~0
    rng = np.random.default_rng(4)
    z[2] = rng.standard_normal(V) * 2
    z[2, rng.choice(V, V // 2, replace=False)] = -np.inf  # half of the vocabulary masked
    z[3] = rng.standard_normal(V) * 2
    z[3, :V - 10] = -np.inf                               # all but the last 10 masked
    _, _, h, _, _ = _run(nv, z)
    ref = _check_entropy(h, z)
    assert abs(h[0] - np.log(V)) <= 64 * U * np.log(V)
    assert 0.0 <= h[1] < 1e-6
    assert ref[3] < np.log(10) + 1e-12


def test_temperature_rule_and_step_state(nv):
    """Six tokens of four rows with steps closing at chosen tokens: the
    state (sum, count) and the temperature follow the oracle's reading,
    evaluated on the GPU's own entropies."""
    import torch
    note("reset temperature rule and step state")
    M, V = 4, 8192
    p = _params(nv, t_low=0.1, tau0=2.0, t_base=0.6, t_max=0.9)
    st = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    rng = np.random.default_rng(9)
    ssum, scnt = np.zeros(M), np.zeros(M)
    ends = [[0, 0, 0, 0], [0, 1, 0, 0], [1, 0, 0, 1], [0, 0, 1, 0], [0, 1, 0, 0], [1, 1, 1, 1]]
    seen_low = seen_high = False
    for k, se in enumerate(ends):
        # spreads chosen so that rows cross tau0 = 2 nats in both directions
        sig = np.array([0.5, 3.0, 8.0, 30.0])[(np.arange(M) + k) % M]
        z = (rng.standard_normal((M, V)) * sig[:, None]).astype(np.float32)
        _, _, h, t, _ = _run(nv, z, state=st, step_end=se, params=p)
        _check_entropy(h, z)
        h64 = h.astype(np.float64)
        ssum, scnt, hstep = reset.step_update(ssum, scnt, h64, np.array(se))
        got = st.cpu().numpy()
        assert np.allclose(got[:, 1], scnt) and np.all(got[:, 1] == scnt)
        # the running sum in binary32 (one rounding per token)
        assert np.all(np.abs(got[:, 0] - ssum) <= 8 * U * np.maximum(np.abs(ssum), 1.0))
        want = reset.temperature(h64, got[:, 0].astype(np.float64) / got[:, 1], p.t_low,
                                 np.float32(p.tau0), p.t_base, p.t_max)
        low = h64 < np.float32(p.tau0)
        assert np.array_equal(t == np.float32(p.t_low), low)   # the decision, exactly
        assert np.all(np.abs(t - want) <= 4 * U * want), (t, want)
        seen_low |= bool(low.any())
        seen_high |= bool((~low).any())
    assert seen_low and seen_high                       # both branches of the rule ran


@pytest.mark.parametrize("inplace", [False, True])
def test_scaled_logits_bit_exact(nv, inplace):
    import torch
    note(f"reset scaled logits inplace={inplace}")
    M, V = 3, V_QWEN3 + 1
    rng = np.random.default_rng(11)
    z = (rng.standard_normal((M, V)) * 5).astype(np.float32)
    zz = np.zeros((M, V + 3), np.float32)                  # row stride V + 3 (a multiple of 4)
    zz[:, :V] = z
    zt = torch.from_numpy(zz).cuda()[:, :V]
    st = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    # a separate output: row stride V + 3 (a multiple of 4), padding kept
    ob = torch.full((M, V + 3), float("nan"), device="cuda")
    out = "inplace" if inplace else ob[:, :V]
    h, t, o = nv.reset_temperature(zt, _params(nv), st, None, out=out)
    torch.cuda.synchronize()
    want = reset.scale_logits(z, t.cpu().numpy())
    assert np.array_equal(o.cpu().numpy(), want)
    if inplace:
        assert np.array_equal(zt.cpu().numpy(), want)
    else:
        assert np.array_equal(zt.cpu().numpy(), z)               # input untouched
        assert np.all(np.isnan(ob[:, V:].cpu().numpy()))         # padding untouched


def test_bit_stable_and_graph_replay(nv):
    import torch
    note("reset determinism and graph replay")
    M, V = 8, V_QWEN3
    rng = np.random.default_rng(12)
    z = torch.from_numpy((rng.standard_normal((M, V)) * 4).astype(np.float32)).cuda()
    p = _params(nv)
    st = torch.zeros((M, 2), dtype=torch.float32, device="cuda")
    h0, t0, _ = nv.reset_temperature(z, p, st)
    h1, t1, _ = nv.reset_temperature(z, p, st)
    torch.cuda.synchronize()
    assert np.array_equal(h0.cpu().numpy().view(np.uint32), h1.cpu().numpy().view(np.uint32))
    out = torch.empty_like(z)
    ent = torch.empty(M, device="cuda")
    tmp = torch.empty(M, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())

    def call():
        h, t, _ = nv.reset_temperature(z, p, st, None, out=out)
        ent.copy_(h)
        tmp.copy_(t)
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        call()
    for r in range(3):
        z.copy_(torch.from_numpy((rng.standard_normal((M, V)) * (2 + r)).astype(np.float32)))
        st.zero_()
        torch.empty(1 << 20, device="cuda").fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        he, te = ent.clone(), tmp.clone()
        oe = out.clone()
        st.zero_()
        h, t, o = nv.reset_temperature(z, p, st, None, out=torch.empty_like(z))
        torch.cuda.synchronize()
        assert np.array_equal(he.cpu().numpy().view(np.uint32), h.cpu().numpy().view(np.uint32))
        assert np.array_equal(te.cpu().numpy().view(np.uint32), t.cpu().numpy().view(np.uint32))
        assert np.array_equal(oe.cpu().numpy().view(np.uint32), o.cpu().numpy().view(np.uint32))
