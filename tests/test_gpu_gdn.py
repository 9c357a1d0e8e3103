"""Gated delta rule decode step (kd_gdn_step) against the oracle's gdn_step.

Bar: fp32 on the device against fp64: every state element and output within 2e-5 of the
oracle, scaled by the rms of its head's state (a 128-term dot product in fp32 per row, then
one fused update); over 8 recurrent steps the same bar at 1e-4.  Rows are bit-identical to
their B = 1 call, and the in-place call equals the ping-pong one bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

kd = pytest.importorskip("session_decode_step_amd")
D = 128


def _inputs(r, B, H):
    q = r.standard_normal((B, H, D)).astype(np.float32)
    k = r.standard_normal((B, H, D))
    k = (k / np.linalg.norm(k, axis=2, keepdims=True)).astype(np.float32)
    q = (q / np.linalg.norm(q, axis=2, keepdims=True)).astype(np.float32)
    v = r.standard_normal((B, H, D)).astype(np.float32)
    g = (-r.uniform(0.0, 2.0, (B, H))).astype(np.float32)
    beta = r.uniform(0.0, 1.0, (B, H)).astype(np.float32)
    return q, k, v, g, beta


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def _close(got, ref, tol, what):
    for h in range(ref.shape[0]):
        scale = max(np.sqrt(np.mean(ref[h] ** 2)), 1e-30)
        err = np.max(np.abs(got[h].astype(np.float64) - ref[h])) / scale
        assert err <= tol, f"{what} head {h}: {err:.3e} > {tol}"


@pytest.mark.parametrize("B,H", [(1, 1), (5, 4), (16, 32)])
def test_gdn_step_matches_oracle(B, H):
    say(f"gdn B={B} H={H}")
    r = np.random.default_rng(B * 100 + H)
    q, k, v, g, beta = _inputs(r, B, H)
    S0 = [r.standard_normal((H, D, D)).astype(np.float32) for _ in range(B)]
    sin = [_dev(s) for s in S0]
    sout = [torch.empty_like(s) for s in sin]
    scale = D ** -0.5
    o = kd.kd_gdn_step(_dev(q), _dev(k), _dev(v), _dev(g), _dev(beta), [s.data_ptr() for s in sin],
                       [s.data_ptr() for s in sout], scale).cpu().numpy()
    for b in range(B):
        Sn, on = oracle.gdn_step(S0[b], q[b], k[b], v[b], g[b], beta[b], scale)
        _close(sout[b].cpu().numpy(), Sn, 2e-5, f"state row {b}")
        for h in range(H):
            err = np.max(np.abs(o[b, h] - on[h])) / max(np.sqrt(np.mean(Sn[h] ** 2)) * scale, 1e-30)
            assert err <= 2e-5, f"o row {b} head {h}: {err:.3e}"
        np.testing.assert_array_equal(sin[b].cpu().numpy(), S0[b])     # the input state is untouched
    # rows are B-invariant, and the in-place call equals the ping-pong one
    for b in (0, B - 1):
        s1 = torch.empty_like(sin[b])
        o1 = kd.kd_gdn_step(_dev(q[b:b + 1]), _dev(k[b:b + 1]), _dev(v[b:b + 1]), _dev(g[b:b + 1]),
                            _dev(beta[b:b + 1]), [sin[b].data_ptr()], [s1.data_ptr()], scale).cpu().numpy()
        np.testing.assert_array_equal(o1[0].view(np.uint32), o[b].view(np.uint32))
        np.testing.assert_array_equal(s1.cpu().numpy().view(np.uint32), sout[b].cpu().numpy().view(np.uint32))
    ip = [s.clone() for s in sin]
    oi = kd.kd_gdn_step(_dev(q), _dev(k), _dev(v), _dev(g), _dev(beta), [s.data_ptr() for s in ip],
                        [s.data_ptr() for s in ip], scale).cpu().numpy()
    np.testing.assert_array_equal(oi.view(np.uint32), o.view(np.uint32))
    for b in range(B):
        np.testing.assert_array_equal(ip[b].cpu().numpy().view(np.uint32), sout[b].cpu().numpy().view(np.uint32))


def test_gdn_recurrence_over_steps():
    """Eight steps in place from a zero state: the state and outputs follow the oracle's
    recurrence; with beta = 1, no decay and a repeated unit key the state recalls v at k."""
    say("gdn recurrence")
    B, H, steps = 3, 8, 8
    r = np.random.default_rng(7)
    st = [torch.zeros((H, D, D), dtype=torch.float32, device="cuda") for _ in range(B)]
    S = [np.zeros((H, D, D)) for _ in range(B)]
    scale = D ** -0.5
    for t in range(steps):
        q, k, v, g, beta = _inputs(r, B, H)
        o = kd.kd_gdn_step(_dev(q), _dev(k), _dev(v), _dev(g), _dev(beta), [s.data_ptr() for s in st],
                           [s.data_ptr() for s in st], scale).cpu().numpy()
        for b in range(B):
            S[b], on = oracle.gdn_step(S[b], q[b], k[b], v[b], g[b], beta[b], scale)
            _close(st[b].cpu().numpy(), S[b], 1e-4, f"step {t} row {b}")
            for h in range(H):
                assert np.max(np.abs(o[b, h] - on[h])) <= 1e-4 * max(np.sqrt(np.mean(S[b][h] ** 2)), 1e-30)
    # write-and-recall: no decay, beta = 1, query = key
    q, k, v, g, beta = _inputs(r, B, H)
    o = kd.kd_gdn_step(_dev(k), _dev(k), _dev(v), _dev(np.zeros_like(g)), _dev(np.ones_like(beta)),
                       [s.data_ptr() for s in st], [s.data_ptr() for s in st], 1.0).cpu().numpy()
    np.testing.assert_allclose(o, v, rtol=0, atol=2e-4 * np.abs(v).max())


def test_gdn_degenerate_cases():
    """No decay and beta = 0 leave the state unchanged bit for bit (exp(0) = 1 and a zero
    correction are exact); beta = 0 alone is a pure decay; a zero state with a unit key and
    beta = 1 becomes v k^T, whose readout at q = k is v."""
    say("gdn degenerate cases")
    B, H = 4, 8
    r = np.random.default_rng(11)
    q, k, v, g, beta = _inputs(r, B, H)
    S0 = [r.standard_normal((H, D, D)).astype(np.float32) for _ in range(B)]
    sin = [_dev(s) for s in S0]
    sout = [torch.empty_like(s) for s in sin]
    zeros = np.zeros((B, H), dtype=np.float32)
    kd.kd_gdn_step(_dev(q), _dev(k), _dev(v), _dev(zeros), _dev(zeros), [s.data_ptr() for s in sin],
                   [s.data_ptr() for s in sout], 1.0)
    for b in range(B):
        np.testing.assert_array_equal(sout[b].cpu().numpy().view(np.uint32), S0[b].view(np.uint32))
    kd.kd_gdn_step(_dev(q), _dev(k), _dev(v), _dev(g), _dev(zeros), [s.data_ptr() for s in sin],
                   [s.data_ptr() for s in sout], 1.0)
    for b in range(B):
        ref = np.exp(g[b].astype(np.float64))[:, None, None] * S0[b]
        _close(sout[b].cpu().numpy(), ref, 1e-6, f"pure decay row {b}")
    zs = [torch.zeros((H, D, D), dtype=torch.float32, device="cuda") for _ in range(B)]
    o = kd.kd_gdn_step(_dev(k), _dev(k), _dev(v), _dev(zeros), _dev(np.ones_like(zeros)), [s.data_ptr() for s in zs],
                       [s.data_ptr() for s in zs], 1.0).cpu().numpy()
    for b in range(B):
        ref = v[b].astype(np.float64)[:, :, None] * k[b].astype(np.float64)[:, None, :]
        _close(zs[b].cpu().numpy(), ref, 1e-6, f"zero state row {b}")
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-5 * np.abs(v).max())
