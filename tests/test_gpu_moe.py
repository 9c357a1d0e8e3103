"""Index-level parity of the MoE layer's routing and grouped products (hf2q ADR-040 §0.7 F4
"Tests": the grouped expert product against the per-row one, and expert fan-out stress with
every row on the same experts and every row on different experts; Strata PR #1524 "Fresh
validation and limits": sixteen verify rows through merged experts).

* routing (kd_debug_moe_route): each row's top-8 experts equal the oracle's exactly (ties to
  the lower id), their softmax weights within 1e-6, and the expert buckets (count, rows,
  pairs) equal the ones the oracle's ids define, exactly;
* grouped products (kd_debug_mmvq_grouped, the kernels the step runs): each (row, rank)
  output of the interleaved gate/up product with the SwiGLU epilogue, and of the down
  product, is bit-identical to the plain product of that expert's matrix with that row alone.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as W
from gpu_util import requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

kd = pytest.importorskip("session_decode_step_amd")

SPEC = W.SPEC_C5
E, K, D, FE = SPEC.n_experts, SPEC.n_expert_used, SPEC.d, SPEC.expert_ffn


@pytest.fixture(scope="module")
def layer():
    """Layer 0 of the MoE workload's weights: the fp32 router and the packed experts."""
    L = W.make_layer(SPEC, 5, 0, 0)
    gu = kd.kd_pack_weight(kd.interleave_experts(L["e_gate"], L["e_up"], E))   # [E 2Fe, d]
    dn = kd.kd_pack_weight(L["e_down"])                                           # [E d, Fe]
    return {"L": L, "gu": gu, "dn": dn, "router": torch.from_numpy(L["router"]).cuda()}


def _buckets(ids: np.ndarray):
    """Per expert, the (row, pair) lists of rows routed to it in ascending row order, from
    each row's ids (the definition of the buckets the grouped products read)."""
    B = ids.shape[0]
    count = np.zeros(E, dtype=np.int64)
    rows = np.full((E, 16), -1, dtype=np.int64)
    pairs = np.full((E, 16), -1, dtype=np.int64)
    for b in range(B):
        for r in range(K):
            e = int(ids[b, r])
            rows[e, count[e]] = b
            pairs[e, count[e]] = b * K + r
            count[e] += 1
    return count, rows, pairs


def _route_and_check(z: np.ndarray, router: torch.Tensor, W_r: np.ndarray, what: str):
    zt = torch.from_numpy(z.astype(np.float32)).cuda()
    g = kd.kd_debug_moe_route(zt, router, K)
    g = {k: v.cpu().numpy() for k, v in g.items()}
    r = z.astype(np.float32).astype(np.float64) @ W_r.astype(np.float64).T
    near = 0
    for b in range(z.shape[0]):
        ids, p = oracle.router_topk(r[b], K)
        srt = np.sort(r[b])[::-1]
        if srt[K - 1] - srt[K] < 1e-6 * abs(srt[K - 1]):
            near += 1
            say(f"  {what}: row {b} near tie (gap {srt[K - 1] - srt[K]:.3e})")
            continue
        np.testing.assert_array_equal(g["ids"][b], ids, err_msg=f"{what} row {b}")
        np.testing.assert_allclose(g["p"][b], p, rtol=0, atol=1e-6, err_msg=f"{what} row {b}")
    np.testing.assert_allclose(g["logits"], r, rtol=0, atol=1e-5 * np.abs(r).max())
    # buckets: exactly those the GPU's own ids define (and, without near ties, the oracle's)
    count, rows, pairs = _buckets(g["ids"])
    np.testing.assert_array_equal(g["count"], count)
    for e in range(E):
        c = int(count[e])
        np.testing.assert_array_equal(g["rows"][e, :c], rows[e, :c])
        np.testing.assert_array_equal(g["pairs"][e, :c], pairs[e, :c])
    say(f"  {what}: {z.shape[0]} rows routed as the oracle, {near} near ties; "
        f"{int((count > 0).sum())} active experts, largest bucket {int(count.max())}")
    assert near == 0
    return g


def _grouped_equals_per_row(layer, z: np.ndarray, g, what: str):
    """The grouped gate/up (SwiGLU) and down products over the route's buckets against each
    expert's plain product with one row, bit for bit."""
    B = z.shape[0]
    x = kd.kd_quantize_act_q8(torch.from_numpy(z.astype(np.float32)).cuda())
    count = torch.from_numpy(g["count"]).cuda()
    rows = torch.from_numpy(g["rows"]).cuda()
    pairs = torch.from_numpy(g["pairs"]).cuda()
    gu, dn = layer["gu"], layer["dn"]
    gu1 = kd.PackedWeight(gu.fmt, 2 * FE, gu.k, gu.qs, gu.d)        # group 0 of E groups of 2Fe rows
    h = kd.kd_debug_mmvq_grouped(gu1, E, x, B, count, rows, pairs, B * K, swiglu=True)
    dn1 = kd.PackedWeight(dn.fmt, D, dn.k, dn.qs, dn.d)
    y = kd.kd_debug_mmvq_grouped(dn1, E, h, B * K, count, pairs, pairs, B * K, swiglu=False)
    torch.cuda.synchronize()
    hq, hd = h.qs.cpu().numpy(), h.d.cpu().numpy()
    NQf = (FE + 127) // 128
    y = y.cpu().numpy()
    for b in range(B):
        xb = kd.act_rows_view(x, b, 1)
        for r in range(K):
            e, j = int(g["ids"][b, r]), b * K + r
            h1 = kd.kd_mmvq_swiglu(kd.weight_group(gu, e, 2 * FE), xb, 1)
            np.testing.assert_array_equal(h1.qs.cpu().numpy(), hq[j * NQf * 128:(j + 1) * NQf * 128],
                                          err_msg=f"{what}: SwiGLU codes row {b} rank {r}")
            np.testing.assert_array_equal(h1.d.cpu().numpy().view(np.uint32),
                                          hd[j * NQf * 4:(j + 1) * NQf * 4].view(np.uint32))
            y1 = kd.kd_mmvq_q4_0(kd.weight_group(dn, e, D), kd.act_rows_view(h, j, 1), 1)
            np.testing.assert_array_equal(y1.cpu().numpy()[0].view(np.uint32), y[j].view(np.uint32),
                                          err_msg=f"{what}: down row {b} rank {r}")
    say(f"  {what}: {B * K} (row, rank) outputs of both grouped products equal the per-row products")


def test_routing_of_sixteen_verify_rows(layer):
    """16 rows of N(0,1)-like FFN inputs (unit-RMS rows times the norm gains' spread)."""
    rng = np.random.default_rng(71)
    z = rng.standard_normal((16, D)) * (1 + 0.1 * rng.standard_normal(D))
    g = _route_and_check(z, layer["router"], layer["L"]["router"], "random rows")
    _grouped_equals_per_row(layer, z, g, "random rows")


def test_fanout_all_rows_on_the_same_experts(layer):
    """Every row nearly the same vector: all 16 rows pick the same 8 experts, so 8 buckets
    hold 16 rows each (the grouped product's largest group)."""
    rng = np.random.default_rng(72)
    base = rng.standard_normal(D)
    z = base[None, :] + 1e-4 * rng.standard_normal((16, D))
    g = _route_and_check(z, layer["router"], layer["L"]["router"], "same experts")
    assert sorted(int(c) for c in g["count"] if c) == [16] * K
    _grouped_equals_per_row(layer, z, g, "same experts")


def test_fanout_two_clusters_of_rows(layer):
    """Rows 0..5 near one vector and rows 6..15 near another: buckets of 6 and 10 rows (the
    grouped product's two- and three-slot workgroups), each output bit-identical to its row's
    plain product."""
    rng = np.random.default_rng(74)
    a, c = rng.standard_normal(D), rng.standard_normal(D)
    z = np.concatenate([a[None, :] + 1e-4 * rng.standard_normal((6, D)),
                        c[None, :] + 1e-4 * rng.standard_normal((10, D))])
    g = _route_and_check(z, layer["router"], layer["L"]["router"], "two clusters")
    counts = sorted(int(x) for x in g["count"] if x)
    assert 6 in counts and 10 in counts, counts
    _grouped_equals_per_row(layer, z, g, "two clusters")


def test_fanout_every_row_on_its_own_experts(layer):
    """A router whose experts 8b .. 8b+7 respond to direction u_b only, and rows along u_b:
    the 16 rows take 128 distinct experts, every bucket holds one row."""
    rng = np.random.default_rng(73)
    Wr = (0.02 * rng.standard_normal((E, D))).astype(np.float32)
    idx = np.arange(16) * 97 + 5                    # 16 distinct coordinates
    for e in range(E):
        Wr[e, idx[e // K]] += np.float32(1.0 + 0.01 * (e % K))
    z = 0.05 * rng.standard_normal((16, D))
    z[np.arange(16), idx] += 4.0
    g = _route_and_check(z, torch.from_numpy(Wr).cuda(), Wr, "own experts")
    assert np.array_equal(np.sort(g["ids"], axis=1), np.arange(E).reshape(16, K))
    assert int(g["count"].max()) == 1 and int(g["count"].sum()) == E
    _grouped_equals_per_row(layer, z, g, "own experts")


def test_routing_ties_go_to_the_lower_id(layer):
    """Rows whose router logits tie exactly (duplicated router rows): the lower expert id wins
    each tie, as in the oracle."""
    rng = np.random.default_rng(74)
    Wr = (0.02 * rng.standard_normal((E, D))).astype(np.float32)
    Wr[65] = Wr[3]          # experts 3 and 65 always tie; 10 and 100 as well
    Wr[100] = Wr[10]
    Wr[3] += np.float32(0.5) * np.sign(Wr[3])   # large enough to be selected
    Wr[65] = Wr[3]
    z = np.abs(rng.standard_normal((4, D))) * np.sign(Wr[3])[None, :]   # aligned with expert 3's row
    zt = torch.from_numpy(z.astype(np.float32)).cuda()
    g = kd.kd_debug_moe_route(zt, torch.from_numpy(Wr).cuda(), K)
    ids = g["ids"].cpu().numpy()
    logits = g["logits"].cpu().numpy()
    for b in range(4):
        assert logits[b, 3] == logits[b, 65]
        ref, _ = oracle.router_topk(logits[b].astype(np.float64), K)   # the same fp32 logits
        np.testing.assert_array_equal(ids[b], ref)
        assert list(ids[b]).index(3) < list(ids[b]).index(65)
