"""Parity of the individual steps (through the C ABI) against the oracle:
routing, sorting and MX quantisation bit-exact; the gate dot within its
floating-point error bound; the specified sigmoid bitwise."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import inputs

pytestmark = pytest.mark.gpu


def _m():
    import routed_shared_experts_amd as m
    return m


def _route_gpu(logits, topk, **kw):
    m = _m()
    T, E = logits.shape
    n_pseudo = kw.get("n_pseudo", 0)
    ids = torch.empty((T, topk + n_pseudo), dtype=torch.int32, device=logits.device)
    w = torch.empty((T, topk + n_pseudo), dtype=torch.float32, device=logits.device)
    score = m.MOE_SCORE_SIGMOID if kw.pop("score", "softmax") == "sigmoid" else m.MOE_SCORE_SOFTMAX
    m.moe_route(logits, ids, w, topk=topk, score=score, **kw)
    torch.cuda.synchronize()
    return ids.cpu().numpy(), w.cpu().numpy()


def test_spec_sigmoid_bitwise_host_equals_device(gpu):
    """sigmoid through shared_gate_dot with H = 4, x = (v, 0, 0, 0), g = e0:
    the dot is exactly v, so the output is the device's specified sigmoid."""
    m = _m()
    step = 97
    pats = np.arange(0, 0x42A00001, step, dtype=np.uint32)          # |v| <= 80 (all exponents)
    pats = np.concatenate([pats, pats | np.uint32(0x80000000),
                           np.array([0x42A00000, 0x42C80000, 0xC2C80000, 0x7F000000, 0xFF000000], np.uint32)])
    v = pats.view(np.float32)
    for lo in range(0, v.size, 1 << 22):
        chunk = v[lo:lo + (1 << 22)]
        x = np.zeros((chunk.size, 4), np.float32)
        x[:, 0] = chunk
        xt = torch.from_numpy(x).to(gpu)
        g = torch.tensor([1.0, 0.0, 0.0, 0.0], device=gpu)
        out = torch.empty(chunk.size, dtype=torch.float32, device=gpu)
        m.shared_gate_dot(xt, g, out, apply_sigmoid=True)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        ref = oracle.spec_sigmoid(chunk)
        bad = np.nonzero(got.view(np.uint32) != ref.view(np.uint32))[0]
        assert bad.size == 0, [(float(chunk[i]), float(got[i]), float(ref[i])) for i in bad[:5]]


@pytest.mark.parametrize("name", workloads.CONFIG_ORDER)
def test_route_bit_exact_on_workloads(gpu, name):
    cfg = workloads.CONFIGS[name]
    logits = inputs(cfg, gpu)["logits"]
    bias = inputs(cfg, gpu)["bias"]
    kw = dict(score=cfg.score, bias=bias, n_group=cfg.n_group, topk_group=cfg.topk_group,
              group_score_topk=cfg.group_score_topk, renormalize=cfg.renormalize,
              routed_scaling_factor=cfg.routed_scaling_factor)
    ids, w = _route_gpu(logits, cfg.topk, **kw)
    rid, rw = oracle.route(logits.cpu().numpy(), topk=cfg.topk, score=cfg.score,
                           bias=None if bias is None else bias.cpu().numpy(), n_group=cfg.n_group,
                           topk_group=cfg.topk_group, group_score_topk=cfg.group_score_topk,
                           renormalize=cfg.renormalize, routed_scaling_factor=cfg.routed_scaling_factor)
    assert np.array_equal(ids, rid)
    assert np.abs(w - rw).max() <= 1e-6 * cfg.routed_scaling_factor
    load = workloads.realised_load(ids, cfg.E)
    print(f"{name}: realised load {load}")


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_route_ties_equal_logits_and_pseudo_slots(gpu, score):
    rng = np.random.default_rng(12)
    tie = rng.integers(-1, 2, (300, 64)).astype(np.float32)
    ids, w = _route_gpu(torch.from_numpy(tie).to(gpu), 8, score=score)
    rid, rw = oracle.route(tie, topk=8, score=score)
    assert np.array_equal(ids, rid)
    assert np.abs(w - rw).max() <= 1e-6
    eq = torch.zeros((5, 128), device=gpu)
    gamma = torch.linspace(0.1, 0.5, 5, device=gpu)
    ids, w = _route_gpu(eq, 8, score=score, routed_scaling_factor=2.5, n_pseudo=3, gamma=gamma)
    assert np.array_equal(ids[:, :8], np.tile(np.arange(8), (5, 1)))
    assert np.all(w[:, :8] == np.float32(0.3125))
    assert np.array_equal(ids[:, 8:], np.tile([128, 129, 130], (5, 1)))
    assert np.array_equal(w[:, 8:], np.repeat(gamma.cpu().numpy()[:, None], 3, 1))


def test_route_grouped_with_ties_and_k_equals_e(gpu):
    rng = np.random.default_rng(13)
    lg = rng.integers(-2, 3, (257, 256)).astype(np.float32)
    bias = (rng.integers(-1, 2, 256) * 0.125).astype(np.float32)
    for gk, gtop in [(4, 2), (3, 1), (8, 2)]:
        ids, w = _route_gpu(torch.from_numpy(lg).to(gpu), 8, score="sigmoid", bias=torch.from_numpy(bias).to(gpu),
                            n_group=8, topk_group=gk, group_score_topk=gtop)
        rid, rw = oracle.route(lg, topk=8, score="sigmoid", bias=bias, n_group=8, topk_group=gk,
                               group_score_topk=gtop)
        assert np.array_equal(ids, rid)
        assert np.abs(w - rw).max() <= 1e-6
    lg = rng.normal(0, 1, (33, 4)).astype(np.float32)
    ids, w = _route_gpu(torch.from_numpy(lg).to(gpu), 4, routed_scaling_factor=1.5)
    rid, rw = oracle.route(lg, topk=4, routed_scaling_factor=1.5)
    assert np.array_equal(ids, rid) and np.abs(w - rw).max() <= 1e-6
    ids, w = _route_gpu(torch.from_numpy(lg).to(gpu), 2, renormalize=False)
    rid, rw = oracle.route(lg, topk=2, renormalize=False)
    assert np.array_equal(ids, rid) and np.abs(w - rw).max() <= 1e-6


@pytest.mark.parametrize("renormalize", [True, False])
def test_route_softmax_with_groups(gpu, renormalize):
    """Softmax scores with grouped top-k (group score: the largest one or the
    sum of the two largest logits of the group), several group sizes,
    against the oracle bit-exact."""
    rng = np.random.default_rng(14)
    lg = rng.normal(0, 1.5, (300, 64)).astype(np.float32)
    lg[::5] = np.round(lg[::5])  # tie-heavy rows
    lg_t = torch.from_numpy(lg).to(gpu)
    for ng, gk, gtop in [(8, 3, 2), (8, 4, 1), (4, 2, 2), (16, 5, 2)]:
        ids, w = _route_gpu(lg_t, 6, score="softmax", n_group=ng, topk_group=gk, group_score_topk=gtop,
                            renormalize=renormalize, routed_scaling_factor=1.75)
        rid, rw = oracle.route(lg, topk=6, score="softmax", n_group=ng, topk_group=gk, group_score_topk=gtop,
                               renormalize=renormalize, routed_scaling_factor=1.75)
        assert np.array_equal(ids, rid), (ng, gk, gtop)
        assert np.abs(w - rw).max() <= 2e-6


@pytest.mark.parametrize("E", [320, 512])
def test_route_at_the_expert_and_slot_limits(gpu, E):
    """E up to 512 routed experts (eight per lane) and k + pseudo slots up to
    64, plain and grouped, against the oracle bit-exact."""
    rng = np.random.default_rng(E)
    lg = rng.normal(0, 1, (97, E)).astype(np.float32)
    lg[::7] = np.round(lg[::7])  # some tie-heavy rows
    lg_t = torch.from_numpy(lg).to(gpu)
    ids, w = _route_gpu(lg_t, 48, n_pseudo=16, gamma=torch.full((97,), 0.25, device=gpu))
    rid, rw = oracle.route(lg, topk=48)
    assert np.array_equal(ids[:, :48], rid) and np.abs(w[:, :48] - rw).max() <= 1e-6
    assert np.array_equal(ids[:, 48:], np.tile(np.arange(E, E + 16), (97, 1)))
    bias = (rng.integers(-2, 3, E) * 0.0625).astype(np.float32)
    ids, w = _route_gpu(lg_t, 8, score="sigmoid", bias=torch.from_numpy(bias).to(gpu), n_group=32, topk_group=4)
    rid, rw = oracle.route(lg, topk=8, score="sigmoid", bias=bias, n_group=32, topk_group=4)
    assert np.array_equal(ids, rid) and np.abs(w - rw).max() <= 1e-6


def _sort_gpu(ids_np, n_experts, block_m, dev, zero=None, scratch=True):
    m = _m()
    T, k = ids_np.shape
    cap = m.moe_sort_capacity(T, k, n_experts, block_m)
    sb = m.moe_sort_scratch_bytes(T, k, n_experts)
    scr = torch.empty(max(sb, 4), dtype=torch.uint8, device=dev) if (scratch and sb) else None
    ids = torch.from_numpy(ids_np.astype(np.int32)).to(dev)
    srt = torch.full((cap,), -7, dtype=torch.int32, device=dev)
    bexp = torch.full((cap // block_m,), -7, dtype=torch.int32, device=dev)
    counts = torch.empty(n_experts, dtype=torch.int32, device=dev)
    offs = torch.empty(n_experts + 1, dtype=torch.int32, device=dev)
    nb = torch.empty(1, dtype=torch.int32, device=dev)
    m.moe_sort_tokens(ids, n_experts, block_m, cap, srt, bexp, counts, offs, nb, scratch=scr, zero=zero)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (srt, bexp, counts, offs, nb)]


@pytest.mark.parametrize("scratch", [True, False])
@pytest.mark.parametrize("block_m", [16, 32, 64, 128])
@pytest.mark.parametrize("shape", [(1, 1, 1), (5, 2, 8), (32, 9, 65), (4096, 12, 68), (8192, 9, 257),
                                   (1000, 9, 130)])
def test_sort_bit_exact(gpu, block_m, shape, scratch):
    T, k, E = shape
    rng = np.random.default_rng(T * 31 + k)
    # distinct experts per token with a skewed (Zipf-like) load and some empty experts
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    p[::7] = 0 if E > 7 else p[::7]
    p /= p.sum()
    ids = np.stack([rng.choice(E, size=k, replace=False, p=p) if k <= (p > 0).sum() else rng.permutation(E)[:k]
                    for _ in range(T)])
    srt, bexp, counts, offs, nb = _sort_gpu(ids, E, block_m, gpu, scratch=scratch)
    r = oracle.sort_tokens(ids, E, block_m)
    n = r["offsets"][-1]
    assert nb[0] == r["num_blocks"]
    assert np.array_equal(counts, r["counts"]) and np.array_equal(offs, r["offsets"])
    assert np.array_equal(srt[:n], r["sorted_pair_ids"])
    assert np.all(srt[n:] == T * k)
    assert np.array_equal(bexp[:nb[0]], r["block_expert"]) and np.all(bexp[nb[0]:] == -1)


def test_sort_clears_the_zero_region(gpu):
    ids = np.arange(8, dtype=np.int32).reshape(4, 2)
    z = torch.full((1 << 20,), 3.0, device=gpu)
    _sort_gpu(ids, 8, 16, gpu, zero=z)
    assert torch.count_nonzero(z).item() == 0


@pytest.mark.parametrize("H", [32, 1024, 2048, 4096, 65536, 131072])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gate_dot_k_sweep(gpu, H, dtype):
    m = _m()
    T = 3
    g0 = torch.Generator(device="cpu").manual_seed(H)
    x = torch.randn((T, H), generator=g0).to(dtype)
    g = (torch.randn(H, generator=g0) * 0.02).to(dtype)
    xd, gd = x.to(gpu), g.to(gpu)
    x64, g64 = x.double().numpy(), g.double().numpy()
    dot = x64 @ g64
    K = H
    u = 2.0 ** -24
    bound = K * u / (1 - K * u) * (np.abs(x64) @ np.abs(g64))
    out = torch.empty(T, device=gpu)
    m.shared_gate_dot(xd, gd, out, apply_sigmoid=False)
    torch.cuda.synchronize()
    assert np.all(np.abs(out.cpu().numpy() - dot) <= bound)
    m.shared_gate_dot(xd, gd, out, apply_sigmoid=True)
    torch.cuda.synchronize()
    sig = 1 / (1 + np.exp(-dot))
    # sigmoid' <= 1/4, plus the specified sigmoid's own 3 ulp
    assert np.all(np.abs(out.cpu().numpy() - sig) <= bound / 4 + 3 * 2.0 ** -24)


@pytest.mark.parametrize("T,H", [(1, 32), (7, 96), (512, 4096)])
def test_mx_quant_bit_exact(gpu, T, H):
    m = _m()
    g0 = torch.Generator(device="cpu").manual_seed(T * H)
    x = (torch.randn((T, H), generator=g0) * torch.exp2(torch.randint(-10, 10, (T, 1), generator=g0).float()))
    x[0, :32] = 0.0
    if H >= 64:
        x[0, 32] = 500.0 * 2 ** -4
    xb = x.to(torch.bfloat16)
    codes = torch.empty((T, H), dtype=torch.uint8, device=gpu)
    scales = torch.empty((T, H // 32), dtype=torch.uint8, device=gpu)
    m.moe_quant_mx(xb.to(gpu), codes, scales)
    torch.cuda.synchronize()
    rs, rq = oracle.mx_quantize(xb.float().numpy())
    assert np.array_equal(scales.cpu().numpy(), rs)
    assert np.array_equal(codes.cpu().numpy(), rq)


def _tiled_bytes(b, rows, row_bytes):
    """The tiled layout of a row-major byte matrix, from its definition: tile
    (row block, K tile) of 2048 bytes; chunk c = 4h + g of tile row r at
    h * 1024 + (16 g + r) * 16."""
    nkt = row_bytes // 128
    t = b.reshape(rows // 16, 16, nkt, 2, 4, 16)          # [rb, r, kt, h, g, byte]
    return t.transpose(0, 2, 3, 4, 1, 5).reshape(-1)       # [rb, kt, h, g, r, byte]


@pytest.mark.parametrize("rows,cols,dtype", [(16, 64, torch.bfloat16), (48, 384, torch.bfloat16),
                                             (32, 256, torch.float32), (64, 640, torch.uint8)])
def test_pack_weights_bit_exact(gpu, rows, cols, dtype):
    m = _m()
    g = torch.Generator().manual_seed(rows * 1000 + cols)
    raw = torch.randint(0, 256, (rows, cols * torch.empty((), dtype=dtype).element_size()), dtype=torch.uint8,
                        generator=g)
    src = raw.view(dtype).to(gpu)
    dst = m.moe_pack_weights(src)
    torch.cuda.synchronize()
    got = dst.view(torch.uint8).cpu().numpy().reshape(-1)
    exp = _tiled_bytes(raw.numpy(), rows, raw.shape[1])
    assert np.array_equal(got, exp)


@pytest.mark.parametrize("rows,sb", [(16, 4), (48, 64), (32, 12)])
def test_pack_mx_scales_bit_exact(gpu, rows, sb):
    m = _m()
    g = torch.Generator().manual_seed(rows + sb)
    raw = torch.randint(0, 256, (rows, sb), dtype=torch.uint8, generator=g)
    dst = m.moe_pack_mx_scales(raw.to(gpu))
    torch.cuda.synchronize()
    t = raw.numpy().reshape(rows // 16, 16, sb // 4, 4)    # [rb, r, kt, q]
    exp = t.transpose(0, 2, 3, 1).reshape(-1)              # [rb, kt, q, r]
    assert np.array_equal(dst.cpu().numpy().reshape(-1), exp)
