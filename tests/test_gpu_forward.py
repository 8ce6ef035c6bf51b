"""Parity of the fused layer forward (moe_forward through the C ABI) against
the oracle, in both shared-expert modes: small shapes compared on every
output (several tiles, ragged tails, masked pseudo-expert chunks), the five
workloads at full size on sampled tokens, edge cases, and the identities the
method must keep on the GPU."""

import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import TOL, inputs, run_forward, assert_close, compare

pytestmark = pytest.mark.gpu

LC = workloads.LayerConfig

SMALL = {
    # f32: pseudo chunks of 64 over I_s = 96 -> the second chunk is masked to 32 columns
    "small_f32": LC("small_f32", T=37, H=128, E=8, I=64, I_s=96, topk=3, fmt="f32", logits="iid"),
    # bf16: ragged T, I_s = 192 over I = 128 -> masked second chunk
    "small_bf16": LC("small_bf16", T=100, H=256, E=8, I=128, I_s=192, topk=2, fmt="bf16", logits="iid"),
    "small_mxfp8": LC("small_mxfp8", T=70, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4,
                      topk_group=2, routed_scaling_factor=2.5, fmt="mxfp8", gated=False, bias_std=0.1),
    "small_a8w8": LC("small_a8w8", T=90, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid", n_group=4,
                     topk_group=2, fmt="a8w8", gated=False, logits="zipf", zipf_s=1.2),
    # per-expert biases on both stages, GELU or SiLU (general epilogue of every kernel family)
    "small_bias_gelu_bf16": LC("small_bias_gelu_bf16", T=90, H=256, E=16, I=128, I_s=256, topk=4, fmt="bf16",
                               bias13_std=0.2, bias2_std=0.01, activation="gelu_tanh"),
    "small_bias_mxfp8": LC("small_bias_mxfp8", T=70, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid",
                           n_group=4, topk_group=2, fmt="mxfp8", gated=False, bias_std=0.1, bias13_std=0.3,
                           bias2_std=0.03),
    "small_bias_gelu_a8w8": LC("small_bias_gelu_a8w8", T=90, H=512, E=16, I=256, I_s=256, topk=4, score="sigmoid",
                               n_group=4, topk_group=2, fmt="a8w8", gated=False, bias13_std=0.3, bias2_std=0.04,
                               activation="gelu_tanh"),
    "small_bias_gelu_mxfp4": LC("small_bias_gelu_mxfp4", T=70, H=512, E=16, I=256, I_s=512, topk=4,
                                score="sigmoid", n_group=4, topk_group=2, fmt="mxfp4", gated=False, bias_std=0.1,
                                bias13_std=0.3, bias2_std=0.03, activation="gelu_tanh"),
    "tiny_bias_gelu_f32": LC("tiny_bias_gelu_f32", T=8, H=64, E=4, I=32, I_s=64, topk=2, fmt="f32",
                             logits="linear", bias13_std=0.1, bias2_std=0.001, activation="gelu_tanh"),
    "decode_bias_gelu_bf16": LC("decode_bias_gelu_bf16", T=24, H=512, E=16, I=256, I_s=256, topk=4, fmt="bf16",
                                bias13_std=0.2, bias2_std=0.01, activation="gelu_tanh"),
    # softmax scores with grouped top-k (routing in its own launch)
    "small_softmax_groups": LC("small_softmax_groups", T=80, H=256, E=32, I=128, I_s=128, topk=6,
                               score="softmax", n_group=8, topk_group=3, fmt="bf16"),
    # MXFP4 weights, MX-fp8 activations; I_s = 512 over I = 256: two pseudo chunks
    "small_mxfp4": LC("small_mxfp4", T=70, H=512, E=16, I=256, I_s=512, topk=4, score="sigmoid", n_group=4,
                      topk_group=2, routed_scaling_factor=2.5, fmt="mxfp4", gated=False, bias_std=0.1),
    # H = 2112: 33 stage-2 column tiles, several tile groups per XCD queue, so
    # the bf16 reduction counts arrivals per (token, tile) instead of per group
    "wide_bf16": LC("wide_bf16", T=150, H=2112, E=8, I=128, I_s=128, topk=2, fmt="bf16", logits="zipf",
                    zipf_s=1.1),
}


@pytest.mark.parametrize("block_m", [0, 16, 32, 128, 256])
@pytest.mark.parametrize("mode", ["pseudo", "aux"])
@pytest.mark.parametrize("name", list(SMALL))
def test_small_layers_all_outputs(gpu, name, mode, block_m):
    """block_m = 16 takes the one-wave register-streamed GEMM kernels; 32-256
    take the tiled kernels (weights in registers, token rows through LDS) for
    bf16 / MX / a8w8 and the LDS-staged fallback for f32 (up to 128); 0 is the
    automatic choice."""
    cfg = SMALL[name]
    if cfg.fmt in ("f32", "mxfp4") and block_m == 256:
        pytest.skip("256-row blocks: the LDS-staged kernels, which take neither f32 nor e2m1 weights")
    if mode == "pseudo" and cfg.fmt == "a8w8" and cfg.I_s > cfg.I:
        pytest.skip("per-row fp8 intermediate needs a single pseudo chunk")
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode, block_m=block_m)
    rel, floor, r = assert_close(cfg, out, inp)
    print(f"{name}/{mode}/bm{block_m}: max|err|/rms={rel:.3e} floor={floor:.3e}")
    if (cfg.bias13_std or cfg.bias2_std) and mode == "pseudo" and block_m == 0:
        # the check has teeth: dropping either bias moves the output by much
        # more than the tolerance
        host = workloads.to_host(inp)
        rms = np.sqrt((r["y"] ** 2).mean())
        for drop in (("b13", "bs13"), ("b2", "bs2")):
            y0 = oracle.moe_layer(dict(host, **{k: None for k in drop}), cfg)["y"]
            assert np.abs(y0 - r["y"]).max() / rms > 5 * TOL[cfg.fmt], drop


@pytest.mark.parametrize("block_m", [16, 32, 64, 128, 256])
def test_block_m_variants(gpu, block_m):
    cfg = SMALL["small_bf16"]
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, "pseudo", block_m=block_m)
    assert_close(cfg, out, inp)


@pytest.mark.parametrize("T", [64, 65])
@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_decode_blocks_with_many_tokens_per_expert(gpu, T, mode):
    """16-row blocks at T <= 64 find their pairs by scanning the routing ids
    (block = sub-block * E' + expert, no sort launch); heavily skewed routing
    gives an expert nearly every token, i.e. several sub-blocks, and so do the
    two pseudo chunks.  T = 65 takes the sorted path with the same blocks."""
    cfg = LC(f"skew{T}", T=T, H=256, E=8, I=128, I_s=256, topk=2, fmt="bf16", logits="zipf", zipf_s=2.0)
    inp = inputs(cfg, gpu)
    ids = workloads.to_host(inp)["logits"].argmax(axis=1)
    assert np.bincount(ids, minlength=cfg.E).max() > 32  # the top expert spans three or more sub-blocks
    out, _ = run_forward(cfg, inp, mode, block_m=16)
    assert_close(cfg, out, inp)


@pytest.mark.parametrize("E", [64, 6, 96])
@pytest.mark.parametrize("T", [32, 64])
def test_decode_routing_inside_stage1_with_tied_logits(gpu, T, E):
    """At decode sizes (16-row self-sorted blocks, softmax, E <= 64 and a
    multiple of 4, pseudo mode) the stage-1 launch routes the tokens itself and
    each GEMM wave selects its expert's tokens with the routing's rule; logits
    in {-1, 0, 1} make most selections ties (lower index first).  E = 6, E = 96
    and the aux mode take the separate routing launch; all must match the
    oracle."""
    cfg = LC(f"ties{T}_{E}", T=T, H=256, E=E, I=128, I_s=128, topk=min(8, E), fmt="bf16", logits="iid")
    inp = dict(inputs(cfg, gpu))
    rng = np.random.default_rng(T * 100 + E)
    inp["logits"] = torch.from_numpy(rng.integers(-1, 2, (T, E)).astype(np.float32)).to(gpu)
    for mode in ("pseudo", "aux"):
        out, _ = run_forward(cfg, inp, mode, block_m=16)
        rel, _, _ = assert_close(cfg, out, inp)
        print(f"ties T={T} E={E} {mode}: max|err|/rms={rel:.3e}")


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_tiny_f32_workload(gpu, mode):
    cfg = workloads.CONFIGS["tiny_f32"]
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode)
    rel, floor, _ = assert_close(cfg, out, inp)
    print(f"tiny_f32/{mode}: max|err|/rms={rel:.3e}")


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_decode_bf16_workload_full(gpu, mode):
    cfg = workloads.CONFIGS["decode_bf16"]
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode)
    rel, floor, _ = assert_close(cfg, out, inp)
    print(f"decode_bf16/{mode}: max|err|/rms={rel:.3e} floor={floor:.3e}")


def _sample(T, n, seed):
    rng = np.random.default_rng(seed)
    s = np.sort(rng.choice(T, size=min(n, T), replace=False))
    return np.unique(np.concatenate([[0, T - 1], s]))


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_prefill_bf16_workload_sampled(gpu, mode):
    cfg = workloads.CONFIGS["prefill_bf16"]
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode)
    rel, floor, _ = assert_close(cfg, out, inp, tokens=_sample(cfg.T, 256, 1))
    print(f"prefill_bf16/{mode}: max|err|/rms={rel:.3e} floor={floor:.3e}")


@pytest.mark.parametrize("block_m", [0, 16])
@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_mxfp8_workload_sampled(gpu, mode, block_m):
    cfg = workloads.CONFIGS["mxfp8"]
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode, block_m=block_m)
    rel, floor, _ = assert_close(cfg, out, inp, tokens=_sample(cfg.T, 24, 2), lazy=True)
    print(f"mxfp8/{mode}: max|err|/rms={rel:.3e} floor={floor:.3e}")


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_a8w8_large_workload_sampled(gpu, mode):
    cfg = workloads.CONFIGS["a8w8_large"]
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode)
    rel, floor, _ = assert_close(cfg, out, inp, tokens=_sample(cfg.T, 6, 3), lazy=True)
    print(f"a8w8_large/{mode}: max|err|/rms={rel:.3e} floor={floor:.3e}")


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_empty_batch(gpu, mode):
    """T = 0 through the binding: the forward succeeds, launches nothing and
    leaves the stream usable."""
    cfg = SMALL["small_bf16"]
    inp = inputs(cfg, gpu)
    empty = dict(inp, x=inp["x"][:0], logits=inp["logits"][:0])
    out, _ = run_forward(cfg.replace(T=0), empty, mode)
    assert tuple(out.shape) == (0, cfg.H)
    out2, _ = run_forward(cfg, inp, mode)  # a full call right after
    assert_close(cfg, out2, inp)


@pytest.mark.parametrize("mode", ["pseudo", "aux"])
def test_512_experts(gpu, mode):
    """The largest expert count (eight logits per routing lane, 513-514
    sort buckets with the pseudo chunks), most experts with one or two pairs."""
    cfg = LC("e512", T=300, H=128, E=512, I=64, I_s=128, topk=8, fmt="bf16", logits="iid")
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, mode)
    assert_close(cfg, out, inp)


def test_single_token_and_single_expert(gpu):
    cfg = LC("t1", T=1, H=128, E=1, I=64, I_s=64, topk=1, fmt="bf16", logits="iid")
    inp = inputs(cfg, gpu)
    for mode in ("pseudo", "aux"):
        out, _ = run_forward(cfg, inp, mode)
        assert_close(cfg, out, inp)


def test_k_equals_e_and_no_shared(gpu):
    cfg = LC("kE", T=40, H=128, E=4, I=64, I_s=0, topk=4, fmt="bf16", logits="iid", gated=False)
    inp = inputs(cfg, gpu)
    out, _ = run_forward(cfg, inp, "none")
    assert_close(cfg, out, inp)


def test_shared_only_bit_identical_across_modes(gpu):
    """routed_scaling_factor = 0 zeroes every routed weight, so the output is
    gamma * S(x) whichever way the shared expert runs (one pseudo chunk)."""
    cfg = workloads.CONFIGS["decode_bf16"].replace(routed_scaling_factor=0.0)
    inp = inputs(workloads.CONFIGS["decode_bf16"], gpu)
    a, _ = run_forward(cfg, inp, "pseudo")
    a = a.clone()
    b, _ = run_forward(cfg, inp, "aux")
    assert torch.equal(a, b)
    assert_close(cfg, b, inp)


def test_routed_scale_fold_on_gpu(gpu):
    """s = 2 (power of two): routed part doubles exactly in fp32; compare the
    fp32-output layer against 2 x the s = 1 routed-only output."""
    base = SMALL["small_f32"].replace(I_s=0, gated=False)
    inp = inputs(base, gpu)
    y1, _ = run_forward(base, inp, "none")
    y1 = y1.clone()
    y2, _ = run_forward(base.replace(routed_scaling_factor=2.0), inp, "none")
    assert torch.allclose(y2, 2 * y1, rtol=0, atol=4e-6 * float(y1.abs().max()))


def test_repeated_calls_are_deterministic_in_ids(gpu):
    cfg = SMALL["small_bf16"]
    inp = inputs(cfg, gpu)
    a, layer = run_forward(cfg, inp, "pseudo")
    a = a.clone()
    for _ in range(3):
        b = layer.forward()
    torch.cuda.synchronize()
    rel = (a.float() - b.float()).abs().max().item() / a.float().pow(2).mean().sqrt().item()
    assert rel <= 2 * TOL["bf16"]
