"""Parity at the full workload sizes, in the launch configurations the benchmark uses, on sampled rows.

Each test runs the HIP path on the whole workload and checks a sample of output rows against the oracle
computed row by row: for the grouped GEMMs, up to three routes of every active expert (its first, middle and
last route, so tile edges are covered) against the oracle's binary64 accumulators, to the 5e-3 per-expert
bar; for the fused MLP, a sample of tokens against the oracle's binary32 accumulators before the final
rounding, to the fused bar (error within 5e-3 of the token's combine scale, see gpu_util.check_fused).  Rows of non-local routes must keep their poison bytes.
"""
import numpy as np
import pytest
import torch

import synth
import weight_only_int4_amd as w4
from gpu_util import POISON, bits, check_act, check_fused, check_gemm, f32, i32, poison_bf16, u16

pytestmark = pytest.mark.gpu



def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.load()


def sample_routes(ids, E, per_expert=3):
    flat = ids.reshape(-1)
    rows = []
    for e in np.unique(flat[(flat >= 0) & (flat < E)]):
        r = np.nonzero(flat == e)[0]
        rows.extend(sorted({int(r[0]), int(r[len(r) // 2]), int(r[-1])})[:per_expert])
    bad = np.nonzero((flat < 0) | (flat >= E))[0]
    rows.extend(bad[:8].tolist())
    return np.array(sorted(rows), np.int32)


def run_case(orc, label, E, N, K, ids, a_row_div, rows_A, codes, scales, expected_rows=0.0):
    T = ids.shape[0]
    k = ids.shape[1]
    rng = np.random.default_rng(N + K + T)
    A = synth.activations(rng, rows_A, K)
    w = w4.pack_weights(torch.from_numpy(codes).cuda(), u16(scales))
    plan = w4.plan_select(T, k, E, N, K, expected_rows)
    _say("%s: %r" % (label, plan))
    route = w4.route_prep(i32(ids), E, plan.block_m)
    out = poison_bf16(route["R"], N)
    w4.grouped_gemm(u16(A), a_row_div, w, route, plan, out=out)
    got = bits(out)
    rows = sample_routes(ids, E)
    acc, _ = orc.grouped_gemm(A, a_row_div, codes, scales, ids, acc64=True, rows=rows)
    worst = check_gemm(got, acc, ids, E, rows=rows, label=label)
    _say("  %d sampled rows, worst ratio %.2e" % (len(rows), worst))


def run_silu_case(orc, label, E, N, K, ids, a_row_div, rows_A, codes, scales, expected_rows=0.0):
    """gate_up with the SiLU*mul epilogue on sampled routes, against the oracle's binary64 gate/up values."""
    T, k = ids.shape
    rng = np.random.default_rng(N + K + T + 1)
    A = synth.activations(rng, rows_A, K)
    w = w4.pack_weights(torch.from_numpy(codes).cuda(), u16(scales))
    plan = w4.plan_select(T, k, E, N, K, expected_rows)
    if plan.n_blocks < 2:
        plan.n_blocks = 2
    _say("%s: %r" % (label, plan))
    route = w4.route_prep(i32(ids), E, plan.block_m)
    h = poison_bf16(route["R"], N // 2)
    w4.grouped_gemm_silu(u16(A), a_row_div, w, route, plan, out=h)
    got = bits(h)
    rows = sample_routes(ids, E)
    gu, _ = orc.grouped_gemm(A, a_row_div, codes, scales, ids, acc64=True, rows=rows)
    worst = check_act(got, gu, ids, E, rows=rows, label=label)
    _say("  %d sampled rows, worst error / bound %.2f" % (len(rows), worst))


@pytest.fixture(scope="module")
def qwen3_weights():
    c13, s13 = synth.expert_weights(2, 128, 1536, 2048, salt=1)
    c2, s2 = synth.expert_weights(2, 128, 2048, 768, salt=2)
    return c13, s13, c2, s2


@pytest.mark.parametrize("T", [1, 8, 64, 512])
def test_qwen3_gate_up_and_down(orc, qwen3_weights, T):
    c13, s13, c2, s2 = qwen3_weights
    ids = synth.qwen3_routes(T)
    run_case(orc, "qwen3 T%d gate_up" % T, 128, 1536, 2048, ids, 8, T, c13, s13)
    run_case(orc, "qwen3 T%d down" % T, 128, 2048, 768, ids, 1, T * 8, c2, s2)


def test_qwen3_fused_bench_workload(orc, qwen3_weights):
    """The benchmark's default step: fused expert MLP, Qwen3-30B-A3B-shaped, 64 tokens."""
    c13, s13, c2, s2 = qwen3_weights
    T, k, E = 64, 8, 128
    ids = synth.qwen3_routes(T)
    rng = synth.rng_for(2, 7)
    x = synth.activations(rng, T, 2048)
    tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    tw /= tw.sum(axis=1, keepdims=True)
    w13 = w4.pack_weights(torch.from_numpy(c13).cuda(), u16(s13))
    w2 = w4.pack_weights(torch.from_numpy(c2).cuda(), u16(s2))
    _say("qwen3 fused plans %r" % (w4.fused_moe_plans(T, k, w13, w2),))
    got = bits(w4.fused_moe(u16(x), i32(ids), f32(tw), w13, w2))
    sample = np.arange(0, T, 7)
    _, _, y = orc.fused_moe(x[sample], ids[sample], tw[sample], c13, s13, c2, s2)
    worst, plain = check_fused(got[sample], orc.last_out_acc, y, tw[sample], ids[sample], E, label="qwen3 fused")
    _say("  fused worst %.2e of S_t (%.2e of max|out|) over %d tokens" % (worst, plain, len(sample)))


@pytest.fixture(scope="module")
def kimi_weights():
    return synth.expert_weights(3, 48, 4096, 7168, salt=1)


@pytest.mark.parametrize("T", [1, 2, 4, 8, 16, 32, 64, 128, 256])
def test_kimi_decode_share_gate_up(orc, kimi_weights, T):
    codes, scales = kimi_weights
    ids = synth.kimi_decode_routes(T)
    flat = ids.reshape(-1)
    rows_e = max(float(((flat >= 0) & (flat < 48)).sum()) / 48.0, 1.0 / 48.0)
    run_case(orc, "kimi decode T%d gate_up" % T, 48, 4096, 7168, ids, 8, T, codes, scales, expected_rows=rows_e)


@pytest.mark.parametrize("T", [1, 64])
def test_kimi_decode_share_gate_up_silu(orc, kimi_weights, T):
    codes, scales = kimi_weights
    ids = synth.kimi_decode_routes(T)
    flat = ids.reshape(-1)
    rows_e = max(float(((flat >= 0) & (flat < 48)).sum()) / 48.0, 1.0 / 48.0)
    run_silu_case(orc, "kimi decode T%d gate_up+silu" % T, 48, 4096, 7168, ids, 8, T, codes, scales,
                  expected_rows=rows_e)


def test_kimi_prefill_share_gate_up_silu(orc, kimi_weights):
    codes, scales = kimi_weights
    ids = synth.kimi_prefill_routes(8192)
    flat = ids.reshape(-1)
    rows_e = float(((flat >= 0) & (flat < 48)).sum()) / 48.0
    run_silu_case(orc, "kimi prefill T8192 gate_up+silu", 48, 4096, 7168, ids, 8, 8192, codes, scales,
                  expected_rows=rows_e)


def test_kimi_decode_share_down(orc):
    codes, scales = synth.expert_weights(3, 48, 7168, 2048, salt=2)
    ids = synth.kimi_decode_routes(64)
    flat = ids.reshape(-1)
    rows_e = float(((flat >= 0) & (flat < 48)).sum()) / 48.0
    run_case(orc, "kimi decode T64 down", 48, 7168, 2048, ids, 1, 64 * 8, codes, scales, expected_rows=rows_e)


def test_kimi_prefill_share_gate_up(orc, kimi_weights):
    codes, scales = kimi_weights
    ids = synth.kimi_prefill_routes(8192)
    flat = ids.reshape(-1)
    counts = np.bincount(flat[(flat >= 0) & (flat < 48)], minlength=48)
    assert (counts == 0).sum() >= 4, "the skewed routing leaves experts empty"
    rows_e = counts.sum() / 48.0
    run_case(orc, "kimi prefill T8192 gate_up", 48, 4096, 7168, ids, 8, 8192, codes, scales, expected_rows=rows_e)


@pytest.fixture(scope="module")
def deepseek_weights():
    dev = torch.device("cuda:0")
    E, H, I = 256, 7168, 2048
    c13 = synth.codes_device(5001, E, 2 * I, H, dev)
    s13 = synth.scales_device(5002, E, 2 * I, H, dev)
    w13 = w4.pack_weights(c13, s13.contiguous().view(torch.bfloat16))
    c2 = synth.codes_device(5003, E, H, I, dev)
    s2 = synth.scales_device(5004, E, H, I, dev)
    w2 = w4.pack_weights(c2, s2.contiguous().view(torch.bfloat16))
    torch.cuda.synchronize()
    return dict(c13=c13, s13=s13, c2=c2, s2=s2, w13=w13, w2=w2, E=E, H=H, I=I)


def _deepseek_host_weights(d, used):
    """Codes and scales of the experts ``used`` copied from the device, and the id remap onto them."""
    ue = torch.from_numpy(np.asarray(used)).cuda().long()
    c13 = d["c13"][ue].cpu().numpy()
    s13 = d["s13"][ue].view(torch.int16).cpu().numpy().view(np.uint16)
    c2 = d["c2"][ue].cpu().numpy()
    s2 = d["s2"][ue].view(torch.int16).cpu().numpy().view(np.uint16)
    remap = np.full(d["E"], -1, np.int32)
    remap[np.asarray(used)] = np.arange(len(used), dtype=np.int32)
    return c13, s13, c2, s2, remap


@pytest.mark.parametrize("T", [1, 32, 512, 4096])
def test_deepseek_fused(orc, deepseek_weights, T):
    """The DeepSeek-V3-shaped fused step on up to 64 sampled tokens (every token below 64), against the oracle
    on the experts those tokens use."""
    d = deepseek_weights
    E, H, I = d["E"], d["H"], d["I"]
    ids, tw = synth.deepseek_router(T)
    rng = synth.rng_for(5, 7 + T)
    x = synth.activations(rng, T, H)
    _say("deepseek T%d fused plans %r" % (T, w4.fused_moe_plans(T, 8, d["w13"], d["w2"])))
    got = bits(w4.fused_moe(u16(x), i32(ids), f32(tw), d["w13"], d["w2"]))
    sample = np.unique(np.linspace(0, T - 1, min(T, 64)).astype(int))
    used = np.unique(ids[sample])
    c13, s13, c2, s2, remap = _deepseek_host_weights(d, used)
    _, _, y = orc.fused_moe(x[sample], remap[ids[sample]], tw[sample], c13, s13, c2, s2)
    worst, plain = check_fused(got[sample], orc.last_out_acc, y, tw[sample], remap[ids[sample]], len(used),
                               label="deepseek T%d fused" % T)
    _say("  deepseek T%d fused worst %.2e of S_t (%.2e of max|out|) over %d tokens" % (T, worst, plain, len(sample)))


def test_deepseek_t4096_stages(orc, deepseek_weights):
    """Stage by stage at the benchmark's size and plans (prefill, tile lists): gate_up with SiLU*mul and the
    down projection (binary32 output) on the first, middle and last route of every one of the 256 experts,
    against the oracle's binary64 accumulators."""
    d = deepseek_weights
    E, H, I, T, k = d["E"], d["H"], d["I"], 4096, 8
    ids, _ = synth.deepseek_router(T)
    x = synth.activations(synth.rng_for(5, 7 + T), T, H)
    p13, p2 = w4.fused_moe_plans(T, k, d["w13"], d["w2"])
    _say("deepseek T4096 stage plans %r %r" % (p13, p2))
    assert p13.kernel == w4.KERNEL_PREFILL
    route = w4.route_prep(i32(ids), E, p13.block_m)
    h = poison_bf16(T * k, I)
    w4.grouped_gemm_silu(u16(x), k, d["w13"], route, p13, out=h)
    hin = synth.activations(synth.rng_for(5, 99), T * k, I)
    y = w4.grouped_gemm(u16(hin), 1, d["w2"], route, p2, out_f32=True).cpu().numpy().astype(np.float64)
    got_h = bits(h)
    rows = sample_routes(ids, E)
    assert len(rows) >= 3 * E - 2
    c13, s13, c2, s2, _ = _deepseek_host_weights(d, np.arange(E))
    gu, _ = orc.grouped_gemm(x, k, c13, s13, ids, acc64=True, rows=rows)
    worst = check_act(got_h, gu, ids, E, rows=rows, label="deepseek T4096 gate_up+silu")
    _say("  gate_up+silu: %d sampled routes, worst error / bound %.2f" % (len(rows), worst))
    del gu
    yr, _ = orc.grouped_gemm(hin, 1, c2, s2, ids, acc64=True, rows=rows)
    flat = ids.reshape(-1)
    worst = 0.0
    for e in range(E):
        rr = rows[flat[rows] == e]
        ratio = np.abs(y[rr] - yr[rr]).max() / np.abs(yr[rr]).max()
        worst = max(worst, ratio)
        assert ratio <= 5e-3, "down expert %d ratio %.3g" % (e, ratio)
    _say("  down: %d sampled routes, worst ratio %.2e" % (len(rows), worst))


# ------------------------------------------------------------------ MXFP4 weights at the benchmark's sizes

def _fused_sampled(orc, label, x, ids, tw, w13, w2, host_weights, sample, fmt):
    got = bits(w4.fused_moe(u16(x), i32(ids), f32(tw), w13, w2))
    c13, s13, c2, s2 = host_weights
    _, _, y = orc.fused_moe(x[sample], ids[sample], tw[sample], c13, s13, c2, s2, fmt=fmt)
    worst, plain = check_fused(got[sample], orc.last_out_acc, y, tw[sample], ids[sample], c13.shape[0], label=label)
    _say("  %s worst %.2e of S_t (%.2e of max|out|) over %d tokens" % (label, worst, plain, len(sample)))


def test_qwen3_fused_bench_workload_mxfp4(orc, qwen3_weights):
    """The Qwen3-30B-A3B-shaped 64-token step with MXFP4 weights (E2M1 codes, E8M0 scales per 32 k), drawn as
    the benchmark draws them."""
    c13, _, c2, _ = qwen3_weights
    T, k, E = 64, 8, 128
    s13 = synth.mxfp4_scales(synth.rng_for(2, 201), E, 1536, 2048)
    s2 = synth.mxfp4_scales(synth.rng_for(2, 202), E, 2048, 768)
    ids = synth.qwen3_routes(T)
    rng = synth.rng_for(2, 7)
    x = synth.activations(rng, T, 2048)
    tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    tw /= tw.sum(axis=1, keepdims=True)
    w13 = w4.pack_weights_mxfp4(torch.from_numpy(c13).cuda(), torch.from_numpy(s13).cuda())
    w2 = w4.pack_weights_mxfp4(torch.from_numpy(c2).cuda(), torch.from_numpy(s2).cuda())
    _say("qwen3 mxfp4 fused plans %r" % (w4.fused_moe_plans(T, k, w13, w2),))
    _fused_sampled(orc, "qwen3 T64 mxfp4 fused", x, ids, tw, w13, w2, (c13, s13, c2, s2), np.arange(0, T, 7),
                   "mxfp4")


def test_deepseek_fused_mxfp4_t4096(orc):
    """DeepSeek-V3-shaped 4096-token fused step with MXFP4 weights generated on the device (prefill plans with
    tile lists), on sampled tokens; the oracle gets the experts those tokens use."""
    dev = torch.device("cuda:0")
    E, H, I, T = 256, 7168, 2048, 4096
    c13 = synth.codes_device(5101, E, 2 * I, H, dev)
    s13 = synth.mxfp4_scales_device(5102, E, 2 * I, H, dev)
    c2 = synth.codes_device(5103, E, H, I, dev)
    s2 = synth.mxfp4_scales_device(5104, E, H, I, dev)
    w13 = w4.pack_weights_mxfp4(c13, s13)
    w2 = w4.pack_weights_mxfp4(c2, s2)
    ids, tw = synth.deepseek_router(T)
    x = synth.activations(synth.rng_for(5, 7 + T), T, H)
    _say("deepseek T%d mxfp4 fused plans %r" % (T, w4.fused_moe_plans(T, 8, w13, w2)))
    sample = np.unique(np.linspace(0, T - 1, 5).astype(int))
    used = np.unique(ids[sample])
    remap = np.full(E, -1, np.int32)
    remap[used] = np.arange(used.size, dtype=np.int32)
    ue = torch.from_numpy(used).cuda().long()
    host = tuple(t[ue].cpu().numpy() for t in (c13, s13, c2, s2))
    got = bits(w4.fused_moe(u16(x), i32(ids), f32(tw), w13, w2))
    _, _, y = orc.fused_moe(x[sample], remap[ids[sample]], tw[sample], *host, fmt="mxfp4")
    worst, plain = check_fused(got[sample], orc.last_out_acc, y, tw[sample], remap[ids[sample]], len(used),
                               label="deepseek mxfp4")
    _say("  deepseek T%d mxfp4 fused worst %.2e of S_t (%.2e of max|out|) over %d tokens" % (T, worst, plain,
                                                                                           len(sample)))
    del w13, w2, c13, s13, c2, s2
    torch.cuda.empty_cache()


def test_kimi_decode_share_fused_bench_workload(orc, kimi_weights):
    """The Kimi-K2 share's fused step as the benchmark runs it (256 tokens, about 1/8 of routes local, plans for
    T*k/384 rows per local expert), on sampled tokens with at least one local route."""
    codes13, scales13 = kimi_weights
    c2, s2 = synth.expert_weights(3, 48, 7168, 2048, salt=2)
    T, k, E, G = 256, 8, 48, 384
    ids = synth.kimi_decode_routes(T)
    rng = synth.rng_for(3, 7)
    x = synth.activations(rng, T, 7168)
    tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    tw /= tw.sum(axis=1, keepdims=True)
    w13 = w4.pack_weights(torch.from_numpy(codes13).cuda(), u16(scales13))
    w2 = w4.pack_weights(torch.from_numpy(c2).cuda(), u16(s2))
    plans = w4.fused_moe_plans(T, k, w13, w2, expected_rows_per_expert=T * k / G)
    _say("kimi T%d fused plans %r" % (T, plans))
    got = bits(w4.fused_moe(u16(x), i32(ids), f32(tw), w13, w2, plans=plans))
    local = ((ids >= 0) & (ids < E)).any(axis=1)
    assert np.all(got[~local] == 0), "tokens without a local route must be zero"
    sample = np.nonzero(local)[0][::23][:8]
    _, _, y = orc.fused_moe(x[sample], ids[sample], tw[sample], codes13, scales13, c2, s2)
    worst, plain = check_fused(got[sample], orc.last_out_acc, y, tw[sample], ids[sample], E, label="kimi fused")
    _say("  kimi T%d fused worst %.2e of S_t (%.2e of max|out|) over %d tokens" % (T, worst, plain, len(sample)))
