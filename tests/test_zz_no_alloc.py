"""The no-allocation fused call (w4a16_fused_moe_noalloc): intermediates in the library's static device scratch,
results bit for bit those of w4a16_fused_moe with a caller workspace, on consecutive calls that shrink (the
scratch keeps the previous call's contents), with split-K decode plans (their counters are cleared before use),
and a call too large for the scratch refused before anything is launched."""
import numpy as np
import pytest
import torch

import synth
import weight_only_int4_amd as w4
from weight_only_int4_amd import lib as L
from gpu_util import bits, f32, i32, u8, u16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    w4.load()


def _layer(seed, T, E, k, H, I):
    rng = np.random.default_rng(seed)
    x = synth.activations(rng, T, H)
    c13, s13 = synth.codes(rng, E, 2 * I, H), synth.scales(rng, E, 2 * I, H)
    c2, s2 = synth.codes(rng, E, H, I), synth.scales(rng, E, H, I)
    ids = synth.uniform_topk(rng, T, E, k)
    ids[0, :] = -1          # a token without a local route: zero row
    ids[T - 1, 0] = E + 1   # a non-local route
    tw = rng.uniform(0.1, 1.0, (T, k)).astype(np.float32)
    w13 = w4.pack_weights(u8(c13), u16(s13))
    w2 = w4.pack_weights(u8(c2), u16(s2))
    return u16(x), i32(ids), f32(tw), w13, w2


# (T, E, k, H, I): a prefill step (tile list; the planner runs its two GEMMs in one launch), then smaller decode
# steps, one of whose plans split K
CALLS = [(600, 8, 2, 512, 256), (64, 32, 4, 512, 256), (2, 48, 8, 512, 2048), (1, 8, 2, 256, 128)]


def test_noalloc_equals_workspace_call_on_consecutive_calls():
    plans_seen, one_launch = set(), False
    for n, (T, E, k, H, I) in enumerate(CALLS):
        print("noalloc call %d: T=%d E=%d k=%d H=%d I=%d" % (n, T, E, k, H, I), flush=True)
        x, ids, tw, w13, w2 = _layer(500 + n, T, E, k, H, I)
        p13, p2 = w4.fused_moe_plans(T, k, w13, w2)
        plans_seen.add((p13.kernel, p13.k_split > 1 or p2.k_split > 1))
        one_launch |= p13.kernel == w4.KERNEL_PREFILL and bool(p13.flags & L.PLAN_ONE_LAUNCH)
        assert w4.fused_moe_workspace_bytes(T, k, w13, w2) <= L.NOALLOC_SCRATCH_BYTES
        ref = bits(w4.fused_moe(x, ids, tw, w13, w2))
        out = torch.full((T, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
        L.fused_moe_noalloc(x, ids, tw, w13, w2, out)
        got = bits(out)
        assert np.all(got[0] == 0)
        assert np.array_equal(got, ref), "call %d differs in %d values" % (n, int((got != ref).sum()))
        # the same call again on the scratch this call just used
        out.fill_(0)
        L.fused_moe_noalloc(x, ids, tw, w13, w2, out)
        assert np.array_equal(bits(out), ref), "call %d repeated differs" % n
    # the sequence covered a prefill plan and a decode plan that splits K
    assert (w4.KERNEL_PREFILL, False) in plans_seen and (w4.KERNEL_DECODE, True) in plans_seen
    assert one_launch, "no prefill step ran gate_up and down in one launch"


def test_noalloc_refuses_a_step_beyond_the_scratch():
    T, E, k, H, I = 4096, 16, 8, 2048, 256  # y (BF16) alone is T*k*H*2 = 128 MiB
    x, ids, tw, w13, w2 = _layer(7, T, E, k, H, I)
    assert w4.fused_moe_workspace_bytes(T, k, w13, w2) > L.NOALLOC_SCRATCH_BYTES
    out = torch.full((T, H), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    with pytest.raises(w4.W4A16Error) as ei:
        L.fused_moe_noalloc(x, ids, tw, w13, w2, out)
    assert ei.value.code == -4 and "static scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert np.all(bits(out) == 0xFFFF), "a refused call must launch nothing"
