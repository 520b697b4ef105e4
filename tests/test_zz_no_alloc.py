"""The allocation-free forward (moe_expert_forward_noalloc, the library's
static per-GPU scratch in place of a caller workspace) against
moe_expert_forward with a caller-allocated workspace, through the C ABI: the
same kernels run on the same inputs, so outputs must be bit-identical, on two
calls in a row with the second one smaller (the scratch keeps the first
call's contents).  A layer whose workspace exceeds the scratch is refused on
the host with nothing enqueued."""
import numpy as np
import pytest
import torch

from precision_moe_expert_amd import binding, synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


def _pair(d: gu.DevInputs, T: int, chunk: int):
    """Reference (caller workspace) and no-alloc outputs on the first T tokens."""
    c = d.li.cfg
    layer = binding.make_layer(T, c.H, c.I, c.E, c.k, c.fmt, oft=d.oft is not None)
    x, lg = d.x[:T].contiguous(), d.logits[:T].contiguous()
    ref = binding.expert_forward(layer, x, lg, d.w13, d.w2, d.s13, d.s2, adapter=d.oft, chunk_experts=chunk,
                                 g13=d.g13, g2=d.g2)
    got = binding.expert_forward_noalloc(layer, x, lg, d.w13, d.w2, d.s13, d.s2, adapter=d.oft,
                                         chunk_experts=chunk, g13=d.g13, g2=d.g2)
    torch.cuda.synchronize()
    return ref, got


def test_noalloc_decode_layer_twice():
    """Decode-sized Kimi-K2-shaped INT4 + OFT layer (64 tokens, then 19)."""
    cfg = synth.CONFIGS["c5"]
    d = gu.DevInputs(synth.make_inputs(cfg, with_lm=False))
    assert binding.workspace_bytes(d.layer, cfg.chunk) <= binding.NOALLOC_SCRATCH_BYTES
    ref, got = _pair(d, 64, cfg.chunk)
    assert _same(ref, got)
    ref2, got2 = _pair(d, 19, cfg.chunk)
    assert _same(ref2, got2)


@pytest.mark.parametrize("fmt", [binding.FMT_FP8, binding.FMT_MXFP4, binding.FMT_NVFP4])
def test_noalloc_small_layers_twice(fmt):
    cfg = synth.LayerConfig(f"noalloc_f{fmt}", 120 + fmt, T=300, H=512, E=12, k=4, I=384, fmt=fmt, chunk=5,
                            zipf_alpha=1.0)
    d = gu.DevInputs(synth.make_inputs(cfg))
    ref, got = _pair(d, 300, cfg.chunk)
    assert _same(ref, got)
    ref2, got2 = _pair(d, 41, 3)
    assert _same(ref2, got2)


def test_noalloc_refuses_oversized_layer():
    c = synth.CONFIGS["c4"]
    layer = binding.make_layer(c.T, c.H, c.I, c.E, c.k, c.fmt)
    assert binding.workspace_bytes(layer, c.chunk) > binding.NOALLOC_SCRATCH_BYTES
    with pytest.raises(binding.MoeError) as e:
        # the size check fails on the host before any pointer is used
        binding.expert_forward_noalloc(layer, None, None, None, None, None, None, chunk_experts=c.chunk,
                                       out=torch.empty(0, dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == binding.MOE_ERR_WORKSPACE_TOO_SMALL
