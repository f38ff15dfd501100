"""The drop-in modules (DAK paper §5 "Implementation": SplitK_GEMM replaces
nn.Linear, SplitK_FlashAttn replaces scaled dot-product attention) against the
fp64 oracle, bit-identical across offload ratios."""
import numpy as np
import pytest
import torch

import synth
from oracle import attention as oa
from oracle.gemm import gemm, normwise_error, to_f64
import tiered_memory_offloading_amd as dak
from tiered_memory_offloading_amd.nn import SplitK_FlashAttn, SplitK_GEMM

pytestmark = pytest.mark.gpu
TOL = 1e-2


def test_splitk_gemm_replaces_linear():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    torch.manual_seed(0)
    lin = torch.nn.Linear(1024, 1536, bias=True)
    with torch.no_grad():
        lin.weight.copy_(synth.gemm_inputs(1536, 1024, 1, seed=20)[0].float())
        lin.bias.copy_(torch.linspace(-1, 1, 1536))
    lin = lin.to(torch.bfloat16)
    x = synth.gemm_inputs(6, 1024, 1, seed=21)[0].reshape(2, 3, 1024)   # bf16 activations, any leading shape
    W = to_f64(lin.weight.detach())
    b = lin.bias.detach().double().numpy()
    ref = gemm(W, to_f64(x.reshape(6, 1024))) + b[None, :]
    outs = []
    for ratio in (0.0, 0.25, 1.0):
        mod = SplitK_GEMM.from_linear(lin, host_ratio=ratio, out_dtype=torch.float32)
        assert mod.h == {0.0: 0, 0.25: 6, 1.0: 24}[ratio]
        y = mod(x.cuda())
        torch.cuda.synchronize()
        assert y.shape == (2, 3, 1536) and y.dtype == torch.float32
        outs.append(y.cpu())
    assert normwise_error(outs[0].reshape(6, 1536).numpy(), ref) <= TOL
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])
    # default output dtype follows the input's
    y16 = SplitK_GEMM.from_linear(lin, host_ratio=0.25)(x.cuda())
    assert y16.dtype == torch.bfloat16 and torch.equal(y16.cpu(), outs[0].to(torch.bfloat16))


def test_splitk_flashattn_replaces_sdpa():
    B, Hq, Hkv, D, ctx = 4, 8, 2, 128, 700
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=22)
    ref = oa.decode_attention(to_f64(q), to_f64(K), to_f64(V), 1.0 / np.sqrt(D))
    outs = []
    for ratio in (0.0, 0.5, 1.0):
        mod = SplitK_FlashAttn(K, V, host_ratio=ratio, out_dtype=torch.float32)
        assert mod.h == {0.0: 0, 0.5: 2, 1.0: 4}[ratio]
        o = mod(q[:, :, None, :].cuda())            # SDPA's [B, Hq, L=1, D]
        torch.cuda.synchronize()
        assert o.shape == (B, Hq, 1, D)
        outs.append(o.cpu()[:, :, 0, :])
    assert normwise_error(outs[0].numpy(), ref) <= TOL
    assert torch.equal(outs[1], outs[0]) and torch.equal(outs[2], outs[0])
    mod = SplitK_FlashAttn(K, V, host_ratio=0.5)
    with pytest.raises(ValueError):
        mod(q.cuda(), attn_mask=torch.ones(1))
    with pytest.raises(ValueError):
        mod(q[:, :, None, :].expand(B, Hq, 2, D).contiguous().cuda())


def test_splitk_flashattn_head_units_and_ragged_batch():
    B, Hq, Hkv, D, ctx = 3, 8, 2, 128, 2500
    q, K, V = synth.attn_inputs(B, Hq, Hkv, D, ctx, seed=23)
    lens = torch.tensor([2500, 300, 2049])
    ref = oa.decode_attention_lens(to_f64(q), to_f64(K), to_f64(V), 1.0 / np.sqrt(D), lens.tolist())
    base = SplitK_FlashAttn(K, V, out_dtype=torch.float32, ctx_lens=lens)(q.cuda()).cpu()
    for b in range(B):
        assert normwise_error(base[b].numpy(), ref[b]) <= TOL
    mod = SplitK_FlashAttn(K, V, host_ratio=0.5, out_dtype=torch.float32, unit=dak.KV_UNIT_HEAD, ctx_lens=lens)
    assert mod.h == 3 and mod.kv.host_units == 3
    assert torch.equal(mod(q.cuda()).cpu(), base)
