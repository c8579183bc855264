"""The no-allocation entry point (verify_attn_dense_noalloc) against the
workspace entry point (verify_attn_dense) through the C ABI: two calls in a
row on one GPU, the second smaller, each bitwise equal to the workspace
call and within the oracle's tolerance; and the size limit."""

import numpy as np
import pytest
import torch

from oracle import verify_oracle as vo
from long_context_verify_tree_amd import synth
from _util import check_rows, device_inputs, out_to_f64

pytestmark = pytest.mark.gpu


def _case(ops, cfg):
    x = synth.make_inputs(cfg)
    d = device_inputs(x)
    print(f"case noalloc {cfg.name} B={cfg.B} L={cfg.L} N={cfg.N}", flush=True)
    o_ws, l_ws = ops.verify_attn_dense(**d)
    o_na, l_na = ops.verify_attn_dense_noalloc(**d)
    torch.cuda.synchronize()
    assert torch.equal(o_ws.view(torch.int16) if o_ws.dtype == torch.bfloat16 else o_ws,
                       o_na.view(torch.int16) if o_na.dtype == torch.bfloat16 else o_na)
    assert torch.equal(l_ws, l_na)
    ref, rlse = vo.verify_attention(x.q, x.k_cache, x.v_cache, x.k_draft, x.v_draft, x.parent)
    check_rows(out_to_f64(o_na), ref, l_na.cpu().numpy().astype(np.float64), rlse, cfg.dtype, cfg.name)


def test_noalloc_two_calls_second_smaller(gpu_lib):
    big = synth.small_variant(synth.CONFIGS["l70b_tree128_L128k"], L=5000, B=2)        # shared-tile kernel
    small = synth.small_variant(synth.CONFIGS["llama3_8b_chain8_L32k"], L=700, B=1)   # per-wavefront kernel
    _case(gpu_lib, big)
    _case(gpu_lib, small)
    _case(gpu_lib, synth.CONFIGS["tiny_fp32"])


def test_noalloc_rejects_shapes_beyond_the_scratch(gpu_lib):
    limit = gpu_lib.noalloc_scratch_bytes()
    assert limit == 64 << 20
    # 8 sequences x 64 heads x 256 nodes x (D + 1) floats x parts exceeds 64 MiB
    B, Hq, Hkv, N, D, L = 8, 64, 8, 256, 128, 4096
    q = torch.zeros(B, Hq, N, D, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(B, Hkv, L, D, dtype=torch.bfloat16, device="cuda")
    kd = torch.zeros(B, Hkv, N, D, dtype=torch.bfloat16, device="cuda")
    parent = torch.full((B, N), -1, dtype=torch.int32, device="cuda")
    print("case noalloc beyond the scratch", flush=True)
    with pytest.raises(gpu_lib.VerifyAttnError) as ei:
        gpu_lib.verify_attn_dense_noalloc(q, kc, kc, kd, kd, parent)
    assert ei.value.status == gpu_lib.VA_EWORKSPACE
