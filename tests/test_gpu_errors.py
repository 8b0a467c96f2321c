"""Error propagation on the GPU: a launch failure forced from the host (qvd_inject_launch_failure)
surfaces as QVD_EHIP from the entry point that made the launch -- also from the middle of the block's
chain of launches -- and the next call runs normally."""
import numpy as np
import pytest
import torch

import workloads as W
import quantized_video_diffusion_amd as Q
from quantized_video_diffusion_amd import _lib
from _gpu_util import say, bf16_dev, fp16_dev, i32_dev, host_bits

pytestmark = pytest.mark.gpu


def test_injected_launch_failure_in_quantizer():
    x = bf16_dev(W.normal_bf16((64, 4096), seed=3))
    q_ref, s_ref = Q.quant_fp8_per_tensor(x)
    Q.inject_launch_failure(0)
    with pytest.raises(_lib.QvdError) as err:
        Q.quant_fp8_per_tensor(x)
    assert err.value.status == _lib.QVD_EHIP
    assert "injected failure" in str(err.value)
    # the injection was used up: the next call succeeds and equals the first
    q, s = Q.quant_fp8_per_tensor(x)
    assert torch.equal(q, q_ref) and torch.equal(s, s_ref)
    # a cancelled injection never fires
    Q.inject_launch_failure(0)
    Q.inject_launch_failure(-1)
    Q.quant_fp8_per_tensor(x)


@pytest.mark.parametrize("after", [0, 3, 7])
def test_injected_launch_failure_inside_the_block(after):
    """The block stops at the failed launch and reports it; a clean run afterwards equals a clean run
    before."""
    w = W.WORKLOADS["toy_d256_L256"]
    wb = {k: bf16_dev(v) for k, v in W.block_weights(w, 5, 0).items()}
    bw = Q.quantize_block_weights(wb, w.d, w.n_heads, w.mlp)
    mod = Q.adaln_project(999.0, fp16_dev(W.adaln_basis(w, 5)), fp16_dev(W.adaln_proj(w, 5, 0)))
    idx, cnt = W.block_mask(w, 5, 0)
    kv_idx, kv_cnt = i32_dev(idx), i32_dev(cnt)
    x0 = W.activations(w, 5)
    ref = Q.dit_block_forward(bw, mod, bf16_dev(x0), kv_idx, kv_cnt)
    want = host_bits(ref)
    Q.inject_launch_failure(after)
    with pytest.raises(_lib.QvdError) as err:
        Q.dit_block_forward(bw, mod, bf16_dev(x0), kv_idx, kv_cnt)
    assert err.value.status == _lib.QVD_EHIP and "injected failure" in str(err.value)
    say("block launch", after, "->", str(err.value))
    torch.cuda.synchronize()
    got = Q.dit_block_forward(bw, mod, bf16_dev(x0), kv_idx, kv_cnt)
    np.testing.assert_array_equal(host_bits(got), want)
