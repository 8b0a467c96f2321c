"""adaln_modulate_noalloc (the allocation-free entry point) against adaln_modulate, both called
through the C ABI with ctypes: identical codes and scales, on two calls in a row (the second with a
smaller input, so the library's scratch still holds the first call's contents), with dynamic and
static scales; the largest L the scratch takes, and the next L rejected with QVD_EWORKSPACE before
anything is launched."""
import ctypes as C

import numpy as np
import pytest
import torch

import workloads as W
from quantized_video_diffusion_amd import _lib

pytestmark = pytest.mark.gpu

MAX_L = 261872          # (4 MiB - 4,352 bytes of partials and padding) / 16 bytes of row statistics


def _p(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _stream():
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _poisoned(shape, dtype):
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(0xFF)
    return t


def _both(x, mod, half, act=None):
    lib = _lib.lib()
    L, d = x.shape
    q_ref, s_ref = _poisoned((L, d), torch.uint8), _poisoned((1,), torch.float32)
    ws = _poisoned((lib.qvd_adaln_modulate_ws_bytes(L, d),), torch.uint8)
    st = lib.adaln_modulate(_p(x), L, d, _p(mod), half, C.c_float(1e-6), _p(act), _p(q_ref), _p(s_ref),
                            _p(ws), ws.numel(), _stream())
    assert st == _lib.QVD_OK, lib.qvd_last_error()
    q, s = _poisoned((L, d), torch.uint8), _poisoned((1,), torch.float32)
    st = lib.adaln_modulate_noalloc(_p(x), L, d, _p(mod), half, C.c_float(1e-6), _p(act), _p(q), _p(s),
                                    _stream())
    assert st == _lib.QVD_OK, lib.qvd_last_error()
    torch.cuda.synchronize()
    return (q.cpu().numpy(), s.cpu().numpy()), (q_ref.cpu().numpy(), s_ref.cpu().numpy())


def _inputs(w, L, seed):
    x = torch.from_numpy(W.activations(w, seed, L=L).view(np.int16)).cuda().view(torch.bfloat16)
    mod = torch.from_numpy(W.random_mod(w.d, seed=seed, tag=w.tag)).cuda()
    return x, mod


def test_noalloc_matches_adaln_modulate_two_calls():
    w = W.WORKLOADS["trim_block_L4096"]
    for L, half, seed in ((4096, 0, 1), (300, 1, 2)):        # the second call is the smaller one
        x, mod = _inputs(w, L, seed)
        (q, s), (q_ref, s_ref) = _both(x, mod, half)
        np.testing.assert_array_equal(q, q_ref)
        np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
        assert s[0] > 0 and (q != 0xFF).any()
    # a static scale uses no scratch
    x, mod = _inputs(w, 777, 3)
    act = torch.tensor([0.02], dtype=torch.float32, device="cuda")
    (q, s), (q_ref, s_ref) = _both(x, mod, 0, act)
    np.testing.assert_array_equal(q, q_ref)
    assert s[0] == np.float32(0.02)


def test_noalloc_largest_length_and_rejection():
    w = W.WORKLOADS["toy_d256_L256"]
    w128 = W.Workload("d128", 77, d=128, n_heads=1, mlp=512, L=MAX_L + 1, sparse=False, outliers=False)
    x, mod = _inputs(w128, MAX_L + 1, 4)
    (q, s), (q_ref, s_ref) = _both(x[:MAX_L], mod, 1)
    np.testing.assert_array_equal(q, q_ref)
    np.testing.assert_array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    lib = _lib.lib()
    qq, ss = _poisoned((MAX_L + 1, 128), torch.uint8), _poisoned((1,), torch.float32)
    st = lib.adaln_modulate_noalloc(_p(x), MAX_L + 1, 128, _p(mod), 0, C.c_float(1e-6), None, _p(qq), _p(ss),
                                    _stream())
    assert st == _lib.QVD_EWORKSPACE
    assert b"261872" in lib.qvd_last_error()
    torch.cuda.synchronize()
    assert (qq.cpu().numpy() == 0xFF).all()                    # nothing was launched
    # and a toy-width call afterwards still agrees
    x, mod = _inputs(w, 256, 5)
    (q, s), (q_ref, s_ref) = _both(x, mod, 0)
    np.testing.assert_array_equal(q, q_ref)
