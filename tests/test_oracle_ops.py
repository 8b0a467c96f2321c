"""Pins of the oracle's quantizers, GEMM, AdaLN, attention and block against closed forms, brute
force on tiny inputs, special cases that reduce to textbook routines, and invariants."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as W
from oracle import codecs as C, quant as Q, adaln as A, gemm as G, attention as AT, block as B


# --- per-tensor FP8 and INT8 quantizers --------------------------------------------------------

def test_fp8_dynamic_scale_hits_448_and_bounds_error():
    x = W.normal_bf16((300, 77), seed=1, scale=3.0)
    codes, s = Q.quant_fp8_bf16(x)
    xv = C.bf16_to_f64(x)
    amax = np.abs(xv).max()
    assert s == np.float32(amax) / np.float32(448)
    # the element of largest magnitude maps to +-448 exactly
    assert np.abs(C.e4m3_decode(codes)).max() == 448.0
    # relative error of each normal code is at most half a quantum (2^-4) plus fp32 slack
    deq = C.e4m3_decode(codes) * float(s)
    big = np.abs(xv) > float(s) * 2 ** -6
    rel = np.abs(deq - xv)[big] / np.abs(xv)[big]
    assert rel.max() <= 2 ** -4 * (1 + 1e-6)


def test_fp8_with_given_amax_matches_whole_tensor_rule():
    """Row by row with the whole tensor's amax gives the whole-tensor dynamic codes and scale; a
    different amax gives different codes."""
    x = W.bf16_bits_to_f32(W.normal_bf16((200, 64), seed=4, scale=2.0))
    codes, s = Q.quant_fp8_per_tensor(x)
    amax = np.float32(np.abs(x).max())
    for r in (slice(0, 1), slice(50, 120), slice(199, 200)):
        c, s2 = Q.quant_fp8_with_amax(x[r], amax)
        np.testing.assert_array_equal(c, codes[r])
        assert s2 == s
    c, _ = Q.quant_fp8_with_amax(x, amax * np.float32(2))
    assert (c != codes).any()


def test_fp8_zero_tensor_and_static_scale():
    codes, s = Q.quant_fp8_per_tensor(np.zeros(10, np.float32))
    assert s == 1.0 and not codes.any()
    x = np.array([1.0, -2.0, 1000.0], np.float32)
    codes, s = Q.quant_fp8_per_tensor(x, scale_in=np.float32(0.5))
    np.testing.assert_array_equal(C.e4m3_decode(codes), [2.0, -4.0, 448.0])   # 2000 saturates
    assert Q.clip_count(x, 0.5) == 1


def test_int8_qk_tiles_hit_127_and_ragged_tail():
    L, H = 300, 3
    x = W.normal_bf16((L, H, 128), seed=2)
    q, s = Q.quant_int8_qk(x, L, H)
    assert s.shape == (H, 3)
    xv = C.bf16_to_f64(x)
    for h in range(H):
        for i in range(3):
            rows = slice(i * 128, min(L, (i + 1) * 128))
            assert np.abs(q[rows, h]).max() == 127            # every non-zero tile has +-127
            assert s[h, i] == np.float32(np.abs(xv[rows, h]).max()) / np.float32(127)
            err = np.abs(q[rows, h] * float(s[h, i]) - xv[rows, h])
            assert err.max() <= float(s[h, i]) * (0.5 + 1e-5)
    assert np.abs(q.astype(np.int32)).max() <= 127


def test_int8_qk_zero_tile():
    x = np.zeros((130, 1, 128), np.uint16)
    q, s = Q.quant_int8_qk(x, 130, 1)
    assert not q.any() and np.all(s == 1.0)


# --- GEMM ---------------------------------------------------------------------------------------

def _frac_e4m3(c):
    s = -1 if c & 0x80 else 1
    e, m = (c >> 3) & 0xF, c & 7
    return s * (Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))


def test_gemm_fp8_exact_vs_rational_brute_force():
    a = W.random_e4m3_codes((5, 37), seed=3)
    w = W.random_e4m3_codes((4, 37), seed=4, tensor="codes_b")
    acc = G.gemm_acc_fp8(a, w)
    for m in range(5):
        for n in range(4):
            ref = sum(_frac_e4m3(int(a[m, k])) * _frac_e4m3(int(w[n, k])) for k in range(37))
            assert Fraction(float(acc[m, n])) == ref
    y = G.gemm_fp8(a, np.float32(0.3), w, np.float32(0.7), bias=np.arange(4, dtype=np.float32))
    f = float(np.float32(0.3) * np.float32(0.7))
    np.testing.assert_array_equal(y, acc * f + np.arange(4)[None, :])


def test_gemm_fp8_large_k_exact():
    # K = 10,752 (the MLP down projection): the float64 sum is still exact -> order independent
    a = W.random_e4m3_codes((3, 10752), seed=5)
    w = W.random_e4m3_codes((2, 10752), seed=6, tensor="codes_b")
    A_ = C.e4m3_decode(a)
    W_ = C.e4m3_decode(w)
    fwd = G.gemm_acc_fp8(a, w)
    rev = A_[:, ::-1] @ W_[:, ::-1].T
    exact = [[sum(Fraction(float(A_[m, k])) * Fraction(float(W_[n, k])) for k in range(10752))
              for n in range(2)] for m in range(3)]
    np.testing.assert_array_equal(fwd, rev)
    assert all(Fraction(float(fwd[m, n])) == exact[m][n] for m in range(3) for n in range(2))


def test_mxfp4_weight_quant_and_gemm():
    w = W.normal_bf16((6, 96), seed=7, scale=0.05)
    packed, e8 = Q.quant_mxfp4_weight(w)
    assert packed.shape == (6, 48) and e8.shape == (6, 3)
    wv = C.bf16_to_f64(w).reshape(6, 3, 32)
    deq = G.dequant_mxfp4(packed, e8).reshape(6, 3, 32)
    X = C.e8m0_decode(e8)
    # each block's largest element lands in the top binade [4, 8)*X before saturation at 6*X
    assert np.all(np.abs(wv).max(-1) / X >= 4) and np.all(np.abs(wv).max(-1) / X < 8)
    codes = Q.unpack_e2m1(packed).reshape(6, 3, 32)
    np.testing.assert_array_equal(C.e2m1_encode(wv / X[..., None]), codes)
    assert np.all(np.abs(deq) <= 6 * X[..., None])
    a = W.random_e4m3_codes((3, 96), seed=8)
    y = G.gemm_mxfp4(a, np.float32(0.25), packed, e8)
    ref = [[sum(_frac_e4m3(int(a[m, k])) * Fraction(float(deq.reshape(6, 96)[n, k])) for k in range(96))
            for n in range(6)] for m in range(3)]
    np.testing.assert_array_equal(y, np.array(ref, dtype=np.float64) * 0.25)
    # low nibble = even element
    assert (packed[0, 0] & 0xF) == codes.reshape(6, 96)[0, 0]


def test_mxfp4_quantizes_the_given_values_not_their_bf16_rounding():
    """OCP MX rule on exact inputs: a block with amax 4 has X = 1; values just above the E2M1
    midpoints 1.25 and 2.5 round up, the midpoints themselves go to the even code (1.0, 2.0); bf16
    would have rounded the former onto the midpoints.  An amax one fp32 ulp below 4 takes X = 1/2 and
    saturates to 6 X = 3."""
    row = np.zeros((2, 32))
    row[0, :5] = [4.0, 1.25, 1.25 + 2.0 ** -20, 2.5, 2.5 + 2.0 ** -18]
    below4 = float(np.nextafter(np.float32(4.0), np.float32(0.0)))
    row[1, :2] = [below4, -1.0]
    packed, e8 = Q.quant_mxfp4(row)
    codes = Q.unpack_e2m1(packed)
    assert list(e8[:, 0]) == [127, 126]
    assert list(codes[0, :5]) == [6, 2, 3, 4, 5]
    assert list(codes[1, :2]) == [7, 12]                      # 6 X = 3 (saturated); -1 = -2 X (code 4, sign 8)
    pb, eb = Q.quant_mxfp4_weight(C.f64_to_bf16(row))
    assert list(Q.unpack_e2m1(pb)[0, :5]) == [6, 2, 2, 4, 4]
    assert eb[1, 0] == 127                                    # bf16 rounds 4 - ulp up to 4


def test_mxfp4_activation_error_bound():
    """Each dequantized element is within half an E2M1 step of its value, or saturated at 6 X when
    |x| / X > 6 (the block maximum can sit anywhere in [4 X, 8 X))."""
    x = W.bf16_bits_to_f32(W.normal_bf16((64, 256), seed=9, scale=3.0)).astype(np.float64)
    x *= np.exp2(np.random.default_rng(1).integers(-30, 30, size=(64, 1)))
    packed, e8 = Q.quant_mxfp4(x)
    deq = G.dequant_mxfp4(packed, e8)
    X = np.repeat(C.e8m0_decode(e8), 32, axis=1)
    r = np.abs(x) / X
    step = np.where(r < 2, 0.5, np.where(r < 4, 1.0, 2.0))
    sat = r > 6
    assert np.all(np.abs(deq - x)[~sat] <= (step * X)[~sat] / 2)
    np.testing.assert_array_equal(np.abs(deq[sat]), 6 * X[sat])
    assert np.all(np.sign(deq[deq != 0]) == np.sign(x[deq != 0]))


def _frac_mx(packed, e8):
    """Exact rationals of MXFP4 data, element by element from the pinned codecs."""
    codes = Q.unpack_e2m1(packed)
    vals = C.e2m1_decode(codes)
    X = C.e8m0_decode(e8)
    R, K = codes.shape
    return [[Fraction(float(vals[r, k])) * Fraction(float(X[r, k // 32])) for k in range(K)] for r in range(R)]


def test_mxfp4_w4a4_gemm_exact_vs_rational_brute_force():
    a = W.normal_bf16((3, 96), seed=21, scale=1.0)
    w = W.normal_bf16((5, 96), seed=22, scale=0.05)
    ap, ae = Q.quant_mxfp4_weight(a)
    wp, we = Q.quant_mxfp4_weight(w)
    y = G.gemm_mxfp4_w4a4(ap, ae, wp, we)
    A_, W_ = _frac_mx(ap, ae), _frac_mx(wp, we)
    for m in range(3):
        for n in range(5):
            assert Fraction(float(y[m, n])) == sum(A_[m][k] * W_[n][k] for k in range(96))
    b = np.linspace(-1, 1, 5).astype(np.float32)
    np.testing.assert_array_equal(G.gemm_mxfp4_w4a4(ap, ae, wp, we, bias=b), y + b.astype(np.float64)[None, :])


def test_mxfp4_w4a4_block_alignment_and_scale_linearity():
    a = W.normal_bf16((4, 128), seed=23, scale=1.0)
    w = W.normal_bf16((6, 128), seed=24, scale=0.05)
    ap, ae = Q.quant_mxfp4_weight(a)
    wp, we = Q.quant_mxfp4_weight(w)
    y = G.gemm_mxfp4_w4a4(ap, ae, wp, we)
    # activations with only 32-block 2 nonzero: the product of that block alone
    only = ap.copy()
    only[:, :32] = 0
    only[:, 48:] = 0
    Wd = G.dequant_mxfp4(wp, we)
    Ad = G.dequant_mxfp4(ap, ae)
    np.testing.assert_array_equal(G.gemm_mxfp4_w4a4(only, ae, wp, we), Ad[:, 64:96] @ Wd[:, 64:96].T)
    # one more E8M0 step on every block of row 1 doubles row 1 exactly and leaves the others
    ae2 = ae.copy()
    ae2[1] += 1
    y2 = G.gemm_mxfp4_w4a4(ap, ae2, wp, we)
    np.testing.assert_array_equal(y2[1], 2 * y[1])
    np.testing.assert_array_equal(np.delete(y2, 1, 0), np.delete(y, 1, 0))


def test_gelu_vs_math_erf():
    u = np.linspace(-12, 12, 2001)
    ref = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) for v in u])
    np.testing.assert_allclose(G.gelu(u), ref, rtol=1e-14, atol=1e-300)
    assert G.gelu(np.array([0.0]))[0] == 0.0
    assert abs(G.gelu(np.array([10.0]))[0] - 10.0) < 1e-12
    np.testing.assert_allclose(G.gelu(u), torch.nn.functional.gelu(torch.from_numpy(u)).numpy(),
                               rtol=1e-12, atol=1e-15)


# --- AdaLN --------------------------------------------------------------------------------------

def test_timestep_embedding_closed_form():
    e = A.timestep_embedding(999.0, 2688)
    assert e.shape == (2688,)
    assert e[0] == math.cos(999.0) and e[1344] == math.sin(999.0)       # f_0 = 1
    assert abs(e[1343] - math.cos(999.0 * 10000.0 ** (-1343 / 1344))) < 1e-15
    e0 = A.timestep_embedding(0.0, 256)
    np.testing.assert_array_equal(e0, np.r_[np.ones(128), np.zeros(128)])


def test_adaln_factorised_equals_dense_product():
    w = W.WORKLOADS["toy_d256_L256"]
    Bb, Pb = W.adaln_basis(w), W.adaln_proj(w)
    mod = A.adaln_project(874.0, Bb, Pb)
    dense = (C.fp16_to_f64(Pb) @ C.fp16_to_f64(Bb)) @ A.timestep_embedding(874.0, 256)
    np.testing.assert_allclose(mod.reshape(-1).astype(np.float64), dense, rtol=2 ** -23, atol=1e-12)
    assert mod.shape == (6, 256) and mod.dtype == np.float32
    # six vectors: row r of the table is P[r*d:(r+1)*d] c
    c = A.adaln_basis_coords(874.0, Bb)
    np.testing.assert_array_equal(mod[4], (C.fp16_to_f64(Pb)[4 * 256:5 * 256] @ c).astype(np.float32))


def test_layernorm_modulate_plain_ln_and_moments():
    x = W.normal_bf16((64, 256), seed=9, scale=4.0)
    mod = np.zeros((6, 256), np.float32)
    y = A.layernorm_modulate(x, mod, 0, 1e-6).astype(np.float64)
    np.testing.assert_allclose(y.mean(1), 0, atol=1e-6)
    np.testing.assert_allclose(y.var(1), 1, rtol=1e-5)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(C.bf16_to_f64(x)), (256,),
                                         eps=float(np.float32(1e-6))).numpy()
    np.testing.assert_allclose(y, ref, rtol=2 ** -23, atol=1e-7)
    mod = W.random_mod(256, seed=1)
    y2 = A.layernorm_modulate(x, mod, 1, 1e-6).astype(np.float64)
    np.testing.assert_allclose(y2, ref * (1 + mod[4].astype(np.float64)) + mod[3], rtol=1e-6, atol=1e-6)


# --- attention ----------------------------------------------------------------------------------

def _dense_masked_attention(q, sq, k, sk, v, idx, cnt, L):
    """Independent float64 statement: full L x L scores per head, -inf outside kept tiles."""
    H = q.shape[1]
    T = (L + 127) // 128
    out = np.zeros((L, H, 128))
    qd = q.astype(np.float64)
    kd = k.astype(np.float64)
    vd = C.bf16_to_f64(v)
    tile = np.arange(L) // 128
    for h in range(H):
        qs = qd[:, h] * sq[h][tile][:, None].astype(np.float64)
        ks = kd[:, h] * sk[h][tile][:, None].astype(np.float64)
        s = torch.from_numpy(qs @ ks.T / math.sqrt(128))
        keep = torch.zeros(T, T, dtype=torch.bool)
        for i in range(T):
            keep[i, idx[h, i, :cnt[h, i]]] = True
        mask = keep[torch.from_numpy(tile)][:, torch.from_numpy(tile)]
        s = s.masked_fill(~mask, float("-inf"))
        out[:, h] = (torch.softmax(s, dim=-1) @ torch.from_numpy(vd[:, h])).numpy()
    return out


@pytest.mark.parametrize("L,sparse", [(200, True), (391, True), (512, False), (1290, True)])
def test_sparse_attn_vs_dense_masked(L, sparse):
    w = W.Workload("t", 99, d=256, n_heads=2, mlp=1024, L=L, sparse=sparse, outliers=False)
    qb, kb, vb = W.qkv_heads(L, 2, seed=L)
    q, sq = Q.quant_int8_qk(qb, L, 2)
    k, sk = Q.quant_int8_qk(kb, L, 2)
    idx, cnt = W.block_mask(w, seed=1)
    got = AT.sparse_attn(q, sq, k, sk, vb, idx, cnt)
    ref = _dense_masked_attention(q, sq, k, sk, vb, idx, cnt, L)
    np.testing.assert_allclose(got, ref, rtol=0, atol=_f64_bound(vb))


def _f64_bound(vb):
    """Two float64 evaluations of the same softmax-weighted mean (different summation orders, the
    scale applied before or after the product) agree to a few hundred float64 ulps of max|v|."""
    return 1e-13 * np.abs(C.bf16_to_f64(vb)).max()


def test_sparse_attn_v_outside_fp16_range():
    """V is taken as bf16: magnitudes far above 65,504 and far below 2^-14 (outside fp16's normal
    range) enter the product as they are.  Head 0 has key rows scaled by 1e6 in a quarter of the
    dims, head 1 is scaled by 1e-9 throughout; both heads agree with the dense masked statement to
    float64 rounding of their own magnitude, and head 1 is exactly 1e-9-ish times a unit-scale
    attention (no flush to zero)."""
    L, H = 391, 2
    w = W.Workload("t", 97, d=256, n_heads=2, mlp=1024, L=L, sparse=True, outliers=False)
    qb, kb, vb = W.qkv_heads(L, H, seed=11)
    v = C.bf16_to_f64(vb)
    v[::3, 0, :32] *= 1e6
    v[:, 1, :] *= 1e-9
    vb2 = C.f64_to_bf16(v)
    q, sq = Q.quant_int8_qk(qb, L, H)
    k, sk = Q.quant_int8_qk(kb, L, H)
    idx, cnt = W.block_mask(w, seed=2)
    got = AT.sparse_attn(q, sq, k, sk, vb2, idx, cnt)
    ref = _dense_masked_attention(q, sq, k, sk, vb2, idx, cnt, L)
    for h in range(H):
        np.testing.assert_allclose(got[:, h], ref[:, h], rtol=0, atol=_f64_bound(vb2[:, h]))
    assert np.abs(got[:, 0, :32]).max() > 1e5          # the large rows dominate those outputs
    assert 0 < np.abs(got[:, 1]).max() < 1e-7
    assert np.abs(got[:, 1]).min() > 0


def test_sparse_attn_special_cases():
    L, H = 300, 1
    w = W.Workload("t", 98, d=128, n_heads=1, mlp=512, L=L, sparse=False, outliers=False)
    qb, kb, vb = W.qkv_heads(L, H, seed=5)
    q, sq = Q.quant_int8_qk(qb, L, H)
    k, sk = Q.quant_int8_qk(kb, L, H)
    idx, cnt = W.block_mask(w)
    # all tiles kept == ordinary softmax attention (torch SDPA in float64)
    got = AT.sparse_attn(q, sq, k, sk, vb, idx, cnt)
    tile = np.arange(L) // 128
    qs = torch.from_numpy(q[:, 0].astype(np.float64) * sq[0][tile][:, None])
    ks = torch.from_numpy(k[:, 0].astype(np.float64) * sk[0][tile][:, None])
    vs = torch.from_numpy(C.bf16_to_f64(vb[:, 0]))
    ref = torch.nn.functional.scaled_dot_product_attention(qs[None], ks[None], vs[None])[0]
    np.testing.assert_allclose(got[:, 0], ref.numpy(), rtol=0, atol=_f64_bound(vb))
    # diagonal only == block-diagonal attention: tile i only sees itself
    T = 3
    diag = np.arange(T, dtype=np.int32)[None, :, None].copy()
    one = np.ones((1, T), np.int32)
    gd = AT.sparse_attn(q, sq, k, sk, vb, diag, one)
    for i in range(T):
        r = slice(i * 128, min(L, (i + 1) * 128))
        sub = torch.nn.functional.scaled_dot_product_attention(qs[r][None], ks[r][None], vs[r][None])[0]
        np.testing.assert_allclose(gd[r, 0], sub.numpy(), rtol=0, atol=_f64_bound(vb))
    # constant V -> every output row is that constant (weights normalised by their own sum)
    vc = np.full_like(vb, 0x3F80)          # 1.0
    np.testing.assert_allclose(AT.sparse_attn(q, sq, k, sk, vc, idx, cnt), 1.0, rtol=0, atol=1e-13)
    # no kept tile -> the row attends to nothing: zeros (the empty softmax is read as zero weight)
    none = np.zeros((1, T), np.int32)
    assert not AT.sparse_attn(q, sq, k, sk, vb, diag, none).any()
    # Q = 0 -> uniform weights: the mean of the kept V rows
    gz = AT.sparse_attn(np.zeros_like(q), sq, k, sk, vb, diag, one)
    for i in range(T):
        r = slice(i * 128, min(L, (i + 1) * 128))
        np.testing.assert_allclose(gz[r, 0], np.broadcast_to(C.bf16_to_f64(vb[r, 0]).mean(0), gz[r, 0].shape),
                                   rtol=1e-12, atol=1e-14)


def test_mask_draw_structure():
    w = W.WORKLOADS["attn_480p"]
    idx, cnt = W.block_mask(w, seed=0)
    assert idx.shape == (21, 264, 53) and np.all(cnt == 53)
    assert np.all(np.diff(idx, axis=-1) > 0)                     # sorted, distinct
    assert np.all((idx == np.arange(264)[None, :, None]).any(-1))  # diagonal present
    assert idx.min() >= 0 and idx.max() < 264
    assert W.kept_tiles_per_row(670) == 135 and W.kept_tiles_per_row(2) == 1
    # 80% sparsity: kept fraction 53/264 = 20.08%
    assert abs(53 / 264 - 0.2) < 0.002


# --- block --------------------------------------------------------------------------------------

def _toy_block(seed=0, gate=None, L=None):
    w = W.WORKLOADS["toy_d256_L256"]
    L = w.L if L is None else L
    x = W.activations(w, seed, L=L)
    qw = B.quantize_block_weights(W.block_weights(w, seed))
    mod = W.random_mod(w.d, seed=seed, tag=w.tag, gate=gate)
    idx, cnt = W.block_mask(w, seed, L=L)
    return w, x, qw, mod, idx, cnt


def test_block_zero_gates_is_identity():
    w, x, qw, mod, idx, cnt = _toy_block(gate=0.0)
    out = B.dit_block(x, mod, qw, idx, cnt, w.n_heads)
    np.testing.assert_array_equal(out, x)


def test_block_close_to_unquantized_float64_block():
    """Gates 1 and no modulation: the quantized block tracks a float64 pre-LN transformer block
    written with torch ops on the bf16 master weights (quantization error only)."""
    w, x, qw, mod, idx, cnt = _toy_block(seed=3, gate=1.0)
    mod[[0, 1, 3, 4]] = 0.0
    out, inter = B.dit_block(x, mod, qw, idx, cnt, w.n_heads, keep=True)
    wb = {k: torch.from_numpy(C.bf16_to_f64(v)) for k, v in W.block_weights(w, 3).items()}
    xt = torch.from_numpy(C.bf16_to_f64(x))
    ln = lambda t: torch.nn.functional.layer_norm(t, (w.d,), eps=1e-6)
    qkv = ln(xt) @ wb["w_qkv"].T
    q, k, v = (qkv[:, i * 256:(i + 1) * 256].reshape(256, 2, 128).transpose(0, 1) for i in range(3))
    att = torch.nn.functional.scaled_dot_product_attention(q, k, v).transpose(0, 1).reshape(256, 256)
    x1 = xt + att @ wb["w_o"].T
    x2 = x1 + torch.nn.functional.gelu(ln(x1) @ wb["w_up"].T) @ wb["w_down"].T
    got = C.bf16_to_f64(out)
    branch_ref = (x2 - xt).numpy()
    branch_got = got - xt.numpy()
    rel = np.sqrt(((branch_got - branch_ref) ** 2).mean() / (branch_ref ** 2).mean())
    assert rel < 0.08, rel
    # the attention-branch input scale is the amax rule on the modulated LN output
    y = A.layernorm_modulate(x, mod, 0, 1e-6)
    assert inter["s1"] == np.float32(np.abs(y).max()) / np.float32(448)


def test_block_static_scales_and_mxfp4_run():
    w, x, qw, mod, idx, cnt = _toy_block(seed=4)
    out_dyn, it = B.dit_block(x, mod, qw, idx, cnt, w.n_heads, keep=True)
    st = [it["s1"], it["so"], it["s2"], it["sg"]]
    out_st = B.dit_block(x, mod, qw, idx, cnt, w.n_heads, act_scales=st)
    np.testing.assert_array_equal(out_st, out_dyn)     # static == dynamic when given the same s
    wb = W.block_weights(w, 4)
    qm = {}
    for site in B.SITES:
        qm["w_" + site], qm["e8_" + site] = Q.quant_mxfp4_weight(wb["w_" + site])
    out4 = B.dit_block(x, mod, qm, idx, cnt, w.n_heads, act_scales=st, fmt="mxfp4")
    d8 = C.bf16_to_f64(out_dyn) - C.bf16_to_f64(x)
    d4 = C.bf16_to_f64(out4) - C.bf16_to_f64(x)
    assert np.sqrt(((d4 - d8) ** 2).mean() / (d8 ** 2).mean()) < 0.3


def _w4a4_weights(w, seed):
    wb = W.block_weights(w, seed)
    qm = {}
    for site in B.SITES:
        qm["w_" + site], qm["e8_" + site] = Q.quant_mxfp4_weight(wb["w_" + site])
    return qm


def test_block_w4a4_zero_gates_is_identity():
    w, x, _, mod, idx, cnt = _toy_block(gate=0.0)
    out = B.dit_block(x, mod, _w4a4_weights(w, 0), idx, cnt, w.n_heads, fmt="w4a4")
    np.testing.assert_array_equal(out, x)


def test_block_w4a4_tracks_fp8_block():
    """Both operands 4-bit: the block's branch (out - x) stays close to the FP8 block's, and the GEMM
    inputs are the MXFP4 quantization of the modulated LayerNorm outputs, O and GELU."""
    w, x, qw, mod, idx, cnt = _toy_block(seed=4)
    out8 = B.dit_block(x, mod, qw, idx, cnt, w.n_heads)
    out4, it = B.dit_block(x, mod, _w4a4_weights(w, 4), idx, cnt, w.n_heads, fmt="w4a4", keep=True)
    d8 = C.bf16_to_f64(out8) - C.bf16_to_f64(x)
    d4 = C.bf16_to_f64(out4) - C.bf16_to_f64(x)
    rel = np.sqrt(((d4 - d8) ** 2).mean() / (d8 ** 2).mean())
    assert 0.01 < rel < 0.4, rel
    y = A.layernorm_modulate(x, mod, 0, 1e-6).astype(np.float64)
    deq = G.dequant_mxfp4(*it["h1"])
    assert np.sqrt(((deq - y) ** 2).mean() / (y ** 2).mean()) < 0.15
    assert it["s1"] is None and it["so"] is None and it["sg"] is None
    assert it["g8"][0].shape == (w.L, w.mlp // 2) and it["g8"][1].shape == (w.L, w.mlp // 32)


# --- calibration ----------------------------------------------------------------------------------

def test_calibration_zero_clips_and_uncalibrated_clips():
    d_in, nb, tok = 512, 8, 64
    ch, fac, a0 = W.outlier_spec(d_in, 137.0, site=3, n_batches=nb, tokens=tok)
    batches = [W.apply_outliers(W.calibration_batch(d_in, b, site=3, tokens=tok), ch, fac)
               for b in range(nb)]
    amax = max(float(np.abs(b).max()) for b in batches)
    assert abs(amax / a0 - 137.0) < 1e-4
    s = Q.calibrated_scale(amax)
    assert float(s) * 448 >= amax
    assert sum(Q.clip_count(b, s) for b in batches) == 0
    s_uncal = Q.calibrated_scale(a0)
    assert sum(Q.clip_count(b, s_uncal) for b in batches) > 0
    # a site without outliers calibrated on its own draw does not clip either
    plain = [W.calibration_batch(d_in, b, site=0, tokens=tok) for b in range(nb)]
    s0 = Q.calibrated_scale(max(float(np.abs(b).max()) for b in plain))
    assert sum(Q.clip_count(b, s0) for b in plain) == 0


def test_calibrated_scale_rounds_up():
    # pick an amax whose fp32(amax/448)*448 falls below amax
    for a in np.random.default_rng(0).uniform(1, 100, 2000).astype(np.float32):
        s = Q.calibrated_scale(a)
        assert float(s) * 448 >= float(a)
        assert float(np.nextafter(s, np.float32(0))) * 448 < float(a)
