"""Helpers of the GPU parity tests: device transfer, the comparison rules, and near-tie detection."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import codecs as OC

DEV = "cuda"


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_dev(bits) -> torch.Tensor:
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to(DEV).view(torch.bfloat16)


def fp16_dev(bits) -> torch.Tensor:
    a = np.ascontiguousarray(bits).view(np.int16)
    return torch.from_numpy(a).to(DEV).view(torch.float16)


def u8_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).to(DEV)


def i32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def f32_dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().cpu().numpy()


def bf16_f64(t: torch.Tensor) -> np.ndarray:
    return OC.bf16_to_f64(host_bits(t))


# --- near-tie detection (decisions taken on fp32 values that the two sides may form in a
#     different summation order) -------------------------------------------------------------------

_E4M3_MAGS = np.array(sorted({abs(float(v)) for v in OC.e4m3_decode(np.arange(0x7F, dtype=np.uint8))}))
_E4M3_MIDS = np.concatenate([(_E4M3_MAGS[:-1] + _E4M3_MAGS[1:]) / 2, [464.0]])
TIE_REL = 2.0 ** -12


def e4m3_near_tie(v) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    i = np.clip(np.searchsorted(_E4M3_MIDS, a), 1, len(_E4M3_MIDS) - 1)
    dist = np.minimum(np.abs(a - _E4M3_MIDS[i - 1]), np.abs(a - _E4M3_MIDS[i]))
    return dist <= TIE_REL * np.maximum(a, 2.0 ** -9)


def int8_near_tie(v) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    dist = np.abs(a - (np.floor(a) + 0.5))
    return (dist <= TIE_REL * np.maximum(a, 1.0)) | (np.abs(a - 127.5) <= TIE_REL * 127.5)


def bf16_near_tie(y, rel: float = TIE_REL, floor: float = 0.0) -> np.ndarray:
    """The float64 value y lies within rel*|y| of a bf16 rounding midpoint.  The FP8 MFMA
    accumulates 128 products per instruction with a relative error of about 2^-14.6 (measured
    against the exact float64 sum), so a bf16 decision that close to its midpoint may go either way."""
    y = np.abs(np.asarray(y, dtype=np.float64))
    _, e = np.frexp(np.where(y > 0, y, 1.0))
    q = np.ldexp(1.0, e - 1 - 7)                     # bf16 spacing in y's binade
    t = y / q
    return np.abs(t - (np.floor(t) + 0.5)) * q <= rel * y + floor


def assert_codes_equal_except_ties(got, want, pre, kind: str, max_frac: float = 1e-4, name="",
                                   upstream=None):
    """Codes must be equal, except where the oracle's pre-rounding value sits within 2^-12 of a
    rounding midpoint (or the saturation threshold), or -- when `upstream` (the float64 value
    before an intermediate bf16 rounding) is given -- where that value sits within
    2^-12 |value| + 1e-4 RMS(values) of a bf16 midpoint; there a neighbouring code is accepted.
    E4M3 +0 and -0 are the same value: where both sides round to zero, the sign of the zero follows the
    sign of a value below the format's resolution, which the two sides' cancellation errors decide;
    such a difference is accepted and counted with the near-ties."""
    got = np.asarray(got).reshape(-1)
    want = np.asarray(want).reshape(-1)
    pre = np.asarray(pre).reshape(-1)
    bad = np.nonzero(got != want)[0]
    if bad.size == 0:
        return 0
    if upstream is not None:
        up = np.asarray(upstream, dtype=np.float64).reshape(-1)
        # the accumulation error is relative to the accumulator's scale, not to each value
        up_near = bf16_near_tie(up[bad], floor=1e-4 * float(np.sqrt(np.mean(up ** 2))))
    else:
        up_near = np.zeros(bad.size, bool)
    if kind == "e4m3":
        zeros = ((got[bad].astype(np.int64) & 0x7F) == 0) & ((want[bad].astype(np.int64) & 0x7F) == 0)
        near = e4m3_near_tie(pre[bad]) | up_near | zeros
        gv = OC.e4m3_decode(got[bad].astype(np.uint8))
        wv = OC.e4m3_decode(want[bad].astype(np.uint8))
        adj = np.abs(gv - wv) <= np.maximum(np.abs(wv), np.abs(gv)) * 2.0 ** -3 + 2.0 ** -9
    else:
        near = int8_near_tie(pre[bad]) | up_near
        adj = np.abs(got[bad].astype(np.int32) - want[bad].astype(np.int32)) <= 1
    ok = near & adj
    if not ok.all():
        k = bad[~ok][:8]
        raise AssertionError(f"{name}: {int((~ok).sum())} code mismatches away from ties, e.g. idx "
                             f"{k.tolist()} got {got[k].tolist()} want {want[k].tolist()} pre {pre[k].tolist()}")
    assert bad.size <= max(8, max_frac * got.size), f"{name}: {bad.size} near-tie flips"
    return int(bad.size)


def assert_close_rms(got, want, rel: float, name=""):
    """max |got - want| <= rel * RMS(want)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.max(np.abs(got - want))) if got.size else 0.0
    assert np.isfinite(got).all(), f"{name}: non-finite output"
    assert err <= rel * rms, f"{name}: max|err| = {err:.3e} > {rel:g} * RMS {rms:.3e}"
    return err / rms if rms else 0.0


def assert_bf16_close(got_bits, want_f64, rel_rms: float = 1e-3, name="", ulps: int = 1):
    """bf16 outputs: within `ulps` bf16 ulps of the exact value plus rel_rms * RMS."""
    got = OC.bf16_to_f64(got_bits)
    want = np.asarray(want_f64, dtype=np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    ulp = ulps * np.abs(want) * 2.0 ** -7
    err = np.abs(got - want)
    bad = err > ulp + rel_rms * rms
    assert not bad.any(), (f"{name}: {int(bad.sum())} bf16 outputs off by more than 1 ulp + "
                           f"{rel_rms:g} RMS; worst {float(err.max()):.3e} (RMS {rms:.3e})")
