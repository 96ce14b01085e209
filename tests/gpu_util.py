"""Helpers shared by the GPU parity tests (inputs go to the device; expected
values always come from the CPU oracle)."""
import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
# The error bound of every fp32 output: max |y - y_ref| / sum |w_hat| |x|.
TOL = 2e-3
# bf16 has 8 significant bits: rounding to nearest even moves a value v by
# at most 2^-8 |v| (unit roundoff), and by at most 2^-8 of the rounded value.
BF16_U = 2.0 ** -8


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return dev(bits.view(np.int16)).view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return oracle.product.bf16_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.cpu().numpy()


def group_reference(W, bits, group):
    """Oracle codes/meta words and W_hat for fp32 W."""
    q, s, o = oracle.rtn.quantize(W, bits, group)
    words = oracle.fmt.pack_codes(q, bits)
    meta = oracle.fmt.pack_meta(s, o)
    return q, s, o, words, meta, oracle.rtn.dequantize(q, s, o, group)


def check_err(y, y_ref, D, tol=TOL):
    err = oracle.product.normalized_error(y, y_ref, D)
    assert err <= tol, f"normalized error {err:.3e} > {tol}"
    return err


def check_bf16_out(y16, y32, y_ref, D):
    """A bf16 output (y16) against the fp32 output of the same call (y32) and
    the oracle: y16 must be y32 rounded to nearest even, bit for bit, and
    |y16 - y_ref| <= 2e-3 D + 2^-8 |y16| element-wise (the bound of the fp32
    result plus the output type's own rounding)."""
    from workloads import f32_to_bf16_bits
    y16 = np.asarray(y16, dtype=np.float64)
    y32 = np.asarray(y32, dtype=np.float32)
    want = oracle.product.bf16_to_f64(f32_to_bf16_bits(y32))
    assert np.array_equal(y16, want), "bf16 output is not the fp32 result rounded to nearest even"
    check_err(y32, y_ref, D)
    excess = np.abs(y16 - y_ref) - BF16_U * np.abs(y16)
    err = np.max(np.where(D > 0, excess / np.where(D > 0, D, 1.0), np.where(excess > 0, np.inf, 0.0)))
    assert err <= TOL, f"bf16 output error beyond its rounding {err:.3e} > {TOL}"
    return err
