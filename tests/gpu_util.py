"""Helpers shared by the GPU parity tests (inputs go to the device; expected
values always come from the CPU oracle)."""
import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0") if torch.cuda.is_available() else None
TOL = 2e-3
# Prefill feeds the matrix cores bf16 tiles (unit roundoff 2^-8).  RTN: each
# weight is rounded once, so |y - y_ref| <= 2^-8 sum|w_hat||x| plus the fp32
# accumulation; on the configs' reductions (K >= 512) the errors concentrate
# near 1e-4, far inside 2e-3, but a short reduction can approach 2^-8.
PREFILL_RTN_BOUND = 2.0 ** -8 + 2.0 ** -14
# Binary prefill rounds s2*x and t = (s2*x) V to bf16: against the factored
# magnitude |s1| r sum|s2 x| the error is <= 2 * 2^-8 (1 + 2^-8).
PREFILL_BINLR_FACT_BOUND = 2.0 ** -7 * (1 + 2.0 ** -8) + 2.0 ** -14


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
