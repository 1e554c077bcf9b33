"""Shared pieces of the GPU merge tests: run a synthetic case through the C ABI,
run the same host tensors through the fp64 oracle, and compare.

Tolerance (the reading of "within 2 bf16 ULP" used throughout): with r the
fp64 oracle value and A = sum_s (w_s/S)|O_s| the magnitude of the terms that
were summed,
    |g - r| <= 2 ulp_bf16(r) + 2^-16 A,   ulp_bf16(r) = 2^(floor(log2 |r|) - 7);
for fp16 payloads the same with ulp_f16(r) = 2^(max(floor(log2 |r|), -14) - 10).
The second term only matters under cancellation (|r| << A), where fp32
accumulation error of order cp * 2^-24 A can exceed 2 ulp(r) although every
step is correctly rounded.  Every check reports how many elements needed that
term (the "floor") and asserts that each of them is a cancellation: |r| <
2^-8 A (without cancellation |r| is close to A and 2 ulp(r) alone covers the
fp32 error many times over).  The merged LSE must satisfy
|L_g - L_r| <= 1e-5 max(|L_r|, 1), and -inf must match exactly.
"""
import sys

import numpy as np
import torch

import context_lse_merge_amd as dcp
import oracle
import synth

LAYOUT = {"bhc": dcp.DCP_LSE_BHC, "bh1": dcp.DCP_LSE_BH1}
MODE = {"e": dcp.DCP_LSE_BASE_E, "2": dcp.DCP_LSE_BASE_2}
OLAYOUT = {"bhc": oracle.LSE_BHC, "bh1": oracle.LSE_BH1}
OMODE = {"e": oracle.BASE_E, "2": oracle.BASE_2}


def announce(msg):
    """Name the case on the real stderr (not captured) before touching the GPU."""
    print("[gpu-case] " + msg, file=sys.__stderr__, flush=True)


def bf16_ulp(r):
    a = np.maximum(np.abs(r), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)


def f16_ulp(r):
    """Spacing of IEEE binary16 at |r|: 2^(e - 10), with e >= -14 (subnormals are 2^-24 apart)."""
    a = np.maximum(np.abs(r), 2.0 ** -14)
    return np.exp2(np.floor(np.log2(a)) - 10)


def payload_ulp(r, dtype):
    return f16_ulp(r) if dtype == torch.float16 else bf16_ulp(r)


def bits_of(t):
    """Raw bf16 bits of a (GPU or CPU) bf16 tensor as uint16 numpy."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def gpu_merge(case, capacity=None, with_lse=True, attn=None, lse=None, out=None, out_lse=None, stream=None):
    """Run ``case`` through dcp_lse_combine on cuda:0.  ``attn``/``lse`` override the
    device copies (e.g. strided views).  Returns (out, out_lse) as GPU tensors."""
    dev = torch.device("cuda:0")
    if attn is None:
        attn = case.attn.to(dev)
    if lse is None:
        lse = case.lse.to(dev)
    B, hl = case.B, case.h_local
    if out is None:
        out = torch.empty((B, hl, synth.D), dtype=case.attn.dtype, device=dev)
    if with_lse and out_lse is None:
        out_lse = torch.empty((B, hl), dtype=torch.float32, device=dev)
    cap = capacity or max(B, 1)
    announce("dcp_lse_combine %s capacity=%d attn=%s strides=%s lse=%s%s" % (
        case.name, cap, tuple(attn.shape), attn.stride(), case.lse_layout, tuple(lse.shape)))
    dtype = dcp.DCP_DTYPE_FP16 if case.attn.dtype == torch.float16 else dcp.DCP_DTYPE_BF16
    ws = dcp.dcp_workspace_create(cap, hl, case.cp, dtype=dtype, stream=stream)
    try:
        dcp.dcp_lse_combine(ws, attn, lse, LAYOUT[case.lse_layout], MODE[case.lse_mode], out,
                            out_lse if with_lse else None, stream=stream)
        torch.cuda.synchronize()
    finally:
        ws.close()
    return out, out_lse


def oracle_merge(case, lse=None):
    lse_np = (case.lse if lse is None else lse).contiguous().numpy()
    return oracle.merge(synth.bits16(case.attn.contiguous()), lse_np, case.cp, OLAYOUT[case.lse_layout],
                        OMODE[case.lse_mode], dtype=synth.payload_name(case.attn))


def check_against_oracle(case, out, out_lse, ref=None):
    """Assert the GPU result meets the tolerance; returns a small report dict."""
    r, rL, A = ref if ref is not None else oracle_merge(case)
    g = out.float().cpu().double().numpy()
    assert not np.isnan(g).any(), "%s: NaN in the merged output" % case.name
    err = np.abs(g - r)
    ulp = payload_ulp(r, case.attn.dtype)
    ulp_tol = 2 * ulp
    tol = ulp_tol + 2.0 ** -16 * A
    bad = err > tol
    assert not bad.any(), "%s: %d elements out of tolerance; worst |g-r| = %.4g at %s (r = %.6g, tol %.3g)" % (
        case.name, int(bad.sum()), err.max(), np.unravel_index(np.argmax(err - tol), err.shape),
        r.flat[np.argmax(err - tol)], tol.flat[np.argmax(err - tol)])
    floored = err > ulp_tol
    not_cancel = floored & (np.abs(r) >= 2.0 ** -8 * A)
    assert not not_cancel.any(), "%s: %d elements needed the 2^-16 A floor without cancellation (|r| >= 2^-8 A)" % (
        case.name, int(not_cancel.sum()))
    report = {"max_err_ulps": float(np.max(err / ulp)), "needed_floor": int(floored.sum()), "elements": int(err.size),
              "max_err_over_A": float(np.max(err / np.maximum(A, 1e-300)))}
    if out_lse is not None:
        gL = out_lse.cpu().double().numpy()
        inf = np.isneginf(rL)
        assert np.array_equal(np.isneginf(gL), inf), "%s: -inf pattern of the merged LSE differs" % case.name
        d = np.abs(gL[~inf] - rL[~inf])
        lim = 1e-5 * np.maximum(np.abs(rL[~inf]), 1.0)
        assert np.all(d <= lim), "%s: merged LSE off by %.3g (limit %.3g)" % (case.name, d.max(),
                                                                              lim[np.argmax(d - lim)])
        report["max_lse_rel"] = float(np.max(d / np.maximum(np.abs(rL[~inf]), 1.0))) if d.size else 0.0
    announce("%s: %d elements, max error %.3f ulp, %d needed the cancellation floor (all with |r| < 2^-8 A)%s" % (
        case.name, report["elements"], report["max_err_ulps"], report["needed_floor"],
        ", merged LSE max rel err %.2e" % report["max_lse_rel"] if "max_lse_rel" in report else ""))
    return report
