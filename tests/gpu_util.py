"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import numpy as np
import torch

import oracle
from late_interaction_retrieval_amd import inputs

DEV = "cuda:0"
D_MODEL = 128

# fp16/bf16 tolerances (spec protocol): |d score| <= 1e-3 * Lq per pair;
# an argmax may differ from the oracle's only where its similarity is within
# 1e-3 of the row maximum; gradients: relative error <= 1e-3, over the whole
# tensor (Frobenius) and over every non-zero row.
SCORE_TOL_PER_QTOKEN = 1e-3
ARGMAX_TIE_TOL = 1e-3
GRAD_REL_TOL = 1e-3


def oracle_dtype(dtn):
    return oracle.F16 if dtn == inputs.F16 else oracle.BF16


def to_dev(a, dtn=None):
    """numpy -> device tensor; uint16 arrays with dtn=BF16 become bfloat16."""
    a = np.ascontiguousarray(a)
    if dtn == inputs.BF16 or (dtn is None and a.dtype == np.uint16):
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def pad_width(a, d=D_MODEL):
    """Zero-pad the last axis to d (zeros leave every dot product unchanged)."""
    out = np.zeros(a.shape[:-1] + (d,), a.dtype)
    out[..., :a.shape[-1]] = a
    return out


def sub_corpus(D_packed, cu, docs, d_scale=None):
    """The packed tokens of the listed documents, with their own cu_seqlens."""
    parts = [D_packed[cu[b]:cu[b + 1]] for b in docs]
    lens = np.array([cu[b + 1] - cu[b] for b in docs], np.int32)
    sub = np.concatenate(parts) if parts else D_packed[:0]
    out = (sub, inputs.cu_seqlens(lens))
    if d_scale is not None:
        out = out + (np.concatenate([d_scale[cu[b]:cu[b + 1]] for b in docs]),)
    return out


def check_scores(got, ref, Lq, where=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape
    inf_ref = np.isneginf(ref)
    assert np.array_equal(np.isneginf(got), inf_ref), where + ": -inf pattern differs"
    err = np.abs(got[~inf_ref] - ref[~inf_ref])
    tol = SCORE_TOL_PER_QTOKEN * Lq
    assert err.size == 0 or err.max() <= tol, "%s: max |dscore| %.3g > %.3g" % (where, err.max(), tol)
    return float(err.max()) if err.size else 0.0


def check_argmax(got, ref_amax, ref_rowmax, sim_at_got, lens_per_doc, where=""):
    """got [Nq,B,Lq] from the GPU.  Accept equality, or an in-range index whose
    oracle similarity is within ARGMAX_TIE_TOL of the oracle row maximum."""
    got = np.asarray(got)
    lens = np.asarray(lens_per_doc)[None, :, None]
    empty = np.broadcast_to(lens == 0, got.shape)
    assert np.all(got[empty] == -1), where + ": empty document must give -1"
    in_range = (got >= 0) & (got < lens)
    assert np.all(in_range | empty), where + ": argmax out of range"
    diff = (got != ref_amax) & ~empty
    ok = sim_at_got[diff] >= ref_rowmax[diff] - ARGMAX_TIE_TOL
    assert np.all(ok), "%s: %d argmax entries are not near-ties" % (where, int((~ok).sum()))
    return int(diff.sum())


def check_grad(got, ref, name, where=""):
    """Gradient parity (Flash-MaxSim Section 4.2, Eqs. (dq), (dd)): the relative
    Frobenius error over the whole tensor, the largest relative error of any
    row whose reference is non-zero (a dropped or doubled source in a single
    row fails this even when the global norm hides it), exact zeros where the
    reference row is zero, and the cosine of the two tensors.  Returns a
    one-line summary."""
    got = np.asarray(got, np.float64).reshape(-1, np.shape(ref)[-1])
    ref = np.asarray(ref, np.float64).reshape(-1, np.shape(ref)[-1])
    assert got.shape == ref.shape, "%s %s: shape" % (where, name)
    fro = rel_fro(got, ref)
    rn = np.linalg.norm(ref, axis=1)
    nz = rn > 0
    row_err = np.linalg.norm(got[nz] - ref[nz], axis=1) / rn[nz]
    worst = float(row_err.max()) if row_err.size else 0.0
    den = np.linalg.norm(got) * np.linalg.norm(ref)
    cos = float((got * ref).sum() / den) if den > 0 else 1.0
    assert fro <= GRAD_REL_TOL, "%s %s: relative Frobenius error %.3g" % (where, name, fro)
    assert worst <= GRAD_REL_TOL, "%s %s: row %d relative error %.3g" % (
        where, name, int(np.flatnonzero(nz)[np.argmax(row_err)]), worst)
    assert np.all(got[~nz] == 0.0), "%s %s: %d rows must be exactly 0" % (where, name, int((got[~nz] != 0).any(1).sum()))
    return "%s: fro %.2e, worst row %.2e over %d rows, cosine %.9f" % (name, fro, worst, int(nz.sum()), cos)


def rel_fro(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def infonce_grad(scores, tau):
    """dL/dscores of L = mean_q [logsumexp_b(s_qb / tau) - s_qq / tau] (fp64)."""
    s = np.asarray(scores, np.float64) / tau
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=1, keepdims=True)
    Nq = p.shape[0]
    eye = np.zeros_like(p)
    eye[np.arange(Nq), np.arange(Nq)] = 1.0
    return (p - eye) / (tau * Nq)
