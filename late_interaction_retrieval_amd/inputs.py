"""Seeded synthetic inputs shaped like the paper's workloads.

This module only draws and formats data; it holds none of the MaxSim
arithmetic, so both the HIP path (through the binding) and the CPU oracle can
be fed the same host bytes from it.

Recipe (one definition for every workload):
  * token rows are ``x ~ N(0, 1)`` in fp32, drawn in chunks of ``CHUNK`` rows
    with ``numpy.random.default_rng([seed, workload_id, stream, chunk])``;
  * every row is divided by its fp32 L2 norm (token embeddings are
    l2-normalised, paper Section 3.1), then rounded to nearest-even into fp16
    or bf16 (bf16 is returned as its uint16 bit pattern);
  * int8 rows are quantised from the same normalised fp32 rows, symmetric and
    per token: ``scale = max_k |x_k| / 127`` and
    ``q = clip(rint(x / scale), -127, 127)`` (ties to even); an all-zero row
    gets scale 1 (the paper gives only "per-token symmetric", Section 4.3);
  * document lengths are integer-uniform on an inclusive range, drawn with
    ``default_rng([seed, workload_id, 2])``;
  * streams: 0 = queries, 1 = documents, 2 = lengths, 3 = extra draws.
"""
from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CHUNK = 1 << 18  # rows per generator chunk
STREAM_Q, STREAM_D, STREAM_LEN, STREAM_EXTRA = 0, 1, 2, 3

F16 = "f16"
BF16 = "bf16"
I8 = "i8"


def _workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(x):
    """Round fp32 to bf16 (nearest, ties to even) and return the uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_rows(seed, workload_id, stream, chunk, n, d):
    rng = np.random.default_rng([seed, workload_id, stream, chunk])
    x = np.empty((n, d), np.float32)
    rng.standard_normal(out=x, dtype=np.float32)
    return x


def l2_normalise(x):
    norm = np.sqrt(np.einsum("ij,ij->i", x, x, dtype=np.float32))
    norm[norm == 0] = 1.0
    return x / norm[:, None]


def quantise_rows(x):
    """Symmetric per-token int8 quantisation of fp32 rows -> (int8 rows, fp32 scales)."""
    amax = np.max(np.abs(x), axis=1)
    scale = (amax / np.float32(127.0)).astype(np.float32)
    scale[scale == 0] = 1.0
    q = np.clip(np.rint(x / scale[:, None]), -127, 127).astype(np.int8)
    return q, scale


def unit_rows(seed, workload_id, stream, n, d, dtype):
    """n l2-normalised N(0,1) rows of width d in ``dtype``.

    Returns fp16 array, bf16 bits (uint16), or (int8 rows, fp32 scales).
    """
    if dtype == I8:
        out = np.empty((n, d), np.int8)
        scales = np.empty(n, np.float32)
    else:
        out = np.empty((n, d), np.float16 if dtype == F16 else np.uint16)
        scales = None

    def fill(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        x = l2_normalise(normal_rows(seed, workload_id, stream, c, hi - lo, d))
        if dtype == F16:
            out[lo:hi] = x.astype(np.float16)
        elif dtype == BF16:
            out[lo:hi] = f32_to_bf16_bits(x)
        else:
            q, s = quantise_rows(x)
            out[lo:hi] = q
            scales[lo:hi] = s

    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return (out, scales) if dtype == I8 else out


def lengths(seed, workload_id, B, lo, hi):
    """B document lengths, integer-uniform on [lo, hi]."""
    rng = np.random.default_rng([seed, workload_id, STREAM_LEN])
    return rng.integers(lo, hi + 1, size=B, dtype=np.int64).astype(np.int32)


def cu_seqlens(lens):
    cu = np.zeros(len(lens) + 1, np.int64)
    np.cumsum(lens, out=cu[1:])
    if cu[-1] >= 2**31:
        raise ValueError("total token count does not fit int32 cu_seqlens")
    return cu.astype(np.int32)


def pad_packed(D_packed, cu, Ld_max):
    """Scatter a packed [T, d] corpus into a zero-padded [B, Ld_max, d] tensor."""
    B = len(cu) - 1
    out = np.zeros((B, Ld_max) + D_packed.shape[1:], D_packed.dtype)
    for b in range(B):
        n = cu[b + 1] - cu[b]
        out[b, :n] = D_packed[cu[b]:cu[b + 1]]
    return out


# ----------------------------------------------------------------------------
# The five workloads.  ``scale_docs`` shrinks the document count (the oracle
# then finishes in seconds) while keeping every other property.
# ----------------------------------------------------------------------------

WORKLOADS = {
    "colbert_tiny": dict(id=1, Nq=1, Lq=32, B=1000, Ld=(180, 180), d=128, dtype=F16),
    "colbert_rerank_varlen": dict(id=2, Nq=64, Lq=32, B=10000, Ld=(32, 300), d=128, dtype=F16),
    "colpali_fwd": dict(id=3, Nq=4, Lq=1024, B=10000, Ld=(1024, 1024), d=128, dtype=BF16),
    "contrastive_train": dict(id=4, Nq=64, Lq=1024, B=64, Ld=(1024, 1024), d=128, dtype=BF16,
                              tau=0.02),
    "int8_varlen": dict(id=5, Nq=32, Lq=32, B=100000, Ld=(32, 512), d=128, dtype=I8),
    # the training step over a ragged in-batch corpus (packed backward)
    "contrastive_train_varlen": dict(id=7, Nq=64, Lq=1024, B=64, Ld=(256, 1024), d=128, dtype=BF16,
                                     tau=0.02),
}


def make(name, seed=0, B=None, Nq=None, Lq=None, Ld=None):
    """Host arrays for one workload.

    Keys: Q [Nq, Lq, d]; D_packed [T, d]; cu_seqlens [B+1]; lens [B]; Ld_max;
    for int8 also q_scale [Nq, Lq] and d_scale [T].  The document set is
    always generated packed; ``pad_packed`` gives the padded form.
    Optional overrides shrink a workload for tests (same recipe, same seed).
    """
    w = dict(WORKLOADS[name])
    if B is not None:
        w["B"] = B
    if Nq is not None:
        w["Nq"] = Nq
    if Lq is not None:
        w["Lq"] = Lq
    if Ld is not None:
        w["Ld"] = Ld if isinstance(Ld, tuple) else (Ld, Ld)
    lo, hi = w["Ld"]
    if lo == hi:
        lens = np.full(w["B"], lo, np.int32)
    else:
        lens = lengths(seed, w["id"], w["B"], lo, hi)
    cu = cu_seqlens(lens)
    T = int(cu[-1])
    out = dict(name=name, Nq=w["Nq"], Lq=w["Lq"], B=w["B"], d=w["d"], Ld_max=hi, dtype=w["dtype"],
               lens=lens, cu_seqlens=cu, T=T)
    if "tau" in w:
        out["tau"] = w["tau"]
    if w["dtype"] == I8:
        q, qs = unit_rows(seed, w["id"], STREAM_Q, w["Nq"] * w["Lq"], w["d"], I8)
        dq, ds = unit_rows(seed, w["id"], STREAM_D, T, w["d"], I8)
        out.update(Q=q.reshape(w["Nq"], w["Lq"], w["d"]), q_scale=qs.reshape(w["Nq"], w["Lq"]),
                   D_packed=dq, d_scale=ds)
    else:
        out["Q"] = unit_rows(seed, w["id"], STREAM_Q, w["Nq"] * w["Lq"], w["d"],
                             w["dtype"]).reshape(w["Nq"], w["Lq"], w["d"])
        out["D_packed"] = unit_rows(seed, w["id"], STREAM_D, T, w["d"], w["dtype"])
    return out


def fp16_of_int8_workload(w, seed=0):
    """fp16 versions (Q [Nq, Lq, d], D_packed [T, d]) of the same normalised
    rows an int8 workload from ``make`` was quantised from: the rescoring
    pass of the two-stage scan reads these."""
    wid = WORKLOADS[w["name"]]["id"]
    q = unit_rows(seed, wid, STREAM_Q, w["Nq"] * w["Lq"], w["d"], F16).reshape(w["Nq"], w["Lq"], w["d"])
    dd = unit_rows(seed, wid, STREAM_D, w["T"], w["d"], F16)
    return q, dd


def random_rows(seed, n, d, dtype, workload_id=99, stream=STREAM_EXTRA):
    """Small helper for tests: n unit rows under an arbitrary id/stream."""
    return unit_rows(seed, workload_id, stream, n, d, dtype)


# Point clouds for the Chamfer distance (paper Section 4.2 "Generalization to
# Chamfer Distance": two point sets in R^3, up to 100K points).  Recipe: each
# cloud is a noisy sample of the unit sphere, the shape-matching setting the
# page names: directions x ~ N(0, I_3) divided by their fp32 norm, then
# per-coordinate N(0, sigma^2) noise, all fp32, drawn with
# ``default_rng([seed, CHAMFER_ID, stream, item])`` (stream 0 = P, 1 = Q).
CHAMFER_ID = 6
CHAMFER_WORKLOADS = {
    "chamfer_100k": dict(Bt=1, N=100000, M=100000),
    "chamfer_batch": dict(Bt=32, N=2048, M=2048),
}


def sphere_cloud(seed, stream, item, n, sigma=0.01):
    """n points near the unit sphere, fp32 [n, 3]."""
    rng = np.random.default_rng([seed, CHAMFER_ID, stream, item])
    x = np.empty((n, 3), np.float32)
    rng.standard_normal(out=x, dtype=np.float32)
    nrm = np.sqrt((x * x).sum(axis=1, dtype=np.float32))
    x /= np.where(nrm > 0, nrm, np.float32(1))[:, None]
    noise = np.empty((n, 3), np.float32)
    rng.standard_normal(out=noise, dtype=np.float32)
    x += np.float32(sigma) * noise
    return x


def point_clouds(seed=0, Bt=1, N=1000, M=1000, sigma=0.01):
    """(P [Bt, N, 3], Q [Bt, M, 3]) fp32: batch item b of P and of Q are two
    independent noisy samples of the unit sphere."""
    P = np.stack([sphere_cloud(seed, 0, b, N, sigma) for b in range(Bt)]) if Bt else np.zeros((0, N, 3), np.float32)
    Q = np.stack([sphere_cloud(seed, 1, b, M, sigma) for b in range(Bt)]) if Bt else np.zeros((0, M, 3), np.float32)
    return P, Q


def make_chamfer(name, seed=0, **over):
    w = dict(CHAMFER_WORKLOADS[name])
    w.update({k: v for k, v in over.items() if v is not None})
    P, Q = point_clouds(seed, w["Bt"], w["N"], w["M"])
    return dict(name=name, P=P, Q=Q, **w)
