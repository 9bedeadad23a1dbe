"""Error measures the GPU parity tests share.

The estimate's bar (the tolerance stated for the method's output): G_W
within relative Frobenius error 2e-3 for bf16 inputs with fp32 accumulation
and 1e-5 for the fp32 path.  The parity tests hold every stage output (the
clean loss L_t, the loss reductions rho, the credit r, the error estimate g)
to that relative level over the whole tensor, and each token on its own
(each row of G_W likewise):

  * whole tensor:  ||got - ref||_F / ||ref||_F <= TOL[dtype]
  * per row:       max over tokens t of ||got_t - ref_t|| / ||ref_t||
                   <= ROW_TOL[dtype]   (rows of G_W: max over channels c)

The per-row form is the one that catches a single wrong token, a wrong tail
quad or a wrong sequence, which the whole-tensor norm dilutes.  A row's
error is measured against the larger of its own norm and ROW_FLOOR (1%) of
the root-mean-square row norm: an fp32 sum rounds in proportion to the
magnitudes of its terms, not to its value, so a row whose terms nearly
cancel (a single-element row of G_W when d_in = 1, say) would otherwise
show its rounding at any relative size, while a wrong row is still off by
about the typical row norm and fails by a wide margin.  A tensor whose
reference is exactly zero is compared in absolute terms.

The per-row bar of the fp32 path is not the whole-tensor 1e-5: one token's
value is a handful of fp32 sums, and an fp32 sum of n terms can be off by up
to about n u relative to the sum of the terms' magnitudes (u = 2^-24, the
unit roundoff); over a whole tensor those per-token rounding errors average
out, token by token they do not.  A token whose value is small next to its
terms (a near-zero cross-entropy of a confident head, whose logits carry
absolute rounding of d_in u |x w|; a loss reduction that nearly cancels)
shows its terms' rounding at full size.  ROW_TOL["f32"] = 1e-4 is n u for
n of about 1,700 terms, the length of the longest fp32 sums the fp32 test
shapes form per token (vocabulary columns plus draws, or channels plus
draws).  The bf16 path's bar, 2e-3, already exceeds that bound at every
size tested and is used for rows unchanged.
"""
import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-3}
ROW_TOL = {"f32": 1e-4, "bf16": 2e-3}
ROW_FLOOR = 0.01


def rel(a, b):
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def rows_rel(a, b):
    """Largest per-row relative error (rows along the first axis; each row
    against the larger of its norm and ROW_FLOOR of the RMS row norm) and the
    row where it occurs."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if a.ndim == 1:
        a, b = a[:, None], b[:, None]
    a = a.reshape(a.shape[0], -1)
    b = b.reshape(b.shape[0], -1)
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    floor = ROW_FLOOR * float(np.sqrt(np.mean(den ** 2))) if den.size else 0.0
    den = np.maximum(den, floor)
    err = num / np.where(den > 0, den, 1.0)
    i = int(np.argmax(err)) if err.size else 0
    return (float(err[i]) if err.size else 0.0), i


def stage_errors(got, ref, keys=("loss", "rho", "reward", "g"), g_key="G_W", ref_g_key="G",
                 token_slice=None):
    """Whole and per-row errors of the stage outputs present in `got` (the
    GPU's, fp64 arrays) against the oracle's `ref`; `token_slice` selects the
    tokens of `got` that `ref` covers."""
    errs = {}
    for k in keys:
        if k not in got or k not in ref:
            continue
        a = got[k] if token_slice is None else got[k][token_slice]
        errs[k] = rel(a, ref[k])
        errs[k + "_row"], _ = rows_rel(a, ref[k])
    if g_key in got and ref_g_key in ref:
        errs[g_key] = rel(got[g_key], ref[ref_g_key])
        errs[g_key + "_row"], _ = rows_rel(got[g_key], ref[ref_g_key])
    return errs


def report(name, errs):
    print(name, " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)


def assert_within(errs, dtype):
    """Every error of `errs` within its bar: ROW_TOL for the per-row entries
    (keys ending in "_row"), TOL for the rest."""
    bad = {k: v for k, v in errs.items()
           if not v <= (ROW_TOL if k.endswith("_row") else TOL)[dtype]}
    assert not bad, (bad, dtype, TOL[dtype], ROW_TOL[dtype])
