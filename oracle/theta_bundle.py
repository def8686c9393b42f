"""Float64 CPU oracle for the theta-bundle projection.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library (no kernels, headers, helpers or constants) and imports nothing from
the ``rank_factored_linear_amd`` package.

Every function is the plain definition of what the method computes, written in
float64 NumPy so that a reader can check it against the pages by eye.  Sources
(the pages are cited by title and section):

* "Banded sharing" (attnquant docs), section "How layers map to bands":
  layers are split into G contiguous bands, as equal in size as possible, with
  the earlier bands taking the remainder.
* "The theta bundle" (weightless docs), component table: W0 [out, in] shared
  per family (per band), s [out], U [out, rank], V [in, rank] per layer; and
  the reconstruction formula weight = diag(s) W0 + U V^T.
* "The theta bundle", section "Analytic decomposition": W0 is the mean of the
  band's matrices, s is the per-row least-squares fit against W0, and the
  residual weight - diag(s) W0 is cut to the requested rank by a truncated SVD
  whose singular values are absorbed into U; rank 0 means no delta.
  The randomized SVD the same section names for large matrices (Halko et
  al., 2009) is randomized_factors, for a caller-drawn probe.
* "Quality" (attnquant docs), section "Reconstruction error": the relative
  Frobenius error of the rebuilt weight against the true weight, averaged over
  layers and projection families.

Readings of points the pages leave open are stated where they are used.
Every function here is pinned by ``tests/test_oracle.py`` against closed
forms, library routines, invariants or brute force; none is parity unpinned.
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Band map  ("Banded sharing", section "How layers map to bands")
# ---------------------------------------------------------------------------


def band_sizes(num_layers: int, num_bands: int) -> list[int]:
    """Sizes of the G contiguous bands, earliest band first.

    The bands are as equal as possible; the remainder of num_layers / G goes
    one layer at a time to the earliest bands.  This is built by dealing the
    layers out one by one rather than by a closed formula, so that it reads as
    the sentence on the page.
    """
    _check_band_args(num_layers, num_bands)
    base = num_layers // num_bands          # every band gets at least this many
    sizes = [base] * num_bands
    leftover = num_layers - base * num_bands
    band = 0
    while leftover > 0:                     # earlier bands take the remainder
        sizes[band] += 1
        leftover -= 1
        band += 1
    return sizes


def band_map(num_layers: int, num_bands: int) -> list[int]:
    """Band of every layer 0..num_layers-1, walking the bands in order."""
    out = []
    for band, size in enumerate(band_sizes(num_layers, num_bands)):
        out.extend([band] * size)
    return out


def band_index(num_layers: int, num_bands: int, layer: int) -> int:
    """Band of one layer (the model config's band_index())."""
    if not (0 <= layer < num_layers):
        raise ValueError(f"layer {layer} outside [0, {num_layers})")
    return band_map(num_layers, num_bands)[layer]


def _check_band_args(num_layers: int, num_bands: int) -> None:
    # Reading: G ranges from 1 (full sharing) to num_layers (passthrough);
    # the page names these two ends and nothing outside them.
    if num_layers < 1:
        raise ValueError("num_layers must be >= 1")
    if not (1 <= num_bands <= num_layers):
        raise ValueError(f"num_bands {num_bands} outside [1, {num_layers}]")


# ---------------------------------------------------------------------------
# bfloat16 storage decoding (exact)
# ---------------------------------------------------------------------------


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 numbers given as their 16-bit patterns.

    A bfloat16 is the top half of an IEEE binary32, so the pattern shifted
    left by 16 bits is the binary32 with the same value; binary32 -> binary64
    is exact.
    """
    b = np.ascontiguousarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Reconstruction and the projection  ("The theta bundle", component table)
# ---------------------------------------------------------------------------


def reconstruct_weight(s: np.ndarray, W0: np.ndarray, U: np.ndarray, V: np.ndarray) -> np.ndarray:
    """weight = diag(s) . W0 + U . V^T   (reconstruct_weight(s, W0, U, V)).

    s scales the rows of W0 (one entry per output feature).  U is [out, rank]
    and V is [in, rank]; with rank 0 the product is the zero matrix.
    """
    s, W0, U, V = (np.asarray(a, dtype=np.float64) for a in (s, W0, U, V))
    _check_bundle(s, W0, U, V)
    return np.diag(s) @ W0 + U @ V.T


def forward(x: np.ndarray, s: np.ndarray, W0: np.ndarray, U: np.ndarray, V: np.ndarray) -> np.ndarray:
    """y = x . weight^T computed from the bundle without forming weight.

    Transposing the reconstruction formula gives
        y = (x . W0^T) . diag(s) + (x . V) . U^T,
    i.e. the output column o of x . W0^T is scaled by s[o] and the rank-r
    correction (x . V) . U^T is added.  x is [tokens, in]; y is [tokens, out].
    """
    x, s, W0, U, V = (np.asarray(a, dtype=np.float64) for a in (x, s, W0, U, V))
    _check_bundle(s, W0, U, V)
    if x.ndim != 2 or x.shape[1] != W0.shape[1]:
        raise ValueError("x must be [tokens, in_dim]")
    main = (x @ W0.T) @ np.diag(s)
    delta = (x @ V) @ U.T
    return main + delta


def forward_dense(x: np.ndarray, weight: np.ndarray) -> np.ndarray:
    """The ordinary linear layer y = x . weight^T."""
    return np.asarray(x, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T


def _check_bundle(s, W0, U, V) -> None:
    if W0.ndim != 2:
        raise ValueError("W0 must be [out_dim, in_dim]")
    out_dim, in_dim = W0.shape
    if s.shape != (out_dim,):
        raise ValueError("s must be [out_dim]")
    if U.ndim != 2 or V.ndim != 2 or U.shape[0] != out_dim or V.shape[0] != in_dim or U.shape[1] != V.shape[1]:
        raise ValueError("U must be [out_dim, rank] and V [in_dim, rank]")


# ---------------------------------------------------------------------------
# Error measure  ("Quality", section "Reconstruction error")
# ---------------------------------------------------------------------------


def relative_frobenius_error(original: np.ndarray, reconstructed: np.ndarray) -> float:
    """||original - reconstructed||_F / ||original||_F.

    The norm of the true weight is the denominator.  Reading for the 0/0 case
    the pages leave open: 0 when the two are equal (including both zero),
    +inf when original is zero and reconstructed is not.
    """
    a = np.asarray(original, dtype=np.float64)
    b = np.asarray(reconstructed, dtype=np.float64)
    if a.shape != b.shape:
        raise ValueError("shapes differ")
    num = np.sqrt(np.sum((a - b) ** 2))
    den = np.sqrt(np.sum(a ** 2))
    if num == 0.0:
        return 0.0
    if den == 0.0:
        return float("inf")
    return float(num / den)


def mean_error(errors) -> float:
    """Unweighted mean of per-(layer, family) errors (the averaged figure)."""
    errors = list(errors)
    if not errors:
        raise ValueError("no errors to average")
    return float(sum(errors) / len(errors))


# ---------------------------------------------------------------------------
# Closed-form decomposition  ("The theta bundle", "Analytic decomposition")
# ---------------------------------------------------------------------------


def shared_block(weights) -> np.ndarray:
    """W0 of one band: the arithmetic mean of the band's weight matrices.

    Reading: summed in layer order in float64, then divided by the count.
    """
    weights = [np.asarray(w, dtype=np.float64) for w in weights]
    if not weights:
        raise ValueError("empty band")
    total = np.zeros_like(weights[0])
    for w in weights:
        total = total + w
    return total / len(weights)


def row_scale(weight: np.ndarray, W0: np.ndarray) -> np.ndarray:
    """Per-output-row least-squares scale: s[o] = <w_o, w0_o> / <w0_o, w0_o>.

    s[o] minimises ||weight[o, :] - s[o] * W0[o, :]||.  Reading for a zero row
    of W0 (0/0, not covered by the pages): the minimum-norm solution s[o] = 0,
    so the residual keeps the whole row.
    """
    weight = np.asarray(weight, dtype=np.float64)
    W0 = np.asarray(W0, dtype=np.float64)
    out_dim = W0.shape[0]
    s = np.zeros(out_dim)
    for o in range(out_dim):
        den = float(np.dot(W0[o], W0[o]))
        if den != 0.0:
            s[o] = float(np.dot(weight[o], W0[o])) / den
    return s


def truncated_factors(residual: np.ndarray, rank: int) -> tuple[np.ndarray, np.ndarray]:
    """U [out, rank], V [in, rank] with U V^T the best rank-r approximation.

    From the thin SVD residual = P diag(sigma) Q^T: U = P[:, :r] diag(sigma[:r])
    (U absorbs the singular values) and V = Q[:, :r].  Rank 0 gives empty
    factors.  Reading: the exact LAPACK SVD is used at every size; the
    randomized SVD the page mentions for large matrices approximates this
    optimum.
    """
    residual = np.asarray(residual, dtype=np.float64)
    out_dim, in_dim = residual.shape
    if rank < 0 or rank > min(out_dim, in_dim):
        raise ValueError(f"rank {rank} outside [0, {min(out_dim, in_dim)}]")
    if rank == 0:
        return np.zeros((out_dim, 0)), np.zeros((in_dim, 0))
    P, sigma, Qt = np.linalg.svd(residual, full_matrices=False)
    U = P[:, :rank] * sigma[:rank][None, :]
    V = Qt[:rank, :].T
    return U, V


def orthonormal_basis(Y: np.ndarray) -> np.ndarray:
    """Orthonormal basis of the columns of Y (reduced QR, a library step)."""
    return np.linalg.qr(np.asarray(Y, dtype=np.float64), mode="reduced")[0]


def randomized_factors(residual: np.ndarray, rank: int, omega: np.ndarray, power_iters: int) -> tuple[np.ndarray, np.ndarray]:
    """U [out, rank], V [in, rank] by the randomized SVD the page names for large
    matrices ("The theta bundle", "Low-rank residual": Halko, Martinsson and
    Tropp, 2009): a randomized range finder with power iterations, then the
    exact SVD of the small projected matrix.

    omega [in, k] is the random probe, k = rank + oversampling, drawn by the
    caller so that every implementation can be run on the same draw.
      1. Q = orthonormal basis of residual . omega  (k columns).
      2. power_iters times: Q' = basis of residual^T . Q, then
         Q = basis of residual . Q'.  Re-orthonormalising at every half step
         keeps the weaker directions that plain powers would round away.
      3. B = Q^T . residual (k x in), B = P diag(sigma) Qt (exact SVD).
      4. U = Q . P[:, :rank] . diag(sigma[:rank]), V = Qt[:rank]^T: U absorbs the
         singular values, as in truncated_factors.
    Readings (the page states neither): the oversampling and the number of
    power iterations are parameters; the GPU bundle path uses k = rank + 16
    and two power iterations.  With k >= min(out, in), or a residual of rank
    <= k, the probe covers the whole column space and the result is the exact
    truncated SVD.
    """
    R = np.asarray(residual, dtype=np.float64)
    omega = np.asarray(omega, dtype=np.float64)
    out_dim, in_dim = R.shape
    if omega.ndim != 2 or omega.shape[0] != in_dim or omega.shape[1] < rank:
        raise ValueError("omega must be [in_dim, k] with k >= rank")
    if rank < 0 or rank > min(out_dim, in_dim) or power_iters < 0:
        raise ValueError("rank or power_iters out of range")
    if rank == 0:
        return np.zeros((out_dim, 0)), np.zeros((in_dim, 0))
    Q = orthonormal_basis(R @ omega)
    for _ in range(power_iters):
        Qp = orthonormal_basis(R.T @ Q)
        Q = orthonormal_basis(R @ Qp)
    B = Q.T @ R
    P, sigma, Qt = np.linalg.svd(B, full_matrices=False)
    U = Q @ (P[:, :rank] * sigma[:rank][None, :])
    V = Qt[:rank, :].T
    return U, V


def decompose(weights, num_bands: int, rank: int) -> dict:
    """Decompose one family's per-layer weights into its theta bundle.

    Returns {"W0": [G arrays], "band": [band per layer], "s", "U", "V": [per
    layer arrays]}.  For each band: W0 = mean of its layers; for each layer:
    s by per-row least squares against its band's W0, then the truncated SVD
    of weight - diag(s) W0.
    """
    weights = [np.asarray(w, dtype=np.float64) for w in weights]
    num_layers = len(weights)
    bands = band_map(num_layers, num_bands)
    W0 = []
    for b in range(num_bands):
        W0.append(shared_block([weights[l] for l in range(num_layers) if bands[l] == b]))
    out = {"W0": W0, "band": bands, "s": [], "U": [], "V": []}
    for l, w in enumerate(weights):
        w0 = W0[bands[l]]
        s = row_scale(w, w0)
        residual = w - np.diag(s) @ w0
        U, V = truncated_factors(residual, rank)
        out["s"].append(s)
        out["U"].append(U)
        out["V"].append(V)
    return out


# The seven projection families of a decoder layer ("The theta bundle",
# section "Projection families"): four attention projections, three MLP.
ATTENTION_FAMILIES = ("q_proj", "k_proj", "v_proj", "o_proj")
MLP_FAMILIES = ("gate_proj", "up_proj", "down_proj")


def decompose_model(weights_by_family: dict, num_bands: int, rank: int, tie_families: str = "all") -> dict:
    """Theta bundles for the projection families of a model ("The theta
    bundle", section "Projection families").

    weights_by_family maps a family name to its per-layer weights.  With
    tie_families="all" every family is decomposed (decompose, per family).
    With tie_families="attn" only the attention families are; the MLP
    families stay plain dense layers holding their own weights.  Reading (the
    page gives no bundle for them): a dense layer is written as the bundle in
    which each layer is its own band (W0 = its weight), s = 1 and rank 0, so
    that reconstruct_weight gives the weight back exactly.
    """
    if tie_families not in ("all", "attn"):
        raise ValueError(f"tie_families must be 'all' or 'attn', not {tie_families!r}")
    out = {}
    for fam, weights in weights_by_family.items():
        if fam not in ATTENTION_FAMILIES + MLP_FAMILIES:
            raise ValueError(f"unknown projection family {fam!r}")
        if tie_families == "attn" and fam in MLP_FAMILIES:
            ws = [np.asarray(w, dtype=np.float64) for w in weights]
            out[fam] = {"W0": ws, "band": list(range(len(ws))),
                        "s": [np.ones(w.shape[0]) for w in ws],
                        "U": [np.zeros((w.shape[0], 0)) for w in ws],
                        "V": [np.zeros((w.shape[1], 0)) for w in ws]}
        else:
            out[fam] = decompose(weights, num_bands, rank)
    return out


def refine_shared_block(weights, s_list, U_list, V_list, W0_prev: np.ndarray) -> np.ndarray:
    """One least-squares update of a band's shared block with the per-layer
    scale and delta held fixed: the alternating least squares the "Quality"
    page reports on (Research: why shared configurations need training).

    W0 minimises sum_l ||W_l - diag(s_l) W0 - U_l V_l^T||_F^2 over the band's
    layers; row by row the minimiser is
        W0[o] = sum_l s_l[o] (W_l - U_l V_l^T)[o] / sum_l s_l[o]^2.
    Reading (not on the pages): a row whose scales are all zero has no least-
    squares information and keeps its previous value.
    """
    W0_prev = np.asarray(W0_prev, dtype=np.float64)
    num = np.zeros_like(W0_prev)
    den = np.zeros(W0_prev.shape[0])
    for w, sl, U, V in zip(weights, s_list, U_list, V_list):
        w, sl, U, V = (np.asarray(a, dtype=np.float64) for a in (w, sl, U, V))
        num += sl[:, None] * (w - U @ V.T)
        den += sl * sl
    out = W0_prev.copy()
    rows = den != 0.0
    out[rows] = num[rows] / den[rows][:, None]
    return out


def als_decompose(weights, num_bands: int, rank: int, iters: int) -> dict:
    """The analytic decomposition followed by `iters` rounds of alternating
    least squares: each round refits every band's W0 with s, U, V fixed
    (refine_shared_block), then every layer's s and U, V against the new W0
    exactly as the analytic decomposition does (row_scale, truncated_factors)."""
    weights = [np.asarray(w, dtype=np.float64) for w in weights]
    bun = decompose(weights, num_bands, rank)
    bands = bun["band"]
    for _ in range(iters):
        for b in range(num_bands):
            members = [l for l in range(len(weights)) if bands[l] == b]
            bun["W0"][b] = refine_shared_block([weights[l] for l in members], [bun["s"][l] for l in members],
                                               [bun["U"][l] for l in members], [bun["V"][l] for l in members],
                                               bun["W0"][b])
        for l, w in enumerate(weights):
            w0 = bun["W0"][bands[l]]
            s = row_scale(w, w0)
            U, V = truncated_factors(w - np.diag(s) @ w0, rank)
            bun["s"][l], bun["U"][l], bun["V"][l] = s, U, V
    return bun


def decomposition_error(weights, bundle: dict) -> list[float]:
    """Per-layer relative Frobenius error of the rebuilt weights."""
    errs = []
    for l, w in enumerate(weights):
        rebuilt = reconstruct_weight(bundle["s"][l], bundle["W0"][bundle["band"][l]], bundle["U"][l], bundle["V"][l])
        errs.append(relative_frobenius_error(w, rebuilt))
    return errs
