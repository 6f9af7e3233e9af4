"""Helpers of the parity tests: error bounds derived from the arithmetic, and the checks.

The bar: bit-exact for integer and index work.  For floating point an element passes when
|y_gpu - y_oracle| <= eps * M, M the oracle's sum of |terms| (M = 0 means exact), and eps is
derived below from how many roundings the kernel's arithmetic can put on a path.

Notation (Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed., section 3.1 and
chapter 4):
  u    unit roundoff: U32 = 2^-24 for binary32, U16 = 2^-8 for bfloat16 (8 significand bits),
       U16H = 2^-11 for binary16 (11 bits; below 2^-14 its spacing is 2^-24, an absolute error)
  g_k  gamma_k = k u / (1 - k u): k successive roundings give a relative error of at most g_k.
       A sum of n terms evaluated in ANY order (any binary tree of n leaves, depth <= n - 1)
       errs by at most g_{n-1} * sum |x_i|; a dot product of n terms, each product exact
       inside a fused multiply-add (or exact as bf16 x bf16 in fp32), by g_n * sum |x_i y_i|.
  (+)  composition: errors e1, e2 on a path compose to (1 + e1)(1 + e2) - 1.

Per-call bounds (both sides see the same inputs):
  pooling            g_{L-1}, L the longest bag (fp32 accumulation; bf16 rows widen exactly)
  dots, fp32         g_d (fused multiply-add chains and sums over d columns)
  dots, bf16 MFMA    g_d against the oracle's bf16-operand mode (products exact in fp32)
  dZ = S Z           g_F (F - 1 pair terms and the dense gradient); a bf16 store of dZ adds
                     U16 * |dZ| (store_bound)
  segment reduce     g_D, D the depth of the reduce-by-key tree (segreduce_depth), which
                     does not grow with a segment's length
  SGD store          sgd_store_bound: fl32(w - lr g) once (fp32 tables), then nearest-even
                     to bf16 or fp16 (16-bit tables: a double rounding), against the oracle's
                     single rounding of the exact value

Chained bounds (one step end to end against the oracle's own chain): each stage's input
error enters its output through the stage's arithmetic (linear stages pass it through, the
pair products take it from both factors) and composes with the stage's own roundings.
`step_bounds` writes these out.
"""
import numpy as np

RTOL_F32 = 1e-5          # the per-call figure for fp32 arithmetic
RTOL_BF16 = 1e-2         # the per-call figure for bf16 storage / bf16 operands
U32 = 2.0 ** -24
U16 = 2.0 ** -8
U16H = 2.0 ** -11        # binary16 (11 significant bits)


def gamma(k, u=U32):
    k = max(int(k), 0)
    return k * u / (1.0 - k * u)


def compose(*eps):
    r = 1.0
    for e in eps:
        r *= 1.0 + e
    return r - 1.0


def segreduce_depth(n, dim, bf16_grads):
    """Most roundings on any path of the backward's reduce-by-key tree over n sorted
    positions of rows of `dim` values.  A level sums a piece of at most KPS positions inside
    a slot (KPS - 1 additions), then joins at most (slots - 1) following pieces of the same
    row in order; the carries of a level form the next level's input, until one chunk of
    slots * KPS positions is left.  slots = 256 / G with G = 16-byte vectors per row rounded
    up to a power of two (at most 64): 4 fp32 values per vector, and at level 0 8 bf16
    gradient values per vector (when dim is a multiple of 8 and at most 512); KPS = 6 for
    bf16 gradient rows, 4 for fp32."""
    def pow2_lanes(vecs):
        G = 1
        while G < 64 and G < vecs:
            G *= 2
        return G
    vecs = max(1, int(dim) // 4)
    slots = 256 // pow2_lanes(vecs)
    slots0 = slots
    if bf16_grads and int(dim) % 8 == 0 and int(dim) // 8 <= 64:
        slots0 = 256 // pow2_lanes(int(dim) // 8)
    kps = 6 if bf16_grads else 4
    chunk = slots * kps
    depth = (kps - 1) + (slots0 - 1)
    blocks = -(-max(int(n), 1) // (slots0 * kps))
    while blocks > 1:
        blocks = -(-(2 * blocks) // chunk)
        depth += (kps - 1) + (slots - 1)
    return depth


LONG_BAG = 4096          # a longer bag is pooled in chunks of LONG_CHUNK occurrences
LONG_CHUNK = 4096


def long_bag_depth(L, dim, table):
    """Most roundings on a path of the pooled sum of a bag of L > LONG_BAG occurrences: a
    chunk's piece is split over the block's lane groups (256 / G of them, G = 16-byte vectors
    per row rounded up to a power of two, at most 64), each adding at most
    ceil(LONG_CHUNK / groups) rows in order, the groups joined pairwise (log2 groups), and the
    bag's chunk sums (at most ceil(L / LONG_CHUNK) + 1 pieces) added by a pairwise tree."""
    per = 4 if table == "f32" else 8
    vecs = max(1, int(dim) // per)
    G = 1
    while G < 64 and G < vecs:
        G *= 2
    groups = 256 // G
    share = -(-LONG_CHUNK // groups)
    pieces = -(-int(L) // LONG_CHUNK) + 1
    return (share - 1) + int(np.log2(groups)) + int(np.ceil(np.log2(pieces)))


def pool_eps(offsets, batch, num_tables, dim=None, table="f32"):
    """Per-bag bound of the pooled sums, shaped [batch, num_tables, 1]: g_{L-1} (the kernels
    add a bag's rows one after another within a share and join the shares' pieces in order,
    so no path has more than L - 1 roundings); with dim given, a bag longer than LONG_BAG
    gets g_D with D = long_bag_depth (its chunked tree)."""
    lens = np.diff(np.asarray(offsets, np.int64)).reshape(num_tables, batch).T
    k = np.maximum(lens - 1, 0).astype(np.float64)
    if dim is not None:
        for idx in zip(*np.nonzero(lens > LONG_BAG)):
            k[idx] = min(k[idx], long_bag_depth(lens[idx], dim, table))
    return (k * U32 / (1.0 - k * U32))[:, :, None]


def store_bound(want, mag, eps, store_bf16):
    """Element-wise bound of a value computed within eps * M in fp32 and stored as bf16
    (nearest-even: a further U16 of the stored value) or kept in fp32."""
    want = np.abs(np.asarray(want, np.float64))
    mag = np.asarray(mag, np.float64)
    if not store_bf16:
        return eps * mag
    return eps * mag * (1.0 + U16) + U16 * want


# Unit roundoff and half the subnormal spacing (the absolute error of a nearest rounding in
# the subnormal range) of the table storage types.
STORE_U = {"f32": U32, "bf16": U16, "f16": U16H}
STORE_ETA = {"f32": 0.0, "bf16": 0.0, "f16": 2.0 ** -25}


def sgd_store_bound(new, gmag, lr, eps_g, table):
    """Bound of |W'_gpu - W'_oracle| per element.  The oracle stores s1(x) with x = w - lr g
    exact and s1 one rounding to the table type; the kernel stores s2(fl32(w - lr g~)) with
    |g~ - g| <= eps_g * gmag (one fused multiply-add, then nearest-even for a 16-bit table).
    A rounding s to the table type errs by at most u|z| + eta (eta: binary16's subnormal
    range, where the spacing is 2^-24 whatever |z|).  table: "f32", "bf16", "f16" (or a bool,
    True for bf16)."""
    if isinstance(table, (bool, np.bool_)):
        table = "bf16" if table else "f32"
    u, eta = STORE_U[table], STORE_ETA[table]
    s1 = u
    s2 = U32 if table == "f32" else (u + U32 + u * U32)
    x = (np.abs(np.asarray(new, np.float64)) + eta) / (1.0 - s1)
    dg = float(lr) * eps_g * np.asarray(gmag, np.float64)
    return dg + s2 * (x + dg) + s1 * x + 2.0 * eta


def step_bounds(max_bag, dim, F, n, compute_bf16, grad_bf16):
    """Relative bounds (times the oracle's M) of one front-end step end to end:
      Z  the pooled vectors; R the interaction output; dZ its gradient (in fp32 before any
      bf16 store); g the row gradients (fp32; from bf16-stored dZ when grad_bf16)."""
    eZ = gamma(max_bag - 1)
    if compute_bf16:
        d = compose(U16, eZ)                           # a bf16 factor against the exact z
        eR = compose(d, d, gamma(dim))
        edZ = compose(U16, d, gamma(F))                # bf16 dP and bf16 z, F terms
    else:
        eR = compose(eZ, eZ, gamma(dim))
        edZ = compose(eZ, gamma(F))
    edZ_in = compose(edZ, U16) if grad_bf16 else edZ   # what the segment reduce reads
    eg = compose(edZ_in, gamma(segreduce_depth(n, dim, grad_bf16)))
    return {"Z": eZ, "R": eR, "dZ": edZ, "dZ_stored": edZ_in, "g": eg}


def _ratio(err, mag):
    m = np.asarray(mag, np.float64)
    return np.where(m > 0, err / np.where(m > 0, m, 1.0), np.where(err > 0, np.inf, 0.0))


def assert_close(got, want, mag, rtol, what=""):
    """|got - want| <= rtol * mag element-wise; prints the worst err/M against the bound."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    return assert_within(got, want, rtol * mag, what, mag=mag)


def assert_within(got, want, bound, what="", mag=None):
    """|got - want| <= bound element-wise (bound from the derivation above)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    bound = np.broadcast_to(np.asarray(bound, dtype=np.float64), want.shape)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite GPU values" % what
    err = np.abs(got - want)
    bad = err > bound
    used = float(np.max(_ratio(err, bound))) if err.size else 0.0
    if mag is not None and err.size:
        print("%s: worst err/M %.3g, bound/M %.3g (%.2f of the bound)" % (
            what, float(np.max(_ratio(err, mag))), float(np.max(_ratio(bound, mag))), used),
            flush=True)
    elif err.size:
        print("%s: %.2f of the bound at worst" % (what, used), flush=True)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d elements outside the bound (worst err/bound %.3g) at "
                             "%s: got %s want %s bound %s" % (
                                 what, int(bad.sum()), bad.size, used, idx.tolist(),
                                 got[tuple(idx[0])], want[tuple(idx[0])], bound[tuple(idx[0])]))
    return used


def worst_ratio(got, want, mag):
    err = np.abs(np.asarray(got, np.float64) - want)
    r = _ratio(err, mag)
    return float(r.max()) if r.size else 0.0
