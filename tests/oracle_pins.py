"""Pins for the CPU oracle: checks against what mathematics and independent
libraries fix, never against the oracle itself.

Each ``pin_*`` function raises ``AssertionError`` when the oracle (or a build
of it with a planted mistake, selected by ``mutation``) disagrees with:
  * numpy's float16 conversions and float32 bit views (independent decoders),
  * the IEEE round-to-nearest-even rule checked on the format grid directly,
  * exact rational arithmetic (``fractions.Fraction``) on tiny shapes,
  * exact integer products, identities, permutations and closed forms,
  * the hand-worked fixtures under ``tests/golden/``.
"""
from __future__ import annotations

import bisect
import json
import os
from fractions import Fraction

import numpy as np

import oracle
from dense_half_precision_amd import inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# --------------------------------------------------------------------------
# Independent decoders and a rational round-to-nearest-even on the grid.
# --------------------------------------------------------------------------
def lib_decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    with np.errstate(invalid="ignore"):  # NaN payloads
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


class Grid:
    """All finite values of a 16-bit format, sorted, with their bit patterns."""

    def __init__(self, dtype: str):
        allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
        vals = lib_decode(allbits, dtype)
        keep = np.isfinite(vals) & (allbits < 0x8000)  # non-negative half; sign handled apart
        vb = sorted(zip(vals[keep].tolist(), allbits[keep].tolist()))
        self.vals = [Fraction(v) for v, _ in vb]
        self.bits = [b for _, b in vb]
        self.maxf = self.vals[-1]
        self.dtype = dtype
        # spacing above the largest finite value, for the overflow threshold
        self.top_ulp = self.vals[-1] - self.vals[-2]
        self.inf_bits = 0x7C00 if dtype == "f16" else 0x7F80

    def round(self, q: Fraction) -> int:
        """RNE of an exact rational, as bits (+0 for zero, -0 kept for -tiny)."""
        neg = q < 0
        a = -q if neg else q
        if a >= self.maxf + self.top_ulp / 2:
            b = self.inf_bits
        else:
            i = bisect.bisect_left(self.vals, a)
            if i < len(self.vals) and self.vals[i] == a:
                b = self.bits[i]
            else:
                lo_v, lo_b = self.vals[i - 1], self.bits[i - 1]
                if i >= len(self.vals):
                    b = lo_b
                else:
                    hi_v, hi_b = self.vals[i], self.bits[i]
                    dl, dh = a - lo_v, hi_v - a
                    if dl < dh:
                        b = lo_b
                    elif dh < dl:
                        b = hi_b
                    else:  # tie: the neighbour whose last significand bit is 0
                        b = lo_b if (lo_b & 1) == 0 else hi_b
            # the grid above holds non-negative values; -0 has bits 0x8000
        if neg:
            b |= 0x8000
        return b


_GRIDS: dict[str, Grid] = {}


def grid(dtype: str) -> Grid:
    if dtype not in _GRIDS:
        _GRIDS[dtype] = Grid(dtype)
    return _GRIDS[dtype]


def exact_gemm(layout: str, dtype: str, A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Exact rational GEMM rounded once to the dtype: a second, independent
    implementation of the definition, for tiny shapes only."""
    Av = [[Fraction(x) for x in row] for row in lib_decode(A, dtype).tolist()]
    Bv = lib_decode(B, dtype)
    Bop = Bv.T if layout == "tn" else Bv
    Bc = [[Fraction(x) for x in col] for col in Bop.T.tolist()]  # columns of Bop
    g = grid(dtype)
    M, N = len(Av), len(Bc)
    out = np.zeros((M, N), dtype=np.uint16)
    for m in range(M):
        for n in range(N):
            s = sum((a * b for a, b in zip(Av[m], Bc[n])), Fraction(0))
            out[m, n] = g.round(s)
    return out


def same_bits(x: np.ndarray, y: np.ndarray, what: str):
    x = np.asarray(x, dtype=np.uint16)
    y = np.asarray(y, dtype=np.uint16)
    assert x.shape == y.shape, f"{what}: shape {x.shape} vs {y.shape}"
    bad = np.argwhere(x != y)
    assert bad.size == 0, (f"{what}: {len(bad)} mismatches, first at {tuple(bad[0])}: "
                           f"{x[tuple(bad[0])]:#06x} vs {y[tuple(bad[0])]:#06x}")


# --------------------------------------------------------------------------
# Rounding / decoding pins.
# --------------------------------------------------------------------------
def pin_decode_exhaustive(mutation: int = 0):
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    for dt in ("f16", "bf16"):
        got = oracle.decode(allbits, dt, mutation=mutation)
        ref = lib_decode(allbits, dt)
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan), f"{dt}: NaN set differs"
        assert np.array_equal(got[~nan], ref[~nan]), f"{dt}: decoded values differ"
        # signed zeros
        assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), f"{dt}: zero sign"


def _finite_sorted(dtype):
    g = grid(dtype)
    return np.array([float(v) for v in g.vals]), np.array(g.bits, dtype=np.uint16)


def pin_round_representable(mutation: int = 0):
    """Every finite value rounds to itself (both signs)."""
    for dt in ("f16", "bf16"):
        vals, bits = _finite_sorted(dt)
        same_bits(oracle.round_to(vals, dt, mutation=mutation), bits, f"{dt} identity")
        nz = vals != 0
        same_bits(oracle.round_to(-vals[nz], dt, mutation=mutation), bits[nz] | 0x8000,
                  f"{dt} identity (negative)")


def pin_round_midpoints(mutation: int = 0):
    """Midpoints go to the even neighbour; a nudge either way goes to the
    nearer one.  Checked on the format grid (the rule itself), and for f16
    also against numpy's float64 -> float16 conversion."""
    for dt in ("f16", "bf16"):
        vals, bits = _finite_sorted(dt)
        lo, hi = vals[:-1], vals[1:]
        mid = (lo + hi) / 2  # exact in float64: at most 12 significant bits
        even = np.where((bits[:-1] & 1) == 0, bits[:-1], bits[1:])
        got = oracle.round_to(mid, dt, mutation=mutation)
        same_bits(got, even, f"{dt} ties-to-even")
        same_bits(oracle.round_to(np.nextafter(mid, -np.inf), dt, mutation=mutation), bits[:-1],
                  f"{dt} just below midpoint")
        same_bits(oracle.round_to(np.nextafter(mid, np.inf), dt, mutation=mutation), bits[1:],
                  f"{dt} just above midpoint")
        # negative side is the mirror image
        same_bits(oracle.round_to(-mid, dt, mutation=mutation), even | 0x8000, f"{dt} -ties")
        if dt == "f16":
            with np.errstate(over="ignore"):
                for x in (mid, np.nextafter(mid, -np.inf), np.nextafter(mid, np.inf)):
                    same_bits(oracle.round_to(x, dt, mutation=mutation),
                              x.astype(np.float16).view(np.uint16), "f16 vs numpy")
        else:
            # bfloat16 midpoints and their float32 neighbours are float32-exact;
            # torch's CPU float32 -> bfloat16 cast is an independent RNE.
            import torch
            m32 = mid.astype(np.float32)
            assert np.array_equal(m32.astype(np.float64), mid)
            for x in (m32, np.nextafter(m32, np.float32(-np.inf)), np.nextafter(m32, np.float32(np.inf))):
                tb = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy()
                same_bits(oracle.round_to(x.astype(np.float64), dt, mutation=mutation),
                          tb.view(np.uint16), "bf16 vs torch")


def pin_round_random(mutation: int = 0):
    """Random doubles across the whole range vs numpy (f16) and vs the grid
    rule (bf16, via exact rationals)."""
    g = np.random.Generator(np.random.PCG64(7))
    x = g.standard_normal(200000) * np.exp2(g.integers(-30, 20, 200000))
    with np.errstate(over="ignore"):
        ref16 = x.astype(np.float16).view(np.uint16)
    same_bits(oracle.round_to(x, "f16", mutation=mutation), ref16, "f16 random vs numpy")
    xb = g.standard_normal(3000) * np.exp2(g.integers(-140, 130, 3000))
    gb = grid("bf16")
    ref = np.array([gb.round(Fraction(v)) for v in xb.tolist()], dtype=np.uint16)
    same_bits(oracle.round_to(xb, "bf16", mutation=mutation), ref, "bf16 random vs grid")


def pin_round_special(mutation: int = 0):
    """Overflow thresholds, subnormal boundaries, inf and NaN."""
    cases_f16 = [
        (65504.0, 0x7BFF), (65519.0, 0x7BFF), (65520.0, 0x7C00), (1e6, 0x7C00),
        (-65520.0, 0xFC00), (2.0**-24, 0x0001), (2.0**-25, 0x0000),
        (np.nextafter(2.0**-25, 1.0), 0x0001), (3 * 2.0**-25, 0x0002), (2.0**-14, 0x0400),
        (np.inf, 0x7C00), (-np.inf, 0xFC00), (0.0, 0x0000), (-0.0, 0x8000),
        (1.0 + 2.0**-11, 0x3C00), (1.0 + 3 * 2.0**-11, 0x3C02),
    ]
    maxbf = float.fromhex("0x1.fep127")
    cases_bf16 = [
        (maxbf, 0x7F7F), (float.fromhex("0x1.ffp127"), 0x7F80),
        (np.nextafter(float.fromhex("0x1.ffp127"), 0.0), 0x7F7F),
        (2.0**-133, 0x0001), (2.0**-134, 0x0000), (2.0**-126, 0x0080),
        (1.0 + 2.0**-8, 0x3F80), (1.0 + 3 * 2.0**-8, 0x3F82), (-np.inf, 0xFF80),
    ]
    for dt, cases in (("f16", cases_f16), ("bf16", cases_bf16)):
        x = np.array([c[0] for c in cases], dtype=np.float64)
        want = np.array([c[1] for c in cases], dtype=np.uint16)
        same_bits(oracle.round_to(x, dt, mutation=mutation), want, f"{dt} special values")
    for dt, nanbits in (("f16", 0x7E00), ("bf16", 0x7FC0)):
        r = oracle.round_to(np.array([np.nan]), dt, mutation=mutation)
        assert lib_decode(r, dt)[0] != lib_decode(r, dt)[0], f"{dt}: NaN must stay NaN"
        assert r[0] == nanbits


# --------------------------------------------------------------------------
# GEMM pins.
# --------------------------------------------------------------------------
TINY_SHAPES = [(1, 1, 1), (2, 3, 5), (3, 2, 8), (5, 8, 3), (8, 16, 17), (17, 5, 33), (16, 33, 16)]


def pin_gemm_bruteforce(mutation: int = 0):
    """Tiny shapes vs exact rational arithmetic, both layouts and dtypes."""
    for dt in ("f16", "bf16"):
        for layout in ("tn", "nn"):
            for s, (M, N, K) in enumerate(TINY_SHAPES):
                A = inputs.draw((M, K), dt, "normal", 50 + s)
                B = inputs.draw((N, K) if layout == "tn" else (K, N), dt, "normal", 80 + s)
                same_bits(oracle.hgemm(layout, dt, A, B, mutation=mutation),
                          exact_gemm(layout, dt, A, B), f"brute force {dt} {layout} {M}x{N}x{K}")


def _bits_of(vals: np.ndarray, dtype: str) -> np.ndarray:
    v = np.asarray(vals, dtype=np.float64)
    if dtype == "f16":
        return v.astype(np.float16).view(np.uint16)
    return inputs.f32_to_bf16_bits(v.astype(np.float32))


def pin_gemm_small_integers(mutation: int = 0):
    """Integer entries whose products and sums are exact: C must equal the
    int64 matmul exactly (f16: |entries| <= 2, K <= 512 gives |C| <= 2048;
    bf16: entries in {-1,0,1}, K <= 256)."""
    g = np.random.Generator(np.random.PCG64(11))
    for dt, hi, shapes in (("f16", 2, [(7, 9, 512), (33, 17, 100)]),
                           ("bf16", 1, [(9, 7, 256), (17, 33, 64)])):
        for layout in ("tn", "nn"):
            for M, N, K in shapes:
                Ai = g.integers(-hi, hi + 1, size=(M, K))
                Bi = g.integers(-hi, hi + 1, size=(K, N))
                Bst = Bi.T.copy() if layout == "tn" else Bi
                want = _bits_of(Ai @ Bi, dt)
                got = oracle.hgemm(layout, dt, _bits_of(Ai, dt), _bits_of(Bst, dt), mutation=mutation)
                same_bits(got, want, f"small integers {dt} {layout} {M}x{N}x{K}")


def pin_gemm_identity_permutation(mutation: int = 0):
    """A = I gives C = Bop exactly; a permutation P gives the permuted rows."""
    g = np.random.Generator(np.random.PCG64(12))
    for dt in ("f16", "bf16"):
        for layout in ("tn", "nn"):
            K, N = 24, 40
            Bop_bits = inputs.draw((K, N), dt, "normal", 99)
            Bst = Bop_bits.T.copy() if layout == "tn" else Bop_bits
            eye = _bits_of(np.eye(K), dt)
            same_bits(oracle.hgemm(layout, dt, eye, Bst, mutation=mutation), Bop_bits,
                      f"identity {dt} {layout}")
            perm = g.permutation(K)
            P = np.zeros((K, K))
            P[np.arange(K), perm] = 1.0
            same_bits(oracle.hgemm(layout, dt, _bits_of(P, dt), Bst, mutation=mutation),
                      Bop_bits[perm], f"permutation {dt} {layout}")


def pin_gemm_closed_forms(mutation: int = 0):
    """All-ones (C = K) and rank-1 dyadic (C = RNE(K * u_m * v_n))."""
    for dt, Ks in (("f16", (1, 7, 64, 2048)), ("bf16", (1, 7, 64, 256))):
        for layout in ("tn", "nn"):
            for K in Ks:
                M, N = 5, 8
                A = _bits_of(np.ones((M, K)), dt)
                B = _bits_of(np.ones((N, K) if layout == "tn" else (K, N)), dt)
                same_bits(oracle.hgemm(layout, dt, A, B, mutation=mutation),
                          _bits_of(np.full((M, N), float(K)), dt), f"all-ones {dt} {layout} K={K}")
    g = np.random.Generator(np.random.PCG64(13))
    for layout in ("tn", "nn"):
        M, N, K = 6, 10, 48
        u = g.integers(-64, 65, size=M) / 64.0
        v = g.integers(-64, 65, size=N) / 128.0
        Aop = np.repeat(u[:, None], K, axis=1)
        Bop = np.repeat(v[None, :], K, axis=0)
        Bst = Bop.T.copy() if layout == "tn" else Bop
        want = (K * np.outer(u, v)).astype(np.float16).view(np.uint16)  # numpy RNE
        same_bits(oracle.hgemm(layout, "f16", _bits_of(Aop, "f16"), _bits_of(Bst, "f16"),
                               mutation=mutation), want, f"rank-1 f16 {layout}")


def pin_gemm_ties(mutation: int = 0):
    """Sums that land exactly on a midpoint of the output grid."""
    # f16: 1 + 2^-11 is halfway between 1 and 1 + 2^-10 -> 1 (even);
    #      1 + 3*2^-11 is halfway between 1+2^-10 and 1+2^-9 -> 1+2^-9 (even).
    for layout in ("tn", "nn"):
        A = _bits_of(np.array([[1.0, 2.0**-11], [1.0, 3 * 2.0**-11]]), "f16")
        Bop = _bits_of(np.array([[1.0], [1.0]]), "f16")
        Bst = Bop.T.copy() if layout == "tn" else Bop
        want = _bits_of(np.array([[1.0], [1.0 + 2.0**-9]]), "f16")
        same_bits(oracle.hgemm(layout, "f16", A, Bst, mutation=mutation), want, f"f16 ties {layout}")
        Ab = _bits_of(np.array([[1.0, 2.0**-8], [1.0, 3 * 2.0**-8]]), "bf16")
        Bb = _bits_of(np.array([[1.0], [1.0]]), "bf16")
        Bbs = Bb.T.copy() if layout == "tn" else Bb
        wantb = _bits_of(np.array([[1.0], [1.0 + 2.0**-6]]), "bf16")
        same_bits(oracle.hgemm(layout, "bf16", Ab, Bbs, mutation=mutation), wantb,
                  f"bf16 ties {layout}")


def pin_gemm_layout_invariants(mutation: int = 0):
    """TN(A, Bt) == NN(A, Bt^T) and TN(A, Bt)^T == TN(Bt, A), bitwise."""
    for dt in ("f16", "bf16"):
        M, N, K = 19, 24, 40
        A = inputs.draw((M, K), dt, "uniform", 31)
        Bt = inputs.draw((N, K), dt, "uniform", 32)
        tn = oracle.hgemm("tn", dt, A, Bt, mutation=mutation)
        same_bits(tn, oracle.hgemm("nn", dt, A, Bt.T.copy(), mutation=mutation),
                  f"TN vs NN {dt}")
        same_bits(tn.T, oracle.hgemm("tn", dt, Bt, A, mutation=mutation), f"transpose {dt}")


def _all_pairs(M: int, N: int, seed: int):
    """Every (row, column) of an M x N output, in a seeded random order."""
    g = np.random.Generator(np.random.PCG64(seed))
    idx = g.permutation(M * N)
    return idx // N, idx % N


def pin_gemm_sampled_matches_full(mutation: int = 0):
    """The sampled entry point returns the same bits as the full one, at
    every element (in a shuffled order) and at stratified samples, both
    layouts and dtypes.  The first shape is square, so that a build that swaps
    a sample's row and column still reads inside the operands and fails on
    the first comparison."""
    for s, (M, N, K) in enumerate(((40, 40, 24), (37, 45, 64), (45, 37, 40))):
        for dt in ("f16", "bf16"):
            for layout in ("tn", "nn"):
                A = inputs.draw((M, K), dt, "uniform", 41 + s)
                B = inputs.draw((N, K) if layout == "tn" else (K, N), dt, "uniform", 42 + s)
                full = oracle.hgemm(layout, dt, A, B, mutation=mutation)
                r, c = _all_pairs(M, N, 43 + s)
                same_bits(oracle.hgemm_sampled(layout, dt, A, B, r, c, mutation=mutation),
                          full[r, c], f"sampled vs full, every element, {dt} {layout} {M}x{N}")
                r, c = inputs.stratified_samples(M, N, 5, bands=8)
                same_bits(oracle.hgemm_sampled(layout, dt, A, B, r, c, mutation=mutation),
                          full[r, c], f"sampled vs full, stratified, {dt} {layout} {M}x{N}")


def pin_golden(mutation: int = 0):
    """Hand-worked fixtures (tests/golden/*.json)."""
    for fn in sorted(os.listdir(GOLDEN)):
        if not fn.endswith(".json"):
            continue
        with open(os.path.join(GOLDEN, fn)) as f:
            case = json.load(f)
        dt, layout = case["dtype"], case["layout"]
        A = _bits_of(np.array(case["A"], dtype=np.float64), dt)
        B = _bits_of(np.array(case["B"], dtype=np.float64), dt)
        want = np.array([int(h, 16) for row in case["C_bits"] for h in row],
                        dtype=np.uint16).reshape(len(case["C_bits"]), -1)
        same_bits(oracle.hgemm(layout, dt, A, B, mutation=mutation), want, f"golden {fn}")


# --------------------------------------------------------------------------
# General form: operation flags, leading dimensions, alpha and beta.
# --------------------------------------------------------------------------
_NAN_BITS = {"f16": 0x7E00, "bf16": 0x7FC0}


def _stored(logical: np.ndarray, transposed: bool, pad: int, fill: int) -> np.ndarray:
    """Store a logical matrix (transposed or not) in a buffer whose rows are
    `pad` elements longer than needed, the padding filled with `fill`."""
    src = logical.T if transposed else logical
    out = np.full((src.shape[0], src.shape[1] + pad), fill, dtype=np.uint16)
    out[:, :src.shape[1]] = src
    return out


def exact_general(dtype, opA_log: np.ndarray, opB_log: np.ndarray, alpha, beta, Cin_log):
    """Exact rational alpha * A B + beta * Cin on logical operands, rounded once."""
    Av = [[Fraction(x) for x in row] for row in lib_decode(opA_log, dtype).tolist()]
    Bc = [[Fraction(x) for x in col] for col in lib_decode(opB_log, dtype).T.tolist()]
    Cv = lib_decode(Cin_log, dtype).tolist() if beta != 0 else None
    g = grid(dtype)
    al, be = Fraction(alpha), Fraction(beta)
    out = np.zeros((len(Av), len(Bc)), dtype=np.uint16)
    for m in range(len(Av)):
        for n in range(len(Bc)):
            v = al * sum((a * b for a, b in zip(Av[m], Bc[n])), Fraction(0))
            if beta != 0:
                v += be * Fraction(Cv[m][n])
            out[m, n] = g.round(v)
    return out


GENERAL_CASES = [  # (M, N, K, alpha, beta)
    (3, 5, 7, 1.0, 0.0), (6, 4, 9, -0.75, 0.0), (5, 6, 8, 1.5, 1.0), (7, 3, 5, 0.5, -0.25),
    (1, 9, 16, 2.0, 3.0), (4, 4, 1, -1.0, 0.5),
]


def pin_general_bruteforce(mutation: int = 0):
    """All four operation-flag combinations, padded leading dimensions and
    dyadic alpha/beta, against exact rational arithmetic."""
    for dt in ("f16", "bf16"):
        for opA in (0, 1):
            for opB in (0, 1):
                for s, (M, N, K, al, be) in enumerate(GENERAL_CASES):
                    A = inputs.draw((M, K), dt, "normal", 300 + s)
                    Bl = inputs.draw((K, N), dt, "normal", 400 + s)
                    Cin = inputs.draw((M, N), dt, "normal", 500 + s)
                    want = exact_general(dt, A, Bl, al, be, Cin)
                    As = _stored(A, opA == 1, 1 + s % 3, 0x3C00)
                    Bs = _stored(Bl, opB == 1, 2 + s % 2, 0x3C00)
                    Cs = _stored(Cin, False, 3, 0x3C00)
                    got = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, al, be, Cs, mutation=mutation)
                    same_bits(got, want, f"general {dt} op{opA}{opB} {M}x{N}x{K} a={al} b={be}")


def pin_general_small_integers(mutation: int = 0):
    """C = 2 AB - Cin on small integers is exact in every format used: it
    must equal the int64 result bit for bit, for every flag combination."""
    g = np.random.Generator(np.random.PCG64(12))
    for dt, hi, (M, N, K) in (("f16", 2, (9, 11, 128)), ("bf16", 1, (7, 13, 32))):
        Ai = g.integers(-hi, hi + 1, size=(M, K))
        Bi = g.integers(-hi, hi + 1, size=(K, N))
        Ci = g.integers(-4, 5, size=(M, N))
        want = _bits_of(2 * (Ai @ Bi) - Ci, dt)
        for opA in (0, 1):
            for opB in (0, 1):
                As = _stored(_bits_of(Ai, dt), opA == 1, 8, 0)
                Bs = _stored(_bits_of(Bi, dt), opB == 1, 16, 0)
                got = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, 2.0, -1.0,
                                  _stored(_bits_of(Ci, dt), False, 8, 0), mutation=mutation)
                same_bits(got, want, f"general integers {dt} op{opA}{opB}")


def pin_general_padding_and_beta_zero(mutation: int = 0):
    """NaN in the padding of every operand, and in C when beta == 0, must not
    reach the result: it equals the packed, NaN-free computation."""
    for dt in ("f16", "bf16"):
        M, N, K = 6, 8, 10
        A = inputs.draw((M, K), dt, "uniform", 61)
        Bl = inputs.draw((K, N), dt, "uniform", 62)
        ref = oracle.gemm(0, 0, dt, M, N, K, A, Bl, mutation=mutation)
        nan = _NAN_BITS[dt]
        for opA in (0, 1):
            for opB in (0, 1):
                As = _stored(A, opA == 1, 5, nan)
                Bs = _stored(Bl, opB == 1, 7, nan)
                Cs = np.full((M, N + 4), nan, dtype=np.uint16)
                got = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, 1.0, 0.0, Cs, mutation=mutation)
                same_bits(got, ref, f"padding/beta=0 {dt} op{opA}{opB}")


def pin_general_matches_layouts(mutation: int = 0):
    """(opA, opB) = (0, 1) and (0, 0) with packed storage, alpha 1, beta 0 are
    the TN and NN layouts, computed by the oracle's separately written loop."""
    for dt in ("f16", "bf16"):
        M, N, K = 13, 11, 37
        A = inputs.draw((M, K), dt, "normal", 71)
        Bt = inputs.draw((N, K), dt, "normal", 72)
        same_bits(oracle.gemm(0, 1, dt, M, N, K, A, Bt, mutation=mutation),
                  oracle.hgemm("tn", dt, A, Bt, mutation=mutation), f"general vs tn {dt}")
        Bn = np.ascontiguousarray(Bt.T)
        same_bits(oracle.gemm(0, 0, dt, M, N, K, A, Bn, mutation=mutation),
                  oracle.hgemm("nn", dt, A, Bn, mutation=mutation), f"general vs nn {dt}")


GENERAL_SAMPLED_CASES = [  # (M, N, K, alpha, beta); the first is square
    (40, 40, 24, 1.5, -0.5), (37, 45, 64, -0.75, 0.25), (45, 37, 17, 2.0, 0.0),
    (29, 51, 9, 1.0, 0.0),
]


def pin_general_sampled_matches_full(mutation: int = 0):
    """The general form's sampled entry point returns the same bits as its
    full one (itself pinned to exact rational arithmetic above), at every
    element in a shuffled order: all four operation-flag pairs, padded
    leading dimensions (the old C's too), dyadic alpha/beta, and an old C
    filled with NaN when beta == 0.  The first case is square, so that a
    build that swaps a sample's row and column still reads inside the
    operands and fails on the first comparison."""
    for s, (M, N, K, al, be) in enumerate(GENERAL_SAMPLED_CASES):
        for dt in ("f16", "bf16"):
            for opA in (0, 1):
                for opB in (0, 1):
                    A = inputs.draw((M, K), dt, "normal", 600 + s)
                    Bl = inputs.draw((K, N), dt, "normal", 700 + s)
                    As = _stored(A, opA == 1, 8 + s % 3, 0x3C00)
                    Bs = _stored(Bl, opB == 1, 3 + s % 2, 0x3C00)
                    if be != 0:
                        Cs = _stored(inputs.draw((M, N), dt, "normal", 800 + s), False, 5, 0x3C00)
                    else:
                        Cs = np.full((M, N + 5), _NAN_BITS[dt], dtype=np.uint16)
                    full = oracle.gemm(opA, opB, dt, M, N, K, As, Bs, al, be, Cs,
                                       mutation=mutation)
                    r, c = _all_pairs(M, N, 900 + s)
                    got = oracle.gemm_sampled(opA, opB, dt, M, N, K, As, Bs, r, c, al, be, Cs,
                                              mutation=mutation)
                    same_bits(got, full[r, c],
                              f"general sampled vs full {dt} op{opA}{opB} {M}x{N}x{K} "
                              f"a={al} b={be}")


ALL_PINS = [
    pin_decode_exhaustive, pin_round_representable, pin_round_midpoints, pin_round_random,
    pin_round_special, pin_gemm_bruteforce, pin_gemm_small_integers,
    pin_gemm_identity_permutation, pin_gemm_closed_forms, pin_gemm_ties,
    pin_gemm_layout_invariants, pin_gemm_sampled_matches_full, pin_golden,
    pin_general_bruteforce, pin_general_small_integers, pin_general_padding_and_beta_zero,
    pin_general_matches_layouts, pin_general_sampled_matches_full,
]
