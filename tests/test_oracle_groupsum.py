"""Pins of the oracle's per-group dot products and of its canonical multi-group accumulation sequence (CPU only).

The GEMMs multiply one 128-wide quantization group at a time (Jet-RL explainers, "Schema de Quantification":
1x128 activation groups, 128x128 weight blocks, FP8 GEMMs in the forward pass and both backward GEMMs).  The
oracle has two readings of a group's dot product p: EXACT (fp32 rounding of the exact sum) and MFMA (the stated
block-alignment model of the gfx950 FP8 matrix instruction).  Each output then follows one fixed sequence:
acc = +0; for each group g in ascending order: acc = fma(p_g, fl32(sa_g * sb_g), acc); out = bf16(acc).

  * tests/golden/group_sums.txt holds hand-derived group sums in both readings.  Every line is checked, and the
    oracle is rebuilt with plausible mistakes planted in its source (blocks of 16 or 4, a cut at 2^(emax-12) or
    2^(emax-14), rounding or flooring instead of cutting toward zero, a subnormal exponent of -7, zero products
    counted in emax, alignment to the largest product instead of the largest exponent sum, block sums added in
    fp32, a truncating final rounding): each mutant must miss at least one golden line.
  * The sequence is pinned with exact rational arithmetic on constructed two-group outputs whose bf16 result
    changes if the scaled add is a multiply then an add, if the groups run in descending order, or if the
    A-row scale is folded into p before the B scale; the oracle rebuilt with each of those mistakes must fail.
"""
import ctypes
import os
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "group_sums.txt")
ORACLE_SRC = os.path.join(os.path.dirname(HERE), "oracle", "jetfp8_oracle.c")


def _load_golden():
    rows = []
    for line in open(GOLDEN):
        body = line.split("#")[0].split()
        if not body:
            continue
        fa, fb, terms, want_model, want_exact = body
        a = np.full(128, int(fa, 16), np.uint8)
        b = np.full(128, int(fb, 16), np.uint8)
        if terms != "-":
            for t in terms.split(","):
                k, ca, cb = t.split(":")
                a[int(k)], b[int(k)] = int(ca, 16), int(cb, 16)
        rows.append((terms, a, b, int(want_model, 16), int(want_exact, 16)))
    return rows


def _bits(f: float) -> int:
    return struct.unpack("<I", struct.pack("<f", f))[0]


def test_golden_group_sums(orc):
    rows = _load_golden()
    assert len(rows) >= 10
    for terms, a, b, want_model, want_exact in rows:
        assert _bits(orc.group_sum(a, b, orc.MFMA)) == want_model, (terms, "matrix-instruction model")
        assert _bits(orc.group_sum(a, b, orc.EXACT)) == want_exact, (terms, "exact")


# ------------------------------------------------------------------------------------- mutant builds

def _build_variant(tmp_path, name, edits):
    """The oracle's C source with each (old, new, count) edit applied (old must occur exactly `count` times),
    compiled with the oracle's own flags into tmp_path; returns the loaded library."""
    src = open(ORACLE_SRC).read()
    for old, new, count in edits:
        assert src.count(old) == count, (name, old, src.count(old))
        src = src.replace(old, new)
    c_path = tmp_path / f"{name}.c"
    so_path = tmp_path / f"lib{name}.so"
    c_path.write_text(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                    "-o", str(so_path), str(c_path), "-lm", "-lpthread"], check=True)
    L = ctypes.CDLL(str(so_path))
    u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
    f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
    u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
    L.jo_group_sum.restype = ctypes.c_float
    L.jo_group_sum.argtypes = [u8p, u8p, ctypes.c_int]
    for fn in ("jo_gemm_fwd", "jo_gemm_dgrad", "jo_gemm_wgrad"):
        f = getattr(L, fn)
        f.restype = None
        f.argtypes = [u8p, f32p, u8p, f32p, u16p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                      ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int]
    return L


_BLOCK_LOOP = ("for (int blk = 0; blk < 16; ++blk) {", "for (int t = 0; t < 8; ++t)", "(blk * 8 + t)")
GROUP_SUM_MUTANTS = {
    "blocks_of_16": [(_BLOCK_LOOP[0], "for (int blk = 0; blk < 8; ++blk) {", 1),
                     ("int64_t prod[8];", "int64_t prod[16];", 1),
                     (_BLOCK_LOOP[1], "for (int t = 0; t < 16; ++t)", 2),
                     (_BLOCK_LOOP[2], "(blk * 16 + t)", 2)],
    "blocks_of_4": [(_BLOCK_LOOP[0], "for (int blk = 0; blk < 32; ++blk) {", 1),
                    (_BLOCK_LOOP[1], "for (int t = 0; t < 4; ++t)", 2),
                    (_BLOCK_LOOP[2], "(blk * 4 + t)", 2)],
    "cut_at_emax_minus_12": [("cut_toward_zero(prod[t], emax - 13 + 18)", "cut_toward_zero(prod[t], emax - 12 + 18)", 1)],
    "cut_at_emax_minus_14": [("cut_toward_zero(prod[t], emax - 13 + 18)", "cut_toward_zero(prod[t], emax - 14 + 18)", 1)],
    "round_to_grid": [("m = (m >> sh) << sh;", "m = ((m + ((int64_t)1 << (sh - 1))) >> sh) << sh;", 1)],
    "floor_to_grid": [("int64_t m = x < 0 ? -x : x;", "int64_t m = x;", 1),
                      ("return x < 0 ? -m : m;", "return m;", 1)],
    "subnormal_exponent_minus_7": [("return e == 0 ? -6 : e - 7;", "return e - 7;", 1)],
    "zeros_set_emax": [("if (prod[t] != 0 && code_exp(ca) + code_exp(cb) > emax)",
                        "if (code_exp(ca) + code_exp(cb) > emax)", 1)],
    "align_to_largest_product": [
        ("if (prod[t] != 0 && code_exp(ca) + code_exp(cb) > emax) emax = code_exp(ca) + code_exp(cb);",
         "if (prod[t] != 0 && ilogb(ldexp((double)prod[t], -18)) > emax) emax = ilogb(ldexp((double)prod[t], -18));",
         1)],
    "block_sums_added_in_fp32": [
        ("static float group_sum_mfma(const uint8_t* a, int64_t sa, const uint8_t* b, int64_t sb) {\n"
         "    int64_t total = 0;",
         "static float group_sum_mfma(const uint8_t* a, int64_t sa, const uint8_t* b, int64_t sb) {\n"
         "    float ftotal = 0.0f;", 1),
        ("        for (int t = 0; t < 8; ++t)\n            if (prod[t] != 0) total += cut_toward_zero(prod[t], emax - 13 + 18);\n"
         "    }\n    return (float)ldexp((double)total, -18);",
         "        int64_t total = 0;\n        for (int t = 0; t < 8; ++t)\n"
         "            if (prod[t] != 0) total += cut_toward_zero(prod[t], emax - 13 + 18);\n"
         "        ftotal += (float)ldexp((double)total, -18);\n    }\n    return ftotal;", 1)],
    "truncating_final_rounding": [
        ("    }\n    return (float)ldexp((double)total, -18);\n}",
         "    }\n    double d = ldexp((double)total, -18);\n    float f = (float)d;\n"
         "    if (fabs((double)f) > fabs(d)) f = nextafterf(f, 0.0f);\n    return f;\n}", 1)],
}


def test_unmutated_build_passes_golden(tmp_path):
    L = _build_variant(tmp_path, "unmutated", [])
    for terms, a, b, want_model, want_exact in _load_golden():
        assert _bits(L.jo_group_sum(a, b, 1)) == want_model, terms
        assert _bits(L.jo_group_sum(a, b, 0)) == want_exact, terms


@pytest.mark.parametrize("mutant", sorted(GROUP_SUM_MUTANTS))
def test_golden_group_sums_catch_mutant(tmp_path, mutant):
    L = _build_variant(tmp_path, mutant, GROUP_SUM_MUTANTS[mutant])
    missed = [terms for terms, a, b, want_model, _ in _load_golden() if _bits(L.jo_group_sum(a, b, 1)) != want_model]
    assert missed, f"mutant {mutant} passes every golden group sum"


# ---------------------------------------------------------------- canonical sequence, exact rationals

def _decode(c: int) -> Fraction:
    s, e, m = (c >> 7) & 1, (c >> 3) & 15, c & 7
    v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def _round(x: Fraction, bits: int) -> Fraction:
    """Nearest value with `bits` significant bits (ties to even significand), unbounded exponent: fp32 for 24,
    bf16 for 8 (the values here stay in the normal range of both)."""
    if x == 0:
        return Fraction(0)
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    ulp = Fraction(2) ** (e - bits + 1)
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return (n * ulp) if x > 0 else -(n * ulp)


def _sequence(groups, variant="c6"):
    """bf16 value of one output from its groups [(a codes, b codes, sa, sb)], exact rationals throughout.
    variant: "c6" (acc = fma(p, fl32(sa*sb), acc), ascending), "mul_add" (acc = fl32(fl32(p*s) + acc)),
    "descending" (C6 with the groups reversed), "fold_sa" (acc = fma(fl32(p*sa), sb, acc))."""
    gs = list(reversed(groups)) if variant == "descending" else groups
    acc = Fraction(0)
    for a, b, sa, sb in gs:
        p = _round(sum((_decode(int(x)) * _decode(int(y)) for x, y in zip(a, b)), Fraction(0)), 24)
        sa, sb = Fraction(sa), Fraction(sb)
        if variant == "mul_add":
            acc = _round(_round(p * _round(sa * sb, 24), 24) + acc, 24)
        elif variant == "fold_sa":
            acc = _round(_round(p * sa, 24) * sb + acc, 24)
        else:
            acc = _round(p * _round(sa * sb, 24) + acc, 24)
    return _round(acc, 8)


def _codes(terms):
    v = np.zeros(128, np.uint8)
    for k, c in terms.items():
        v[k] = c
    return v


def _f32(x: Fraction) -> np.float32:
    f = np.float32(float(x))
    assert Fraction(float(f)) == x
    return f


# Case 1: p0 = 1 + 2^-8 (s0 = 1) puts acc on a bf16 midpoint; p1 = 1 + 2^-15 times s1 = 2^-24 (1 - 2^-15 + 2^-24)
# adds 2^-24 (half an fp32 step) plus about 2^-48.  One rounding (fma) lands above the midpoint -> bf16 rounds up;
# a separately rounded product drops the 2^-48 and the tie goes to even -> bf16 stays at 1.  Descending order rounds
# p1*s1 alone first and loses the excess the same way.
CASE1 = [(_codes({0: 0x38, 1: 0x02}), _codes({0: 0x38, 1: 0x38}), Fraction(1), Fraction(1)),
         (_codes({0: 0x38, 8: 0x01}), _codes({0: 0x38, 8: 0x08}), Fraction(2 ** 24 - 2 ** 9 + 1, 2 ** 48), Fraction(1))]
# Case 2: p0 = 1 + 2^-12, sa0 = 1 + 2^-12, sb0 = 1 + 2^-13: fl32(sa*sb) = 1 + 3*2^-13, and p0 times it rounds up to
# 1 + 5*2^-13 + 2^-23; folding sa into p first gives 1 + 5*2^-13 (two ties to even).  p1 = 27*2^-13 (s1 = 1) then
# lands the sum on 1 + 2^-8 + 2^-23 (bf16 rounds up) or exactly on the midpoint 1 + 2^-8 (bf16 rounds to even, 1).
CASE2 = [(_codes({0: 0x38, 1: 0x08}), _codes({0: 0x38, 1: 0x08}), Fraction(4097, 4096), Fraction(8193, 8192)),
         (_codes({0: 0x08, 1: 0x08, 2: 0x08, 3: 0x08}), _codes({0: 0x20, 1: 0x18, 2: 0x08, 3: 0x04}),
          Fraction(1), Fraction(1))]


def test_constructed_cases_separate_the_sequences():
    """The constructed outputs are bf16 1 + 2^-7 under the canonical sequence and 1.0 under the named variants."""
    up, one = Fraction(129, 128), Fraction(1)
    assert _sequence(CASE1) == up and _sequence(CASE2) == up
    assert _sequence(CASE1, "mul_add") == one and _sequence(CASE1, "descending") == one
    assert _sequence(CASE2, "fold_sa") == one


def _gemm_inputs(cases):
    """Place two-group cases into the forward, DGrad and WGrad layouts.  Case c sits at output row c and output
    column 128 c (so the block-scaled GEMMs give each case its own 128x128 weight block).  Returns per GEMM the
    oracle call's inputs and, per case, the output index."""
    nc = len(cases)
    M, J, Kc = nc, 128 * nc, 256
    # forward: xq [M, Kc], xs [Kc/128, M]; wq [J, Kc], ws [J/128, Kc/128]
    xq = np.zeros((M, Kc), np.uint8)
    xs = np.ones((2, M), np.float32)
    wq = np.zeros((J, Kc), np.uint8)
    ws = np.ones((J // 128, 2), np.float32)
    for c, groups in enumerate(cases):
        for g, (a, b, sa, sb) in enumerate(groups):
            xq[c, g * 128:(g + 1) * 128] = a
            wq[128 * c, g * 128:(g + 1) * 128] = b
            xs[g, c] = _f32(sa)
            ws[c, g] = _f32(sb)
    fwd = (xq, xs, wq, ws)
    # DGrad: dyq [M, N=Kc], dys [N/128, M]; W [N=Kc, K=J] read down its columns, block scales [N/128][K/128]
    dgrad = (xq, xs, np.ascontiguousarray(wq.T), np.ascontiguousarray(ws.T))
    # WGrad: dyq [Mc=Kc, N=M rows of dW], dys [Mc/128, N]; xq [Mc, K=J], xs [Mc/128, K]
    dws = np.ones((2, J), np.float32)
    for c, groups in enumerate(cases):
        for g, (_, _, _, sb) in enumerate(groups):
            dws[g, 128 * c] = _f32(sb)
    wgrad = (np.ascontiguousarray(xq.T), xs, np.ascontiguousarray(wq.T), dws)
    return fwd, dgrad, wgrad, [(c, 128 * c) for c in range(nc)]


def _oracle_outputs(L, which, inputs, mode):
    """Run one GEMM of a (possibly mutant) oracle library L; returns the bf16 output bits."""
    if which == "fwd":
        xq, xs, wq, ws = inputs
        out = np.empty((xq.shape[0], wq.shape[0]), np.uint16)
        L.jo_gemm_fwd(xq, xs, wq, ws, out, xq.shape[0], wq.shape[0], xq.shape[1], None, out.shape[0], mode, 1)
    elif which == "dgrad":
        dyq, dys, w, ws = inputs
        out = np.empty((dyq.shape[0], w.shape[1]), np.uint16)
        L.jo_gemm_dgrad(dyq, dys, w, ws, out, dyq.shape[0], dyq.shape[1], w.shape[1], None, out.shape[0], mode, 1)
    else:
        dyq, dys, xq, xs = inputs
        out = np.empty((dyq.shape[1], xq.shape[1]), np.uint16)
        L.jo_gemm_wgrad(dyq, dys, xq, xs, out, dyq.shape[0], dyq.shape[1], xq.shape[1], None, out.shape[0], mode, 1)
    return out


def _expected_all(which, inputs):
    """Every output of the GEMM under the canonical sequence with exact group sums (exact rationals)."""
    if which == "fwd":
        aq, as_, bq, bs = inputs
        I, J, G = aq.shape[0], bq.shape[0], aq.shape[1] // 128
        grp = lambda i, j, g: (aq[i, g * 128:(g + 1) * 128], bq[j, g * 128:(g + 1) * 128], as_[g, i], bs[j // 128, g])
    elif which == "dgrad":
        aq, as_, w, bs = inputs
        I, J, G = aq.shape[0], w.shape[1], aq.shape[1] // 128
        grp = lambda i, j, g: (aq[i, g * 128:(g + 1) * 128], w[g * 128:(g + 1) * 128, j], as_[g, i], bs[g, j // 128])
    else:
        dq, ds, xq, xs = inputs
        I, J, G = dq.shape[1], xq.shape[1], dq.shape[0] // 128
        grp = lambda i, j, g: (dq[g * 128:(g + 1) * 128, i], xq[g * 128:(g + 1) * 128, j], ds[g, i], xs[g, j])
    out = np.empty((I, J), np.uint16)
    for i in range(I):
        for j in range(J):
            gs = [grp(i, j, g) for g in range(G)]
            v = _sequence([(a, b, Fraction(float(sa)), Fraction(float(sb))) for a, b, sa, sb in gs])
            out[i, j] = _bits(float(v)) >> 16 if v != 0 else 0
    return out


@pytest.mark.parametrize("which", ["fwd", "dgrad", "wgrad"])
def test_canonical_sequence_exact_rationals(orc, which):
    """Every output of each GEMM equals the canonical sequence evaluated with exact rationals (exact group sums);
    the constructed outputs also agree in the matrix-instruction mode (no product is cut in them)."""
    fwd, dgrad, wgrad, where = _gemm_inputs([CASE1, CASE2])
    inputs = {"fwd": fwd, "dgrad": dgrad, "wgrad": wgrad}[which]
    want = _expected_all(which, inputs)
    L = orc.lib()
    got = _oracle_outputs(L, which, inputs, orc.EXACT)
    assert np.array_equal(got, want)
    got_model = _oracle_outputs(L, which, inputs, orc.MFMA)
    for (i, j) in where:
        assert got_model[i, j] == want[i, j] == 0x3F81, (which, i, j)


SEQUENCE_MUTANTS = {
    "mul_then_add": [("acc = fmaf(pg, s, acc);", "acc = pg * s + acc;", 3)],
    "descending_groups": [("for (int64_t g = 0; g < G; ++g) {\n            float pg",
                           "for (int64_t g = G - 1; g >= 0; --g) {\n            float pg", 3)],
    "fold_row_scale_first": [
        ("float s = c->as[g * c->M + m] * c->bs[(n / 128) * G + g];\n            acc = fmaf(pg, s, acc);",
         "acc = fmaf(pg * c->as[g * c->M + m], c->bs[(n / 128) * G + g], acc);", 1),
        ("float s = c->as[g * c->M + m] * c->bs[g * KB + k / 128];\n            acc = fmaf(pg, s, acc);",
         "acc = fmaf(pg * c->as[g * c->M + m], c->bs[g * KB + k / 128], acc);", 1),
        ("float s = c->as[g * c->N + n] * c->bs[g * c->K + k];\n            acc = fmaf(pg, s, acc);",
         "acc = fmaf(pg * c->as[g * c->N + n], c->bs[g * c->K + k], acc);", 1)],
}


@pytest.mark.parametrize("mutant", sorted(SEQUENCE_MUTANTS))
def test_canonical_sequence_catches_mutant(tmp_path, mutant):
    L = _build_variant(tmp_path, mutant, SEQUENCE_MUTANTS[mutant])
    fwd, dgrad, wgrad, where = _gemm_inputs([CASE1, CASE2])
    for which, inputs in (("fwd", fwd), ("dgrad", dgrad), ("wgrad", wgrad)):
        got = _oracle_outputs(L, which, inputs, 0)
        assert any(got[i, j] != 0x3F81 for i, j in where), f"mutant {mutant} passes the constructed {which} outputs"
