"""Validity check of the fused GELU quantizer's codes against the oracle.

The oracle rounds the exact GELU (fp64) to bf16; the kernel evaluates GELU in
fp32 with a stated relative error bound and then rounds to bf16.  The two
bf16 values can differ only for elements whose exact GELU lies within that
bound of a bf16 rounding boundary (or of the 2^-100 flush threshold): such an
element may take either neighbour.  This module lists every element's
admissible bf16 values and accepts a row of kernel codes and its scale if and
only if some admissible choice for every element reproduces them exactly
through the oracle's quantization steps (block FWHT, absmax, r = 127/a,
rint, clamp).  Rows without an ambiguous element must match the oracle
bit for bit.  Used by the GPU tests; the checker itself is tested on the CPU.
"""
from __future__ import annotations

import itertools
import math

import numpy as np

from oracle import tabit_oracle as O

ULP24 = 2.0 ** -24
MAX_KEYS_PER_BLOCK = 12          # at most 3^12 combinations per block


def kernel_gelu_rel_bound(z: np.ndarray) -> np.ndarray:
    """Relative error bound of the kernel's fp32 GELU at z = 2u (exact).

    The kernel forms z = x (k1 + k3 x^2) (4 roundings, 2 rounded constants),
    t = 2^(-|z| log2 e) (1 rounding, 1 constant, the hardware exp2 within 2 ulp),
    s = 1 / (1 + t) (1 rounding, reciprocal within 1 ulp), sigma = s (z >= 0) or
    t s (z < 0), g = x sigma.  An absolute error d in the exponent's argument is a
    relative error d ln 2 of t, i.e. |z| (8 ulp); through s it is damped by
    t / (1 + t), and for z >= 0, |z| t <= 1/e.  Bounds used (ulp = 2^-24):
      z >= 0:  16 ulp,   z < 0:  (16 |z| + 24) ulp
    (about 1.5x the sum of the terms above)."""
    z = np.asarray(z, dtype=np.float64)
    return np.where(z >= 0, 16.0 * ULP24, (16.0 * np.abs(z) + 24.0) * ULP24)


def _flush(v):
    return np.where(np.abs(v) < O.GELU_FLUSH, 0.0, v)


def _bits_to_f64(bits):
    return O.bf16_to_f32(np.asarray(bits, dtype=np.uint16)).astype(np.float64)


def admissible_bf16(x_bits: np.ndarray):
    """(oracle bf16 bits [M, K], list of (m, k, candidate bits tuple)) for ambiguous elements."""
    x = _bits_to_f64(x_bits)
    g = O.gelu_tanh_f64(x)
    ref = O.f64_to_bf16_bits(g)
    z = 2.0 * math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)
    eps = kernel_gelu_rel_bound(z)
    lo = O.f64_to_bf16_bits(_flush(g * (1 - eps)))
    hi = O.f64_to_bf16_bits(_flush(g * (1 + eps)))
    amb = []
    for m, k in zip(*np.nonzero((lo & 0x7FFF) != (hi & 0x7FFF))):
        a, b = int(lo[m, k]), int(hi[m, k])
        # every bf16 value between the two ends (same sign; magnitudes step by one code);
        # the range crosses the flush only at its low end, which is then 0
        s = (a | b) & 0x8000
        ma, mb = sorted((a & 0x7FFF, b & 0x7FFF))
        cands = set()
        for mm in range(ma, mb + 1):
            v = abs(float(_bits_to_f64(mm)))
            if mm == 0 or v >= O.GELU_FLUSH:
                cands.add(s | mm if mm else 0)
        assert int(ref[m, k]) in cands or (int(ref[m, k]) & 0x7FFF) == 0 and 0 in cands
        assert len(cands) <= 3, (m, k, cands)
        amb.append((int(m), int(k), tuple(sorted(cands))))
    return ref, amb


def _codes(y32: np.ndarray, r: np.float32) -> np.ndarray:
    """The oracle's code step on fp32 rotated values y for the row's r."""
    t = (y32.astype(np.float32) * r).astype(np.float32)
    return np.clip(np.rint(t), -127, 127).astype(np.int8)


def check_gelu_quant(x_bits: np.ndarray, had_block: int, q: np.ndarray, s: np.ndarray) -> dict:
    """Raise AssertionError unless (q, s) is an admissible result for every row.

    Returns counts: ambiguous elements and rows, and rows compared bit for bit."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    ref_bits, amb = admissible_bf16(x_bits)
    q_ref, s_ref = O.quantize_act_int8(ref_bits, had_block)
    by_row = {}
    for m, k, c in amb:
        by_row.setdefault(m, []).append((k, c))
    exact_rows = [m for m in range(M) if m not in by_row]
    if exact_rows:
        np.testing.assert_array_equal(q[exact_rows], q_ref[exact_rows])
        np.testing.assert_array_equal(s[exact_rows].view(np.uint32), s_ref[exact_rows].view(np.uint32))
    B = max(had_block, 1)
    for m, elems in by_row.items():
        base = _bits_to_f64(ref_bits[m]).astype(np.float32)
        y_base = O.block_fwht_f32(base[None, :], had_block)[0]
        blocks = {}
        for k, c in elems:
            blocks.setdefault(k // B, []).append((k, c))
        fixed = np.ones(K, dtype=bool)
        for j in blocks:
            fixed[j * B:(j + 1) * B] = False
        fixed_max = np.float32(np.max(np.abs(y_base[fixed]))) if fixed.any() else np.float32(0)
        # per ambiguous block: every combination of admissible values -> rotated block.
        # The kernel's GELU is a function of x alone, so equal inputs take the same
        # value: combinations run over the distinct ambiguous inputs of the block.
        opts = {}
        for j, lst in blocks.items():
            keys = {}
            for k, c in lst:
                keys.setdefault(int(x_bits[m, k]), (c, []))[1].append(k)
            if len(keys) > MAX_KEYS_PER_BLOCK:
                raise AssertionError(f"row {m} block {j}: {len(keys)} distinct ambiguous inputs "
                                     f"(more than {MAX_KEYS_PER_BLOCK}); choose other test inputs")
            groups = list(keys.values())
            ys = []
            for combo in itertools.product(*[c for c, _ in groups]):
                blk = base[j * B:(j + 1) * B].copy()
                for (_, ks), cb in zip(groups, combo):
                    for k in ks:
                        blk[k - j * B] = np.float32(_bits_to_f64(cb))
                yb = O.block_fwht_f32(blk[None, :], had_block)[0]
                ys.append(yb)
            ys = np.stack(ys)
            opts[j] = (ys, np.max(np.abs(ys), axis=1))
        cand_a = {float(fixed_max)} | {float(v) for _, mx in opts.values() for v in mx}
        ok = False
        for a in sorted(cand_a):
            a32 = np.float32(a)
            s_a = np.float32(a32 / np.float32(127.0)) if a32 > 0 else np.float32(0)
            if s_a.view(np.uint32) != s[m].view(np.uint32):
                continue
            r = np.float32(np.float32(127.0) / a32) if a32 > 0 else np.float32(0)
            if fixed.any() and not np.array_equal(_codes(y_base[fixed], r), q[m][fixed]):
                continue
            attained = fixed.any() and fixed_max == a32
            good = True
            for j, (ys, mx) in opts.items():
                want = q[m, j * B:(j + 1) * B]
                sel = [i for i in range(len(ys)) if mx[i] <= a32 and np.array_equal(_codes(ys[i], r), want)]
                if not sel:
                    good = False
                    break
                attained = attained or any(mx[i] == a32 for i in sel)
            if good and attained:
                ok = True
                break
        assert ok, f"row {m}: no admissible choice of the {len(elems)} ambiguous elements gives the kernel's codes"
    return {"ambiguous_elements": len(amb), "ambiguous_rows": len(by_row), "exact_rows": len(exact_rows)}


def check_gelu_quant_mx(x_bits: np.ndarray, had_block: int, packed: np.ndarray,
                        e8m0: np.ndarray) -> dict:
    """As check_gelu_quant, for the MXFP4 format: each 32-element block (its own E8M0
    scale) must equal the oracle's MX quantization of some admissible choice of its
    ambiguous elements (equal inputs sharing one value); blocks without an ambiguous
    element must match bit for bit."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M, K = x_bits.shape
    ref_bits, amb = admissible_bf16(x_bits)
    p_ref, e_ref = O.mx_quantize_rows(O.bf16_to_f32(ref_bits), had_block)
    blk_amb = {}
    for m, k, c in amb:
        blk_amb.setdefault((m, k // 32), {}).setdefault(int(x_bits[m, k]), (c, []))[1].append(k)
    mask = np.ones((M, K // 32), dtype=bool)
    for (m, j) in blk_amb:
        mask[m, j] = False
    pb = np.asarray(packed).reshape(M, K // 32, 16)
    pr = p_ref.reshape(M, K // 32, 16)
    np.testing.assert_array_equal(pb[mask], pr[mask])
    np.testing.assert_array_equal(np.asarray(e8m0)[mask], e_ref[mask])
    for (m, j), keys in blk_amb.items():
        if len(keys) > MAX_KEYS_PER_BLOCK:
            raise AssertionError(f"row {m} block {j}: too many distinct ambiguous inputs")
        groups = list(keys.values())
        base = _bits_to_f64(ref_bits[m, 32 * j:32 * j + 32]).astype(np.float32)
        rows = []
        for combo in itertools.product(*[c for c, _ in groups]):
            blk = base.copy()
            for (_, ks), cb in zip(groups, combo):
                for k in ks:
                    blk[k - 32 * j] = np.float32(_bits_to_f64(cb))
            rows.append(blk)
        pc, ec = O.mx_quantize_rows(np.stack(rows), had_block)
        ok = any(np.array_equal(pc[i], pb[m, j]) and ec[i, 0] == e8m0[m, j] for i in range(len(rows)))
        assert ok, f"row {m} block {j}: no admissible choice gives the kernel's MX bytes"
    return {"ambiguous_elements": len(amb), "ambiguous_blocks": len(blk_amb),
            "exact_blocks": int(mask.sum())}
