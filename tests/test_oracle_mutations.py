"""Planted mistakes in the oracle, each caught by at least one pin.

The oracle is trusted because the `-m "not gpu"` pins of this directory tie it
to what the pages and the mathematics fix: closed forms of Eq. (1) of
"LinQuant: Functional Invariances for Low-Precision Linear Recurrences"
(Theoretical Foundation), hand-worked golden steps, exact-rational brute
force, quantiser and rounding invariants, the dither's golden-ratio sequence,
the bypass recursions and the chunkwise prefill's closed forms.  To show that
the pins bite, each entry below plants one plausible mistake in the oracle's C
source: a dropped term, a wrong sign, index or operand, a wrong rounding,
scale or summation rule.  The mutant is rebuilt on the CPU (`oracle.planted`)
and the pins of its family run against it until one fails.  A mistake that
passes every pin fails this test.
"""
import importlib
import itertools

import pytest

import oracle

DECODE_PINS = ("test_oracle_dot_order", "test_oracle_closed_forms", "test_oracle_quantizer",
               "test_oracle_scale_formats", "test_oracle_head_scale", "test_oracle_bdr_readings",
               "test_oracle_bruteforce")
FAMILIES = {
    "decode": DECODE_PINS,
    "dither": ("test_oracle_dither",),
    "bypass": ("test_oracle_lrb", "test_oracle_lrb_merge_bdr"),
    "prefill": ("test_oracle_prefill",),
}

W_LINE = "      float w = beta * (v[r] - u);"
DECAY_LINES = "        float a = diag ? alpha[c] : alpha[0];\n        float m = s[c / g] * a;"
READOUT = ("      J->o[h * dv + r] = dot_blocked(st, q, dk);\n\n"
           "      /* scale policy, then requantise group by group */")
SRC_LINE = "const float* src = (cfg->policy == LSQO_POLICY_YOKED) ? R : st;"
BDR_STEP = ("            int reversed = (sigma > 0 && c1 < yp) || (sigma < 0 && c1 > yp);\n"
            "            if (reversed) {\n"
            "              c2 = clampd(c1 + sigma, -qm, qm);")
GAMMA = ("          G[t * da + a] = acc;\n"
         "          const float* at = alpha + ((int64_t)(t0 + t) * nh + h) * da;\n"
         "          acc = acc * at[a];")

MUTANTS = {
    # the decode step: Eq. (1), the scale policies, the rounding, the layout
    "delta term dropped": ("decode", [(W_LINE, "      float w = beta * v[r];")]),
    "delta term with the wrong sign": ("decode", [(W_LINE, "      float w = beta * (v[r] + u);")]),
    "beta applied twice": ("decode", [(W_LINE, "      float w = beta * beta * (v[r] - u);")]),
    "diagonal decay of the next column": ("decode", [(
        DECAY_LINES, DECAY_LINES.replace("alpha[c]", "alpha[(c + 1) % dk]"))]),
    "scale of the next group": ("decode", [(
        DECAY_LINES, DECAY_LINES.replace("s[c / g]", "s[(c / g + 1) % ng]"))]),
    "write along q instead of k": ("decode", [(
        "for (int c = 0; c < dk; ++c) st[c] = fmaf(w, k[c], sp[c]);",
        "for (int c = 0; c < dk; ++c) st[c] = fmaf(w, q[c], sp[c]);")]),
    "readout from S' instead of S": ("decode", [(READOUT, READOUT.replace("(st, q", "(sp, q"))]),
    "readout against k": ("decode", [(READOUT, READOUT.replace("(st, q", "(st, k"))]),
    "dynamic scale from S'": ("decode", [(SRC_LINE, SRC_LINE.replace("? R : st", "? R : sp"))]),
    "yoked scale from the quantised state": ("decode", [(SRC_LINE, SRC_LINE.replace("? R : st", "? st : st"))]),
    "dynamic scale over qmax + 1": ("decode", [(
        "          snew = scale_as_stored(amax / (float)qm, cfg->scale_fmt);\n        }\n        float inv",
        "          snew = scale_as_stored(amax / (float)(qm + 1), cfg->scale_fmt);\n        }\n        float inv")]),
    "ties rounded up": ("decode", [(
        "  return (fmod(r, 2.0) == 0.0) ? r : r + 1.0;", "  return r + 1.0;")]),
    "no clamp": ("decode", [("          double c1 = clampd(c0, -qm, qm);", "          double c1 = c0;")]),
    "BDR without the sign of k": ("decode", [(
        "            int sigma = sign_f(w) * sign_f(k[c]);", "            int sigma = sign_f(w);")]),
    "BDR measured from the stored code": ("decode", [(
        "            double yp = (double)sp[c] * (double)inv; /* exact */",
        "            double yp = (double)C[c]; /* exact */")]),
    "BDR repair away from the write": ("decode", [(BDR_STEP, BDR_STEP.replace("c1 + sigma", "c1 - sigma"))]),
    "calibration codes truncated": ("decode", [(
        "        codes[r * dk + c] = (int8_t)clampd(round_half_even(y), -qm, qm);",
        "        codes[r * dk + c] = (int8_t)clampd(trunc(y), -qm, qm);")]),
    "nibbles swapped in pack and unpack": ("decode", [
        ("      packed[r * (dk / 2) + c / 2] = (uint8_t)(lo | (hi << 4));",
         "      packed[r * (dk / 2) + c / 2] = (uint8_t)(hi | (lo << 4));"),
        ("      codes[r * dk + c] = sext4(b & 0x0F);\n      codes[r * dk + c + 1] = sext4(b >> 4);",
         "      codes[r * dk + c] = sext4(b >> 4);\n      codes[r * dk + c + 1] = sext4(b & 0x0F);")]),
    "row dot as one fma chain": ("decode", [(
        "  enum { BLOCK = 32, MAXB = 64 };", "  enum { BLOCK = 1 << 20, MAXB = 64 };")]),
    "block sums added left to right": ("decode", [(
        "  while (nb > 1) {",
        "  for (int i = 1; i < nb; ++i) part[0] = part[0] + part[i];\n  nb = 1;\n  while (nb > 1) {")]),
    "fp32 state: delta term dropped": ("decode", [(
        "  float w = beta * (v_r - u);", "  float w = beta * v_r;")]),
    "fp32 state: decay of the next column": ("decode", [(
        "    float a = (cfg->decay == LSQO_DECAY_DIAG) ? alpha[c] : alpha[0];",
        "    float a = (cfg->decay == LSQO_DECAY_DIAG) ? alpha[(c + 1) % dk] : alpha[0];")]),
    # the golden-ratio Weyl dither
    "Weyl constant off by two": ("dither", [(
        "#define LSQO_WEYL_STEP 0x9E3779B9u", "#define LSQO_WEYL_STEP 0x9E3779BBu")]),
    "dither index column-major": ("dither", [(
        "(uint64_t)r * (uint64_t)dk + (uint64_t)c);", "(uint64_t)c * (uint64_t)dv + (uint64_t)r);")]),
    "dither truncated to 24 bits": ("dither", [(
        "  return (double)(w >> 9) * 0x1p-23;", "  return (double)(w >> 8) * 0x1p-24;")]),
    "dither tie rounded down": ("dither", [(
        "            c0 = fy + ((y - fy >= 1.0 - u) ? 1.0 : 0.0);",
        "            c0 = fy + ((y - fy > 1.0 - u) ? 1.0 : 0.0);")]),
    # the Low-Rank Bypass
    "bypass slot offset by one": ("bypass", [(
        "  const int n_used = (int)(cfg->step % R);", "  const int n_used = (int)((cfg->step + 1) % R);")]),
    "bypass readout without the new write": ("bypass", [("      oo = fmaf(w, kq, oo);", "      (void)kq;")]),
    "bypass buffer not decayed": ("bypass", [(
        "        for (int i = 0; i < dv; ++i) A[j * dv + i] = A[j * dv + i] * ah[0];",
        "        for (int i = 0; i < dv; ++i) A[j * dv + i] = A[j * dv + i];")]),
    "bypass diagonal decay of column 0": ("bypass", [(
        "        for (int c = 0; c < dk; ++c) Bv[j * dk + c] = Bv[j * dk + c] * ah[c];",
        "        for (int c = 0; c < dk; ++c) Bv[j * dk + c] = Bv[j * dk + c] * ah[0];")]),
    "bypass projection without the buffer": ("bypass", [(
        "        for (int j = 0; j < n_used; ++j) u = fmaf(A[j * dv + i], bk[j], u);", "        (void)bk;")]),
    "bypass merge without the last slot": ("bypass", [(
        "          for (int j = 0; j <= n_used; ++j) {", "          for (int j = 0; j < n_used; ++j) {")]),
    # the chunkwise prefill
    "prefill token's own decay in Gamma": ("prefill", [(
        GAMMA, "          const float* at = alpha + ((int64_t)(t0 + t) * nh + h) * da;\n"
               "          acc = acc * at[a];\n          G[t * da + a] = acc;")]),
    # (each prefill edit is planted in both state passes, the per-group one and
    # the per-head one, told apart by the lines around it)
    "prefill without gamma^C": ("prefill", [
        ("          x[c] = fmaf(gam[diag ? c : 0], x[c], H);\n        }",
         "          x[c] = x[c] + H;\n        }"),
        ("            x[c] = fmaf(gam[diag ? c : 0], x[c], H);\n            const float a",
         "            x[c] = x[c] + H;\n            const float a")]),
    "prefill product transposed": ("prefill", [
        ("          for (int t = 0; t < tc; ++t) hacc += (int64_t)Vq[t * dv + r] * (int64_t)Kq[t * dk + c];\n          const",
         "          for (int t = 0; t < tc; ++t) hacc += (int64_t)Vq[t * dv + (c % dv)] * (int64_t)Kq[t * dk + (r % dk)];\n          const"),
        ("            for (int t = 0; t < tc; ++t) hacc += (int64_t)Vq[t * dv + r] * (int64_t)Kq[t * dk + c];",
         "            for (int t = 0; t < tc; ++t) hacc += (int64_t)Vq[t * dv + (c % dv)] * (int64_t)Kq[t * dk + (r % dk)];")]),
    "prefill carries the unquantised state": ("prefill", [(
        "            x[c] = (float)q * snew;   /* the dequantised state carried to the next chunk */",
        "            (void)0;")]),
    "prefill operands rounded half away": ("prefill", [(
        "    q[i] = (int8_t)clampd(round_half_even((double)x[i] * (double)inv), -127, 127);",
        "    q[i] = (int8_t)clampd(round((double)x[i] * (double)inv), -127, 127);")]),
    "prefill without beta": ("prefill", [(
        "        for (int i = 0; i < dv; ++i) BV[t * dv + i] = b * v[row * dv + i];",
        "        (void)b;\n        for (int i = 0; i < dv; ++i) BV[t * dv + i] = v[row * dv + i];")]),
    "prefill decay of column 0": ("prefill", [(
        "GK[t * dk + c] = G[t * da + (diag ? c : 0)] * k[row * dk + c];",
        "GK[t * dk + c] = G[t * da + 0] * k[row * dk + c];")]),
    "prefill with one operand scale": ("prefill", [(
        "      const float sc = s_v * s_k;", "      const float sc = s_v * s_v;")]),
    "prefill scale not rounded to the stored format": ("prefill", [(
        "            snew = scale_as_stored(amax / (float)qm, cfg->scale_fmt);\n          }",
        "            snew = amax / (float)qm;\n          }")]),
    "prefill head scale over the last row only": ("prefill", [(
        "        for (int r = 0; r < dv; ++r) {\n          float* x = S + r * dk;",
        "        for (int r = 0; r < dv; ++r) {\n          amax = 0.0f;\n          float* x = S + r * dk;")]),
    "prefill with the chunk's first decay": ("prefill", [(
        "          const float* at = alpha + ((int64_t)(t0 + t) * nh + h) * da;",
        "          const float* at = alpha + ((int64_t)(t0) * nh + h) * da;")]),
}


def _cases(fn):
    """Keyword arguments of every parametrised case of a pin (the product of its
    parametrize marks)."""
    grids = []
    for m in getattr(fn, "pytestmark", []):
        if m.name != "parametrize":
            continue
        names, values = m.args[0], m.args[1]
        names = [n.strip() for n in names.split(",")] if isinstance(names, str) else list(names)
        rows = []
        for v in values:
            if type(v).__name__ == "ParameterSet":   # pytest.param(...)
                v = v.values
            elif len(names) == 1:
                v = (v,)
            rows.append(dict(zip(names, v)))
        grids.append(rows)
    if not grids:
        return [{}]
    return [{k: val for d in combo for k, val in d.items()} for combo in itertools.product(*grids)]


def _pins(family):
    for mod_name in FAMILIES[family]:
        mod = importlib.import_module(f"tests.{mod_name}")
        for name in sorted(n for n in dir(mod) if n.startswith("test_")):
            fn = getattr(mod, name)
            if not callable(fn) or "planted" in name:
                continue
            if any(m.name == "gpu" for m in getattr(fn, "pytestmark", [])):
                continue
            for kw in _cases(fn):
                yield f"{mod_name}::{name}{kw}", fn, kw


def _first_failure(family):
    for label, fn, kw in _pins(family):
        try:
            fn(**kw)
        except pytest.skip.Exception:
            continue
        except Exception as e:                  # an assertion, or an error the mistake causes
            return f"{label}: {type(e).__name__}"
    return None


@pytest.mark.parametrize("name", list(MUTANTS))
def test_planted_mistake_is_caught(name):
    family, edits = MUTANTS[name]
    with oracle.planted(edits):
        caught = _first_failure(family)
    assert caught is not None, f"no pin of the {family} family catches: {name}"
    print(f"\n{name}: caught by {caught}")


@pytest.mark.parametrize("family", list(FAMILIES))
def test_pins_pass_on_the_oracle(family):
    """The control: every pin of the family passes on the unplanted oracle, so a
    failure above is the planted mistake's."""
    assert _first_failure(family) is None
