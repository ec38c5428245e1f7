"""Writes the closed-form fixtures in this folder.

Every expected number here is the evaluation of a closed form stated in the fixture's
"derivation" field (Python's math module, float64). Nothing is computed by the oracle or by the
GPU library. Run from the repository root: python tests/golden/make_closed_forms.py
"""
import json
import math
import os
import struct
from fractions import Fraction

HERE = os.path.dirname(os.path.abspath(__file__))
LN2 = math.log(2.0)


def worked_softcap30():
    lse = 24.0 + math.log1p(math.exp(-6.0) + math.exp(-24.0))
    nats = [lse - 18.0, lse - 24.0, lse - 0.0]
    return {
        "what": "worked example of the softcapped cross-entropy and bits per byte, values in closed form",
        "source": ("definition only: the pages print no worked example. Softcap s = c*tanh(z/c) is the reading of "
                   "the fused softcapped cross-entropy the pages name (HYDRA Golf site stack list; parameter-golf "
                   "README leaderboard, PR #1787 row); bits per byte as the README introduction scores compression."),
        "derivation": ("H = [[1]] for all three rows, E = [[30 ln 2], [30 ln 3], [0]], c = 30. Then z = E[:,0], "
                       "z/c = ln 2, ln 3, 0 and tanh(ln 2) = 3/5, tanh(ln 3) = 4/5, so s = [18, 24, 0]. "
                       "lse = 24 + log1p(e^-6 + e^-24); nats[t] = lse - s[target[t]] with targets [0, 1, 2]; "
                       "byte_len = [1, 2, 4]; bpb = sum nats / (ln 2 * 7)."),
        "softcap": 30.0,
        "hidden": [[1.0], [1.0], [1.0]],
        "embed": [[30.0 * math.log(2.0)], [30.0 * math.log(3.0)], [0.0]],
        "target": [0, 1, 2],
        "byte_len": [1, 2, 4],
        "expected": {"lse": [lse, lse, lse], "nats": nats, "sum_nats": sum(nats), "sum_bytes": 7,
                     "n_scored": 3, "bpb": sum(nats) / (LN2 * 7), "s": [18.0, 24.0, 0.0]},
    }


def worked_asym():
    s = [18.0, -8.0, 0.0, -3640.0 / 365.0]
    lse = 18.0 + math.log1p(math.exp(-26.0) + math.exp(-18.0) + math.exp(s[3] - 18.0))
    nats = [lse - v for v in s]
    return {
        "what": "worked example of the asymmetric softcap (cap 30 for z >= 0, cap 10 for z < 0), closed form",
        "source": ("definition only: the pages name an 'AsymLogit' head change (HYDRA Golf site leaderboard table, "
                   "entries #1 and #4; README leaderboard, PR #2135 and PR #1945 rows) without defining it; the reading "
                   "taken is s = c_pos tanh(z / c_pos) for z >= 0 and c_neg tanh(z / c_neg) for z < 0."),
        "derivation": ("H = [[1]] x4, E = [[30 ln 2], [-10 ln 3], [0], [-30 ln 3]], caps (30, 10). "
                       "z/c = ln 2 (positive side), -ln 3, 0, -3 ln 3 (negative side); tanh(k ln 3) = (3^(2k) - 1)/(3^(2k) + 1), "
                       "so s = [30 * 3/5, -10 * 4/5, 0, -10 * 728/730] = [18, -8, 0, -3640/365]. "
                       "lse = 18 + log1p(e^-26 + e^-18 + e^(s3 - 18)); targets [0, 1, 2, 3]; byte_len [1, 1, 2, 3]."),
        "caps": [30.0, 10.0],
        "hidden": [[1.0], [1.0], [1.0], [1.0]],
        "embed": [[30.0 * math.log(2.0)], [-10.0 * math.log(3.0)], [0.0], [-30.0 * math.log(3.0)]],
        "target": [0, 1, 2, 3],
        "byte_len": [1, 1, 2, 3],
        "expected": {"s": s, "lse": [lse] * 4, "nats": nats, "sum_nats": sum(nats), "sum_bytes": 7,
                     "n_scored": 4, "bpb": sum(nats) / (LN2 * 7)},
    }


def worked_nocap():
    return {
        "what": "worked example without a cap: one bit and two bits of surprise over three bytes gives 1 bit per byte",
        "source": "definition only (README introduction, bits per byte); c = 0 reads as 'no softcap'.",
        "derivation": ("H = [[1]] x3, E = [[ln 2], [0], [0]], c = 0, so z = s = [ln 2, 0, 0] and lse = ln 4. "
                       "Targets [0, 1, 2] with mask [1, 1, 0]: nats = [ln 2, 2 ln 2, 0]; byte_len = [1, 2, 2]; "
                       "sum bytes over scored rows = 3; bpb = 3 ln 2 / (3 ln 2) = 1."),
        "softcap": 0.0,
        "hidden": [[1.0], [1.0], [1.0]],
        "embed": [[LN2], [0.0], [0.0]],
        "target": [0, 1, 2],
        "mask": [1, 1, 0],
        "byte_len": [1, 2, 2],
        "expected": {"nats": [LN2, 2 * LN2, 0.0], "lse": [2 * LN2, 2 * LN2, 0.0], "sum_nats": 3 * LN2,
                     "sum_bytes": 3, "n_scored": 2, "bpb": 1.0},
    }


def stride64():
    return {
        "what": "scored rows of a stride-64 sliding-window evaluation over 2048-token windows",
        "source": ("parameter-golf README leaderboard, 'Sliding Window Eval' row (stride=64); window length 2048 from "
                   "the '2048 seq length' row and the HYDRA Golf 'Core GPT' card (seq 2048)."),
        "derivation": "each 2048-row window scores its last 64 rows: positions 1984..2047 of every window",
        "T": 4096, "seq_len": 2048, "stride": 64,
        "scored_rows": list(range(1984, 2048)) + list(range(4032, 4096)),
    }


def uniform():
    return {
        "what": "uniform logits: every entry equally likely, so the loss is ln V nats",
        "source": ("definition only (cross-entropy of a uniform distribution); vocab sizes from the pages "
                   "(1024, 8192 BPE; HYDRA Golf 'Core GPT', README 'Naive Baseline')."),
        "derivation": "E = 0 or H = 0 gives z = 0, s = 0 for every v, lse = ln V, nats = ln V = k ln 2 for V = 2^k",
        "cases": [{"V": V, "nats": math.log(V)} for V in (128, 512, 1024, 8192)],
    }


def _half_even(x):
    """Nearest integer to the Fraction x, a tie going to the even neighbour (the definition, spelled out)."""
    f = x.numerator // x.denominator          # floor
    d = x - f
    if d > Fraction(1, 2):
        return f + 1
    if d < Fraction(1, 2):
        return f
    return f if f % 2 == 0 else f + 1


def _bf16_nearest(x):
    """The bfloat16 value nearest to the Fraction x > 0 (8 significant bits), ties to the even
    significand: x = m 2^e with 2^7 <= m < 2^8 rounded to an integer by _half_even."""
    e = x.numerator.bit_length() - x.denominator.bit_length() - 7
    while x / Fraction(2) ** e >= 256:
        e += 1
    while x / Fraction(2) ** e < 128:
        e -= 1
    return _half_even(x / Fraction(2) ** e) * Fraction(2) ** e


def _f32_bits(v):
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def rounding_ties():
    # 1. int8 codes of rows whose quotients E / scale are exact halves
    units = [127.0, 0.5, 1.5, 2.5, 3.5, 126.5, -0.5, -1.5, -2.5, -3.5, -125.5, 64.5, 63.5, 0.0, 10.0, -127.0]
    exps = [-6, 3]
    q8_rows = [[u * 2.0 ** e for u in units] for e in exps]
    codes = [_half_even(Fraction(u)) for u in units]
    # 2. bfloat16 rounding of q * scale where the product lies halfway between two bfloat16 values:
    #    scale = 1 + 2^-8 (float32-exact); for q = 2^k, q * scale = 2^k + 2^(k-8) is a tie
    scale = 1.0 + 2.0 ** -8
    qs = [1, 2, 4, 8, 16, 32, 64, 127, 3, 5, 96, -1, -2, -64, -3, 0] * 2
    dq_rows = [[q * scale for q in qs[:16]] + [q * scale for q in qs[16:]]]
    deq = [float(_bf16_nearest(Fraction(abs(q) * scale)) * (1 if q >= 0 else -1)) if q else 0.0 for q in qs]
    # 3. float32 -> bfloat16 for values exactly halfway (and one bit either side)
    f32 = [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), -(1.0 + 3 * 2.0 ** -8),
           1.0 + 2.0 ** -8 + 2.0 ** -23, 1.0 + 2.0 ** -8 - 2.0 ** -23, 3.0 * 2.0 ** -100 * (1 + 2.0 ** -8),
           255.0 + 0.5, 254.0 + 0.5]
    bf = [float(_bf16_nearest(Fraction(abs(v))) * (1 if v >= 0 else -1)) for v in f32]
    return {
        "what": "round-half-to-even ties of the int8 quantiser, of its bfloat16 dequantisation and of float32 -> bfloat16",
        "source": ("definition only: the quantised tied head's format is a reading (the pages name int8 quantisation, "
                   "trios issue #19, approach table; README leaderboard, GPTQ and LQER rows, without a format); the "
                   "reading fixes round-half-to-even at both steps, as bfloat16 conversion does"),
        "derivation": ("q8: rows units[i] * 2^e with max |unit| = 127, so scale = 2^e exactly and E / scale = units[i]; "
                       "an exact half k + 1/2 goes to the even one of k, k + 1. dequantised: scale = 1 + 2^-8, "
                       "q * scale = 2^k + 2^(k-8) for q = 2^k lies halfway between 2^k and 2^k + 2^(k-7) and goes "
                       "to 2^k (even significand); other q by the nearest 8-bit significand. f32_to_bf16: the same "
                       "rule for values given by their float32 bit patterns. Expected values by exact rational "
                       "arithmetic (fractions.Fraction), not by a rounding routine."),
        "q8": {"exponents": exps, "units": units, "rows": q8_rows, "codes": codes,
               "scales": [2.0 ** e for e in exps]},
        "dequant": {"scale": scale, "codes": qs, "rows_f32": dq_rows, "bf16": deq},
        "f32_to_bf16": {"f32_bits": [_f32_bits(v) for v in f32], "bf16_bits": [_f32_bits(v) >> 16 for v in bf],
                        "bf16": bf},
    }


def window_schedules():
    # written out by hand from the rule; nothing here is computed
    return {
        "what": "scored predictions of each window of a sliding-window evaluation of a token stream",
        "source": ("parameter-golf README leaderboard, 'Sliding Window Eval' row (stride 64, each scored token with a "
                   "long context); the rule for the first window and the stream's end is the reading taken"),
        "derivation": ("prediction p (p = 0 .. n_tokens - 2) is token p + 1 after tokens 0..p; window w covers input "
                       "positions w*stride .. w*stride + window - 1 and scores the predictions there that no earlier "
                       "window scored, until all are scored. E.g. n_tokens = 14, window 8, stride 2: 13 predictions; "
                       "window 0 (positions 0-7) scores 0-7, window 1 (2-9) adds 8, 9, window 2 (4-11) adds 10, 11, "
                       "window 3 (6-13) adds 12 (13 predicts past the end)."),
        "cases": [
            {"n_tokens": 14, "window": 8, "stride": 2,
             "windows": [[0, 1, 2, 3, 4, 5, 6, 7], [8, 9], [10, 11], [12]]},
            {"n_tokens": 5, "window": 8, "stride": 2, "windows": [[0, 1, 2, 3]]},
            {"n_tokens": 1, "window": 8, "stride": 2, "windows": []},
            {"n_tokens": 10, "window": 8, "stride": 8, "windows": [[0, 1, 2, 3, 4, 5, 6, 7], [8]]},
            {"n_tokens": 8, "window": 4, "stride": 1, "windows": [[0, 1, 2, 3], [4], [5], [6]]},
            {"n_tokens": 12, "window": 6, "stride": 4, "windows": [[0, 1, 2, 3, 4, 5], [6, 7, 8, 9], [10]]},
        ],
    }


if __name__ == "__main__":
    for name, obj in [("worked_softcap30.json", worked_softcap30()),
                      ("worked_nocap_one_bit_per_byte.json", worked_nocap()),
                      ("worked_asym_softcap_30_10.json", worked_asym()),
                      ("stride64_windows.json", stride64()), ("uniform_logits.json", uniform()),
                      ("rounding_ties.json", rounding_ties()), ("window_schedules.json", window_schedules())]:
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(obj, f, indent=1)
            f.write("\n")
