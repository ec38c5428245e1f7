"""Writes the closed-form fixtures in this folder.

Every expected number here is the evaluation of a closed form stated in the fixture's
"derivation" field (Python's math module, float64). Nothing is computed by the oracle or by the
GPU library. Run from the repository root: python tests/golden/make_closed_forms.py
"""
import json
import math
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LN2 = math.log(2.0)


def worked_softcap30():
    lse = 24.0 + math.log1p(math.exp(-6.0) + math.exp(-24.0))
    nats = [lse - 18.0, lse - 24.0, lse - 0.0]
    return {
        "what": "worked example of the softcapped cross-entropy and bits per byte, values in closed form",
        "source": ("definition only: the pages print no worked example. Softcap s = c*tanh(z/c) is the reading of "
                   "'fused softcapped CE' (HYDRA Golf site stack list; parameter-golf README leaderboard, PR #1787 row); "
                   "bits per byte as in the README introduction ('evaluated by compression ... bits per byte')."),
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


if __name__ == "__main__":
    for name, obj in [("worked_softcap30.json", worked_softcap30()),
                      ("worked_nocap_one_bit_per_byte.json", worked_nocap()),
                      ("worked_asym_softcap_30_10.json", worked_asym()),
                      ("stride64_windows.json", stride64()), ("uniform_logits.json", uniform())]:
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(obj, f, indent=1)
            f.write("\n")
