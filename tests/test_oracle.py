"""CPU tests of the oracle: every pin, plus a mutation check showing that the
pins catch plausible mistakes planted in copies of the oracle (on the CPU)."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

import oracle
from tests import oracle_pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# (description, exact text in dsa_oracle.c, replacement).  Each is a mistake a
# careful reader could plausibly make; every one must trip at least one pin.
MUTATIONS = [
    ("relu dropped", "double relu = dot > 0.0 ? dot : 0.0;", "double relu = dot;"),
    ("mask excludes the diagonal", "if (j > p) { Srow[j] = -INFINITY; continue; }",
     "if (j >= p) { Srow[j] = -INFINITY; continue; }"),
    ("head weight dropped", "total += (double)wrow[h] * relu;", "total += relu;"),
    ("indexer head stride", "qIrow[(int64_t)h * Di + d]", "qIrow[d]"),
    ("indexer key transposed", "kId[j * Di + d]", "kId[d * Di + (j % Di)]"),
    ("ties to the higher key", "return (x->j < y->j) ? -1 : (x->j > y->j);",
     "return (x->j > y->j) ? -1 : (x->j < y->j);"),
    ("lowest scores kept", "if (x->s > y->s) return -1;\n    if (x->s < y->s) return 1;",
     "if (x->s < y->s) return -1;\n    if (x->s > y->s) return 1;"),
    ("dense rule reports top_k keys", "*count = (int32_t)n;", "*count = top_k;"),
    ("dense rule skips the diagonal key", "for (int64_t j = 0; j < n; ++j) idxrow[j] = (int32_t)j;",
     "for (int64_t j = 0; j + 1 < n; ++j) idxrow[j] = (int32_t)j;"),
    ("selection left in score order",
     "qsort(idxrow, (size_t)top_k, sizeof(int32_t), ascending_int);", ""),
    ("softmax scale dropped", "s[t] = scale * dot;", "s[t] = dot;"),
    ("value taken from the rope end", "const double* v = kvd + (int64_t)sel[t] * Dqk;",
     "const double* v = kvd + (int64_t)sel[t] * Dqk + (Dqk - Dv);"),
    ("query head stride", "const double* qh = qrow + (int64_t)h * Dqk;",
     "const double* qh = qrow;"),
    ("softmax not normalised", "double pt = exp(s[t] - m) / Z;", "double pt = exp(s[t] - m);"),
    ("lse without log", "lserow[h] = m + log(Z);", "lserow[h] = m + Z;"),
    ("score rounded to bf16-ish", "Srow[j] = (float)total;",
     "Srow[j] = (float)(total + 0.25);"),
    ("rope turns the other way", "x[2 * i] = a * c - b * s;\n        x[2 * i + 1] = a * s + b * c;",
     "x[2 * i] = a * c + b * s;\n        x[2 * i + 1] = -a * s + b * c;"),
    ("rope pairs half a width apart", "double a = x[2 * i], b = x[2 * i + 1];\n        x[2 * i] = a * c - b * s;\n        x[2 * i + 1] = a * s + b * c;",
     "double a = x[i], b = x[i + d / 2];\n        x[i] = a * c - b * s;\n        x[i + d / 2] = a * s + b * c;"),
    ("rope exponent i/d", "double ang = p * pow(theta, -2.0 * i / d);", "double ang = p * pow(theta, -1.0 * i / d);"),
    ("rope position off by one", "double p = (double)pos[t];", "double p = (double)pos[t] + 1.0;"),
    ("rms over the sum", "double r = 1.0 / sqrt(ss / n + eps);", "double r = 1.0 / sqrt(ss + eps);"),
    ("eps outside the root", "double r = 1.0 / sqrt(ss / n + eps);", "double r = 1.0 / (sqrt(ss / n) + eps);"),
    ("norm weight dropped", "x[k] = x[k] * r * (double)w[k];", "x[k] = x[k] * r;"),
    ("indexer rope over the whole head", "rope_norm(tmp, d_idx_rope, p, theta);", "rope_norm(tmp, Di, p, theta);"),
    ("k_pe not roped", "rope_norm(tmp + Dl, Dr, p, theta);", ""),
    ("q rope at column 0", "rope_rows_bf16(q + t * H * Dqk, H, Dqk, Dl, Dr, p, theta, tmp);",
     "rope_rows_bf16(q + t * H * Dqk, H, Dqk, 0, Dr, p, theta, tmp);"),
    ("bf16 rounding truncates", "double r = nearbyint(ldexp(m, 8));", "double r = floor(ldexp(m, 8));"),
    ("router weights take the biased score", "weights[t * k + j] = (double)p[key[j].e] / den * scale;",
     "weights[t * k + j] = (double)key[j].s / den * scale;"),
    ("router weights not normalised", "weights[t * k + j] = (double)p[key[j].e] / den * scale;",
     "weights[t * k + j] = (double)p[key[j].e] * scale;"),
    ("router clamp ignored", "double den = sum > min_sum ? sum : min_sum;", "double den = sum;"),
    ("router ties to the higher expert", "return (x->e < y->e) ? -1 : (x->e > y->e);",
     "return (x->e > y->e) ? -1 : (x->e < y->e);"),
    ("router keeps the lowest scores", "if (x->s != y->s) return x->s > y->s ? -1 : 1;",
     "if (x->s != y->s) return x->s < y->s ? -1 : 1;"),
    ("router sigmoid sign", "p[e] = (float)(1.0 / (1.0 + exp(-(double)lg[e])));",
     "p[e] = (float)(1.0 / (1.0 + exp((double)lg[e])));"),
    ("router bias ignored", "key[e].s = p[e] + bias[e];", "key[e].s = p[e];"),
    ("up-projection weight read transposed", "const uint16_t* wrow = wv + ((int64_t)h * Dv + j) * Dl;\n                double acc = 0.0;\n                for (int32_t c = 0; c < Dl; ++c) acc += x[c] * bf16_to_double(wrow[c]);",
     "const uint16_t* wrow = wv + (int64_t)h * Dv * Dl;\n                double acc = 0.0;\n                for (int32_t c = 0; c < Dl; ++c) acc += x[c] * bf16_to_double(wrow[((int64_t)c * Dv + j) % ((int64_t)Dv * Dl)]);"),
    ("up-projection head ignored", "const uint16_t* wrow = wv + ((int64_t)h * Dv + j) * Dl;",
     "const uint16_t* wrow = wv + ((int64_t)j) * Dl;"),
    ("attention output not rounded to bf16", "x[c] = bf16_to_double(double_to_bf16((double)orow[c]));",
     "x[c] = (double)orow[c];"),
    ("o_proj weight read transposed", "const uint16_t* wrow = wo + (int64_t)n * Kin;\n            double acc = 0.0;\n            for (int32_t k = 0; k < Kin; ++k) acc += xr[k] * bf16_to_double(wrow[k]);",
     "double acc = 0.0;\n            for (int32_t k = 0; k < Kin; ++k) acc += xr[k] * bf16_to_double(wo[((int64_t)k * Nout + n) % ((int64_t)Nout * Kin)]);"),
    ("positions taken as 1-based rows", "uint16_t* dst = kv_cache + pos[t] * Dqk;",
     "uint16_t* dst = kv_cache + (pos[t] > 0 ? pos[t] - 1 : 0) * Dqk;"),
    ("dense rope term dropped",
     "for (int32_t d = 0; d < x->Dr; ++d) dot += bf16_to_double(qh[x->Dn + d]) * bf16_to_double(kp[d]);", ""),
    ("dense value read from the key columns", "const uint16_t* v = x->kvb + (j * x->H + h) * Dkv + x->Dn;",
     "const uint16_t* v = x->kvb + (j * x->H + h) * Dkv;"),
    ("dense key ignores the head", "const uint16_t* kn = x->kvb + (j * x->H + h) * Dkv;",
     "const uint16_t* kn = x->kvb + (j * x->H) * Dkv;"),
    ("dense mask bits reversed", "if (!((mrow[j / 32] >> (j % 32)) & 1u))", "if (!((mrow[j / 32] >> (31 - j % 32)) & 1u))"),
    ("dense softmax scale dropped", "s[j] = x->scale * dot;", "s[j] = dot;"),
    ("dense softmax not normalised", "const double pj = exp(s[j] - m) / Z;", "const double pj = exp(s[j] - m);"),
    ("mask keeps non-causal keys", "if (j >= 0 && j < N && j <= p) row[j / 32]", "if (j >= 0 && j < N) row[j / 32]"),
    ("mask ignores count", "for (int32_t t = 0; t < c; ++t) {\n            const int64_t j = idx[i * top_k + t];",
     "for (int32_t t = 0; t < top_k; ++t) {\n            const int64_t j = idx[i * top_k + t];"),
    ("kv_b weight read transposed", "const uint16_t* wrow = w + ((int64_t)h * C + c) * Dl;\n                double acc = 0.0;\n                for (int32_t d = 0; d < Dl; ++d) acc += x[d] * bf16_to_double(wrow[d]);",
     "const uint16_t* wrow = w + ((int64_t)h * C + c) * Dl;\n                double acc = 0.0;\n                for (int32_t d = 0; d < Dl; ++d) acc += x[d] * bf16_to_double(w[((int64_t)h * C + (d % C)) * Dl + (c % Dl)]);"),
    ("kv_b values left in bf16", "(values_f16 && c >= Dn) ? double_to_f16(acc) : double_to_bf16(acc)", "double_to_bf16(acc)"),
    ("fp16 rounding truncates", "double n = nearbyint(ldexp(m, 11));", "double n = floor(ldexp(m, 11));"),
    ("fp16 subnormals flushed", "const double n = nearbyint(ldexp(a, 24));   /* 1024 lands on the smallest normal */",
     "const double n = 0.0;"),
    ("absorption reads the value rows", "acc += qn[c] * bf16_to_double(w[((int64_t)h * C + c) * Dl + d]);",
     "acc += qn[c] * bf16_to_double(w[((int64_t)h * C + Dn + c % (Dv > 0 ? Dv : 1)) * Dl + d]);"),
    ("absorption weight transposed", "acc += qn[c] * bf16_to_double(w[((int64_t)h * C + c) * Dl + d]);",
     "acc += qn[c] * bf16_to_double(w[((int64_t)h * C + (d % C)) * Dl + (c % Dl)]);"),
    ("absorption head stride dropped", "acc += qn[c] * bf16_to_double(w[((int64_t)h * C + c) * Dl + d]);",
     "acc += qn[c] * bf16_to_double(w[((int64_t)c) * Dl + d]);"),
    ("absorption rope not copied", "for (int32_t r = 0; r < Dr; ++r) orow[Dl + r] = qrow[Dn + r];",
     "for (int32_t r = 0; r < Dr; ++r) orow[Dl + r] = 0;"),
]

_RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
import oracle
from tests import oracle_pins
failed = []
with oracle.using_library({lib!r}):
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception as e:   # AssertionError or an oracle error code
            failed.append(pin.__name__)
print("FAILED_PINS", len(failed), failed)
"""


@pytest.mark.parametrize("desc,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(desc, old, new, tmp_path):
    src = open(os.path.join(ROOT, "oracle", "dsa_oracle.c")).read()
    assert src.count(old) == 1, "mutation anchor not found exactly once: %r" % old
    d = tmp_path
    shutil.copy(os.path.join(ROOT, "oracle", "dsa_oracle.h"), d / "dsa_oracle.h")
    (d / "dsa_oracle.c").write_text(src.replace(old, new))
    lib = str(d / "libmutant.so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", lib,
                    str(d / "dsa_oracle.c"), "-lm"], check=True)
    r = subprocess.run([sys.executable, "-c", _RUNNER.format(root=ROOT, lib=lib)],
                       capture_output=True, text=True, timeout=600)
    # a crash of the mutant also counts as caught
    if r.returncode == 0:
        line = [l for l in r.stdout.splitlines() if l.startswith("FAILED_PINS")][-1]
        assert int(line.split()[1]) > 0, "planted mistake '%s' passed every pin" % desc
