"""Mutation check of the oracle's pins (CPU only).

Each mutant below is kv_oracle.c with one plausible mistake planted in it: a
wrong index, a dropped term, a swapped operand, a wrong constant or rounding
rule.  The mutant is compiled on its own and the oracle pin suite
(test_oracle_pins.py) runs against it through KVO_ORACLE_LIB; the pins must
fail for every mutant, and pass for an unmodified copy built the same way.
A mutant whose text no longer occurs exactly once in kv_oracle.c fails the
test too, so the list cannot silently go stale."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kv_oracle.c")

# (name, text in kv_oracle.c, replacement)
MUTANTS = [
    ("slot: row taken from the next token",
     "return (int64_t)block_table[t / page_size] * page_size + t % page_size;",
     "return (int64_t)block_table[t / page_size] * page_size + (t + 1) % page_size;"),
    ("slot: page stride one row short",
     "return (int64_t)block_table[t / page_size] * page_size + t % page_size;",
     "return (int64_t)block_table[t / page_size] * (page_size - 1) + t % page_size;"),
    ("chunk count drops the partial tail",
     "return (e - s + chunk_size - 1) / chunk_size;",
     "return (e - s) / chunk_size;"),
    ("sections: K and V swapped",
     "if (ll == l && k == kv) return off;\n            off += n_c * width",
     "if (ll == l && k != kv) return off;\n            off += n_c * width"),
    ("scales: one per part even for bf16 parts",
     "if (part_kind(fmt, k) != PART_BF16) off += 4;",
     "off += 4;"),
    ("hits: every set flag counted, holes ignored",
     "while (c < n_chunks && mask[c] != 0) c++;",
     "for (int64_t i = 0; i < n_chunks; i++) c += mask[i] != 0;"),
    ("retrieve: tail counted as a full chunk",
     "for (int64_t c = 0; c < n_hit; c++) tokens += kvo_chunk_tokens(s, e, p->chunk_size, c);\n    for (int64_t c = 0; c < n_hit; c++) {\n        if (chunks[c] == NULL) return -1;\n    }\n    /* two writes",
     "for (int64_t c = 0; c < n_hit; c++) tokens += p->chunk_size;\n    for (int64_t c = 0; c < n_hit; c++) {\n        if (chunks[c] == NULL) return -1;\n    }\n    /* two writes"),
    ("layerwise retrieve: every layer but the named one",
     "if (layer >= 0 && l != layer) continue;\n            for (int kv = 0; kv < 2; kv++) {\n                int kind = part_kind(fmt, kv);\n                const uint8_t* sec",
     "if (layer >= 0 && l == layer) continue;\n            for (int kv = 0; kv < 2; kv++) {\n                int kind = part_kind(fmt, kv);\n                const uint8_t* sec"),
    ("bf16 rounding one bit short",
     "double q = ldexp(1.0, E - 7); /* spacing of bf16 values around a */",
     "double q = ldexp(1.0, E - 8); /* spacing of bf16 values around a */"),
    ("e4m3: subnormal range starts one binade low",
     "if (E < -6) E = -6;",
     "if (E < -7) E = -7;"),
    ("e4m3: overflow gives NaN instead of saturating",
     "if (v > 448.0) return (uint8_t)(sign | 0x7E);",
     "if (v > 448.0) return (uint8_t)(sign | 0x7F);"),
    ("e4m3 decode: subnormal step halved",
     "if (e == 0) v = m * ldexp(1.0, -9);",
     "if (e == 0) v = m * ldexp(1.0, -10);"),
    ("e5m2: mantissa rounded with e4m3 spacing",
     "double q = ldexp(1.0, E - 2); /* spacing of E5M2 values around a */",
     "double q = ldexp(1.0, E - 3); /* spacing of E5M2 values around a */"),
    ("fp8 scale maps amax to 447",
     "return amax / 448.0f;",
     "return amax / 447.0f;"),
    ("fp8 group maximum ignores NaN",
     "if (saw_nan) scale = default_nan();",
     "if (0) scale = default_nan();"),
    ("fp8 NaN quotient takes the sign the division gives",
     "if (isnan(y)) code = nan_code(xb);",
     "if (isnan(y)) code = kind == PART_E4M3 ? kvo_e4m3_encode(y) : kvo_e5m2_encode(y);"),
    ("fp8 dequantised NaN left to the product",
     "if (isnan(prod)) x = nan_bf16(*src >> 7);",
     "if (0) x = nan_bf16(*src >> 7);"),
    ("CacheGen: max1 of a NaN row left finite",
     "if (saw_nan) max1 = default_nan();",
     "if (0) max1 = default_nan();"),
    ("CacheGen dequantised NaN left to the product",
     "isnan(x) ? nan_bf16(0) : kvo_bf16_from_float(x)",
     "kvo_bf16_from_float(x)"),
    ("fp8 quotient by reciprocal product",
     "float y = x / scale;          /* binary32 division */",
     "float y = x * (1.0f / scale);"),
    ("fp8 dequantise divides by the scale",
     "float prod = d * scale;       /* binary32 product */",
     "float prod = d / scale;"),
    ("CacheGen: MAX = bins / 2",
     "return bins[l] / 2 - 1;",
     "return bins[l] / 2;"),
    ("CacheGen: ties rounded away from zero",
     "float r = nearbyintf(y);            /* ties to even */",
     "float r = roundf(y);"),
    ("CacheGen: factor as a reciprocal product",
     "float factor = max1 == 0.0f ? 0.0f : (float)MAX / max1;",
     "float factor = max1 == 0.0f ? 0.0f : (float)MAX * (1.0f / max1);"),
    ("CacheGen: scale and offset fused into one rounding",
     "float y = scaled + (float)MAX;          /* binary32 sum */",
     "float y = fmaf(x, factor, (float)MAX);"),
    ("CacheGen dequantise: product before the quotient",
     "float unit = centred / (float)MAX;           /* binary32 quotient */\n                        float x = unit * max1;",
     "float unit = centred * max1;\n                        float x = unit / (float)MAX;"),
    ("CacheGen: max1 of the K rows stored for V",
     "memcpy(max_area + 4 * cg_row(p, l, kv, n_c, j), &max1, 4);",
     "memcpy(max_area + 4 * cg_row(p, l, 0, n_c, j), &max1, 4);"),
]

FLAGS = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def _build(src_text, tmp, name):
    c = os.path.join(tmp, name + ".c")
    so = os.path.join(tmp, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(FLAGS + ["-I", os.path.join(ROOT, "oracle"), "-o", so, c, "-lm"], check=True)
    return so


def _pins(so):
    env = dict(os.environ, KVO_ORACLE_LIB=so)
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        "-x", "-q", "-p", "no:cacheprovider"], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=600)
    return r.returncode, r.stdout[-2000:]


def test_every_mutant_is_caught_by_the_pins(tmp_path):
    text = open(SRC).read()
    for name, old, new in MUTANTS:
        assert text.count(old) == 1, f"mutant '{name}': its text occurs {text.count(old)} times in kv_oracle.c"
    jobs = [("control", _build(text, str(tmp_path), "control"))]
    for k, (name, old, new) in enumerate(MUTANTS):
        jobs.append((name, _build(text.replace(old, new), str(tmp_path), f"mutant{k}")))
    with ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda j: (j[0],) + _pins(j[1]), jobs))
    control = results[0]
    assert control[1] == 0, "the unmodified oracle must pass its pins:\n" + control[2]
    missed = [name for name, rc, out in results[1:] if rc == 0]
    assert not missed, f"pins did not catch: {missed}"
    crashed = [name for name, rc, out in results[1:] if rc != 0 and "failed" not in out]
    assert not crashed, f"mutants that crashed instead of failing a pin: {crashed}"
