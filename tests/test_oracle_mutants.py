"""Plant plausible mistakes in copies of the oracle and check that the pins
catch every one (CPU only).  The mistakes live only in temporary copies of
oracle.c; the oracle itself is never modified."""
import pytest

import oracle
from tests import oracle_pins

# (name, exact text in oracle.c, replacement)
MUTANTS = [
    ("dropped last term",
     "for (int64_t k = 0; k < H; ++k) acc += bf16_value(x[k]) * bf16_value(wv[k]);",
     "for (int64_t k = 0; k + 1 < H; ++k) acc += bf16_value(x[k]) * bf16_value(wv[k]);"),
    ("transposed operand",
     "acc += bf16_value(x[k]) * bf16_value(wv[k]);",
     "acc += bf16_value(x[k]) * bf16_value(w[(k * V + v) % (V * H)]);"),
    ("int dropped term",
     "for (int64_t k = 0; k < H; ++k) acc += (int64_t)x[k] * (int64_t)wv[k];",
     "for (int64_t k = 1; k < H; ++k) acc += (int64_t)x[k] * (int64_t)wv[k];"),
    ("int wrong row stride",
     "const int8_t *x = (const int8_t *)j->x + r * H;",
     "const int8_t *x = (const int8_t *)j->x + r;"),
    ("top-1 ties to highest id",
     "if (i1 < 0 || t > b1) {\n      b2 = b1; i2 = i1;\n      b1 = t; i1 = v;\n    } else if (i2 < 0 || t > b2) {\n      b2 = t; i2 = v;\n    }\n  }\n  ids[0] = (int32_t)i1; ids[1] = (int32_t)i2;\n  vals[0] = b1; vals[1] = b2;\n}\n\nvoid oracle_top2_i64",
     "if (i1 < 0 || t >= b1) {\n      b2 = b1; i2 = i1;\n      b1 = t; i1 = v;\n    } else if (i2 < 0 || t > b2) {\n      b2 = t; i2 = v;\n    }\n  }\n  ids[0] = (int32_t)i1; ids[1] = (int32_t)i2;\n  vals[0] = b1; vals[1] = b2;\n}\n\nvoid oracle_top2_i64"),
    ("top-2 ties to highest id",
     "} else if (i2 < 0 || t > b2) {",
     "} else if (i2 < 0 || t >= b2) {"),
    ("top-2 drops the old top-1",
     "b2 = b1; i2 = i1;",
     "(void)0;"),
    ("log-softmax wrong sign",
     "for (int64_t v = 0; v < V; ++v) out[v] = z[v] - lse;",
     "for (int64_t v = 0; v < V; ++v) out[v] = z[v] + lse - 2.0 * m;"),
    ("log-prob missing max",
     "return z[t] - (m + log(s));",
     "return z[t] - log(s);"),
    ("log-prob sum skips first entry",
     "for (int64_t v = 0; v < V; ++v) s += exp(z[v] - m);\n  return z[t] - (m + log(s));",
     "for (int64_t v = 1; v < V; ++v) s += exp(z[v] - m);\n  return z[t] - (m + log(s));"),
    ("int log-prob drops the scale",
     "for (int64_t v = 0; v < V; ++v) s += exp(scale * (double)(z[v] - zmax));",
     "for (int64_t v = 0; v < V; ++v) s += exp((double)(z[v] - zmax));"),
    ("int scale applied in float32",
     "return (float)((double)z * (double)s);",
     "return (float)z * s;"),
    ("bf16 rounding ties away from zero",
     "double q = nearbyint(ldexp(m, p));",
     "double q = round(ldexp(m, p));"),
    ("margin sign",
     "j->margin_d[r] = vals[0] - vals[1];",
     "j->margin_d[r] = vals[1] - vals[0];"),
    ("integer exp: Horner sign",
     "y = c - rnd(y * r, FIX_NATS);",
     "y = c + rnd(y * r, FIX_NATS);"),
    ("integer exp: coefficient off by one",
     "const uint64_t c = rnd_div((uint64_t)1 << FIX_EXP, factorial(n));",
     "const uint64_t c = rnd_div((uint64_t)1 << FIX_EXP, factorial(n + 1));"),
    ("integer ln: atanh without its factor 2",
     "* (int64_t)ln2_fixed(FIX_EXP) + 2 * (int64_t)acc;",
     "* (int64_t)ln2_fixed(FIX_EXP) + (int64_t)acc;"),
    ("integer softmax: block rescale dropped",
     "S += ((Sb >> 32) * R << 2) + rnd((Sb & 0xffffffffu) * R, FIX_EXP);",
     "S += Sb + 0 * R;"),
    ("integer softmax: scale shift off by one",
     "const int sh = k - FIX_NATS;",
     "const int sh = k - FIX_NATS + 1;"),
    ("quantise: rounds toward zero",
     "const int64_t r = (int64_t)((2 * n + D) / (2 * D));",
     "const int64_t r = (int64_t)(n / D);"),
    ("quantise: step rounded down",
     "mm = ((a << (-ee)) + 126) / 127;",
     "mm = (a << (-ee)) / 127;"),
    ("Philox: key not bumped between rounds",
     "if (r) { k0 += W0; k1 += W1; }",
     "if (r) { k0 += 0 * W0; k1 += W1; }"),
    ("Philox: counter words 1 and 3 swapped in the mix",
     "uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0, y1 = (uint32_t)p1;",
     "uint32_t y0 = (uint32_t)(p1 >> 32) ^ x3 ^ k0, y1 = (uint32_t)p1;"),
    ("Gumbel: low bits of the word",
     "const uint32_t u = out[(v >> 5) & 3] >> 9;",
     "const uint32_t u = out[(v >> 5) & 3] & 0x7fffffu;"),
    ("Gumbel: word of the wrong column tile",
     "const uint32_t u = out[(v >> 5) & 3] >> 9;",
     "const uint32_t u = out[(v >> 6) & 3] >> 9;"),
    ("Gumbel: position in the key instead of the counter",
     "const uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};",
     "const uint32_t key[2] = {(uint32_t)seed, (uint32_t)pos};"),
    ("row scale: exponent sign",
     "const int64_t kk = -((int64_t)sh + ue + E);",
     "const int64_t kk = -((int64_t)sh + ue - E);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = oracle.SOURCE.read_text()
    assert src.count(old) >= 1, f"mutation site for {name!r} not found"
    (tmp_path / "oracle.c").write_text(src.replace(old, new))
    lib = oracle.compile_source(tmp_path / "oracle.c", tmp_path / "mutant.so")
    o = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.FAST:
        try:
            pin(o)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name!r}"
