"""Planted mistakes in a copy of the oracle source must fail a pin.

Each mutation is a plausible slip (a dropped term, a wrong sign, index or
operand); the mutated copy is built in a temporary directory and the pins are
run against it in a child process."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "pkv_oracle.c")
RUNNER = os.path.join(ROOT, "tests", "pin_runner.py")

MUTATIONS = [
    ("softmax sign", "score[t - t0] = exp(score[t - t0] - m);", "score[t - t0] = exp(m - score[t - t0]);"),
    ("dropped scale", "return p->scale * dot;", "return dot;"),
    ("kv head by modulo", "int32_t kvh = h / (p->Hq / p->Hkv);", "int32_t kvh = h % p->Hkv;"),
    ("slot from quotient", "int64_t slot = t % p->B;", "int64_t slot = t / p->B;"),
    ("table bypassed", "int64_t block = p->block_tables[(size_t)s * p->M + block_idx];",
     "int64_t block = block_idx;"),
    ("value transposed", "return (size_t)(b * kv_block_stride + h * kv_head_stride + d * B + t);",
     "return (size_t)(b * kv_block_stride + h * kv_head_stride + t * hs + d);"),
    ("key chunk stride", "+ (d / x) * ((int64_t)B * x) + t * x + d % x);", "+ t * hs + d);"),
    ("new token position", "orc_slot_of_position(block_tables + (size_t)s * M, L - 1, B)",
     "orc_slot_of_position(block_tables + (size_t)s * M, (L - 1) / 2, B)"),
    ("no normalisation", "for (int32_t d = 0; d < p->hs; ++d) o[d] /= l;", ""),
    ("merge weight sign", "double w = pl[k] * exp(pm[k] - Mx);", "double w = pl[k] * exp(Mx - pm[k]);"),
    ("slot offset", "int64_t offset_in_block = pos % B;", "int64_t offset_in_block = 0;"),
    ("fp8 exponent bias", "v = (1.0 + m / 8.0) * ldexp(1.0, e - 7);", "v = (1.0 + m / 8.0) * ldexp(1.0, e - 8);"),
    ("fp8 subnormal scale", "v = m * ldexp(1.0, -9);", "v = m * ldexp(1.0, -10);"),
    ("fp8 ties away from even", "(err == best_err && (c & 1) == 0 && (best & 1) == 1)", "(err == best_err)"),
    ("fp8 overflow to NaN", "if (a > 448.0)\\n        return sign | 0x7E;", "if (a > 448.0)\\n        return sign | 0x7F;"),
    ("fp8 value scale on keys", "double kd = p->k_scale *", "double kd = p->v_scale *"),
    ("causal limit excludes own token", "orc_attend_range(&p, s, qr, h, 0, pos + 1, score, &m, &l, out + (size_t)u * hs);",
     "orc_attend_range(&p, s, qr, h, 0, pos, score, &m, &l, out + (size_t)u * hs);"),
    ("query rows counted from the start", "int64_t pos = (int64_t)seq_lens[s] - n + (qr - q_start[s]);",
     "int64_t pos = qr - q_start[s];"),
    ("query row of the sequence", "double qd = orc_load(p->q, ((size_t)qr * p->Hq + h) * p->hs + d, p->dtype);",
     "double qd = orc_load(p->q, ((size_t)s * p->Hq + h) * p->hs + d, p->dtype);"),
    ("multi-token slot from the start", "int64_t pos = L - n + i;", "int64_t pos = i;"),
    ("fp8 key chunk of 8", "k_pool[orc_key_index(b, h, off, d, Hkv, B, hs, 16)]", "k_pool[orc_key_index(b, h, off, d, Hkv, B, hs, 8)]"),
]


def build(src_text, out_dir):
    c = os.path.join(out_dir, "m.c")
    so = os.path.join(out_dir, "m.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.check_call(["gcc", "-O1", "-std=c11", "-fopenmp", "-shared", "-fPIC", c, "-o", so, "-lm"])
    return so


def run_pins(so):
    env = dict(os.environ, OMP_NUM_THREADS="2")
    return subprocess.run([sys.executable, RUNNER, so], capture_output=True, text=True, timeout=300, env=env)


def test_unmutated_source_passes(tmp_path):
    src = open(SRC).read()
    r = run_pins(build(src, str(tmp_path)))
    assert r.returncode == 0, r.stdout + r.stderr


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    old, new = old.replace("\\n", "\n"), new.replace("\\n", "\n")
    assert src.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    r = run_pins(build(src.replace(old, new), str(tmp_path)))
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin"
