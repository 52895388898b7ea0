"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of ``oracle/gdr_oracle.c`` with one plausible mistake
planted by text substitution (a dropped term, a wrong sign, a wrong index, a
swapped read mode ...). The copy is compiled into a temporary library and the
pins of ``test_oracle_pins.py`` are run against it: at least one must fail.
The real oracle source is never modified.
"""
from __future__ import annotations

import os
import subprocess

import pytest

import oracle
from tests.test_oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "gdr_oracle.c")

# (name, original text, replacement, which occurrence (0-based))
MUTANTS = [
    ("erase_dropped", "x[c] = b * (vt[c] - alpha * x[c]);", "x[c] = b * vt[c];", 0),
    ("erase_not_decayed", "x[c] = b * (vt[c] - alpha * x[c]);", "x[c] = b * (vt[c] - x[c]);", 0),
    ("erase_sign", "x[c] = b * (vt[c] - alpha * x[c]);", "x[c] = b * (vt[c] + alpha * x[c]);", 0),
    ("beta_on_value_only", "x[c] = b * (vt[c] - alpha * x[c]);", "x[c] = b * vt[c] - alpha * x[c];", 0),
    ("state_not_decayed", "Hr[c] = alpha * Hr[c] + kr * x[c];", "Hr[c] = Hr[c] + kr * x[c];", 0),
    ("write_decayed", "Hr[c] = alpha * Hr[c] + kr * x[c];", "Hr[c] = alpha * (Hr[c] + kr * x[c]);", 0),
    ("linear_decay", "const double alpha = exp(ah[t]);", "const double alpha = 1.0 + ah[t];", 0),
    ("beta_one", "const double b = bh[t];", "const double b = 1.0;", 0),
    ("pre_read_uses_key", "const double qr = qt[r];", "const double qr = kt[r];", 0),
    ("post_read_uses_key", "const double qr = qt[r];", "const double qr = kt[r];", 1),
    ("read_mode_swapped", "const int pre = (flags & GDR_ORACLE_READ_PRE) != 0;",
     "const int pre = (flags & GDR_ORACLE_READ_PRE) == 0;", 0),
    ("reverse_ignored", "const int64_t t = rev ? (t_end - 1 - s) : (t_begin + s);",
     "const int64_t t = t_begin + s;", 0),
    ("reverse_off_by_one", "const int64_t t = rev ? (t_end - 1 - s) : (t_begin + s);",
     "const int64_t t = rev ? (t_end - 1 - s + (s > 0)) : (t_begin + s);", 0),
    ("key_head_modulo", "const int64_t khead = head / group;", "const int64_t khead = head % Hk;", 0),
    ("h0_ignored", "if (h0) {", "if (0) {", 0),
    ("h0_wrong_segment", "memcpy(H, h0 + (seq * Hv + head) * dk * dv",
     "memcpy(H, h0 + (head) * dk * dv", 0),
    ("segment_start_skipped", "const int64_t tb = cu_seqlens ? cu_seqlens[seq] : 0;",
     "const int64_t tb = cu_seqlens ? cu_seqlens[seq] + (seq > 0) : 0;", 0),
    ("accumulate_ignored", "for (int64_t c = 0; c < dv; ++c) ot[c] += o[c];",
     "for (int64_t c = 0; c < dv; ++c) ot[c] = o[c];", 0),
    ("erase_uses_query", "x[c] += Hr[c] * kr;", "x[c] += Hr[c] * qt[r];", 0),
    ("decode_pre_reads_key", "for (int64_t c = 0; c < dv; ++c) ov[c] = y[c];",
     "for (int64_t c = 0; c < dv; ++c) ov[c] = x[c];", 0),
    ("decode_erase_not_decayed", "u[c] = b * (vv[c] - alpha * x[c]);", "u[c] = b * (vv[c] - x[c]);", 0),
    ("decode_post_reads_old_state", "ov[c] += Hn[r * dv + c] * qv[r];", "ov[c] += S[r * dv + c] * qv[r];", 0),
    ("decode_outer_transposed", "Hn[r * dv + c] = alpha * S[r * dv + c] + kv[r] * u[c];",
     "Hn[r * dv + c] = alpha * S[r * dv + c] + kv[c % dk] * u[r % dv];", 0),
    ("decode_key_head_modulo", "kh = head / group;", "kh = head % Hk;", 0),
]


def _mutate(text, old, new, occurrence):
    idx = -1
    for _ in range(occurrence + 1):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    assert src.count(old) > occ, "mutation anchor for %s not found" % name
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    c_path = tmp_path / ("%s.c" % name)
    so_path = tmp_path / ("%s.so" % name)
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-shared", "-fPIC", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    variant = oracle.Variant(str(so_path))
    caught = []
    for pin_name, fn in ALL_PINS:
        try:
            fn(variant)
        except (AssertionError, ValueError):
            caught.append(pin_name)
            break
    assert caught, "no pin catches mutant %s" % name
