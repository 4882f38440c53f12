"""Plausible mistakes planted in copies of the oracle source must each fail at
least one pin: this shows the pins can see a dropped term, a wrong sign, a
wrong index or a transposed operand anywhere in the oracle.  Mutants are built
with gcc into a temporary directory; the oracle itself is never modified."""
import os

import numpy as np
import pytest

from oracle import SRC, Oracle, build
from pins import ALL_PINS

# (name, original text, replacement, which occurrence (0-based))
MUTANTS = [
    ("eager_drop_decay", "X[(long)i * dv + j] *= w;", "X[(long)i * dv + j] *= 1.0;", 0),
    ("eager_decay_sign", "double w = exp(log_decay(op, ld, sh, dk, i));",
     "double w = exp(-log_decay(op, ld, sh, dk, i));", 1),
    ("rwkv_decay_sign", "double w = exp(log_decay(op, ld, sh, dk, i));",
     "double w = exp(-log_decay(op, ld, sh, dk, i));", 0),
    ("delta_sign", "b[j] = beta[sh] * (v[j] - acc);", "b[j] = beta[sh] * (v[j] + acc);", 0),
    ("delta_drop_beta", "b[j] = beta[sh] * (v[j] - acc);", "b[j] = (v[j] - acc);", 0),
    ("delta_transposed_read", "acc += X[(long)i * dv + j] * k[i];",
     "acc += X[(long)(j % dk) * dv + (i % dv)] * k[i];", 0),
    ("output_pre_update", "X[(long)i * dv + j] += k[i] * b[j];",
     "X[(long)i * dv + j] += 0.0 * k[i] * b[j];", 0),
    ("rank1_transposed", "X[(long)i * dv + j] += k[i] * b[j];",
     "X[(long)i * dv + j] += k[j % dk] * b[i % dv];", 0),
    ("output_uses_k", "acc += X[(long)i * dv + j] * q[i];", "acc += X[(long)i * dv + j] * k[i];", 1),
    ("rwkv_drop_bonus", "o[j] = acc + mu * v[j];", "o[j] = acc;", 0),
    ("rwkv_bonus_head_index", "mu += q[i] * u[(long)h * dk + i] * k[i];",
     "mu += q[i] * u[i] * k[i];", 0),
    ("rwkv_update_uses_q", "X[(long)i * dv + j] = w * X[(long)i * dv + j] + k[i] * v[j];",
     "X[(long)i * dv + j] = w * X[(long)i * dv + j] + q[i] * v[j];", 0),
    ("gdn_decay_wrong_index", "return op == ORC_GDN ? ld[sh] : ld[sh * dk + i];",
     "return op == ORC_GDN ? ld[0] : ld[sh * dk + i];", 0),
    ("kda_decay_wrong_index", "return op == ORC_GDN ? ld[sh] : ld[sh * dk + i];",
     "return op == ORC_GDN ? ld[sh] : ld[sh * dk + (dk - 1 - i)];", 0),
    ("dl_fold_exponent_sign", "x += exp(Ln[i] - L[(long)m * dk + i]) * a[(long)m * dk + i] *",
     "x += exp(L[(long)m * dk + i] - Ln[i]) * a[(long)m * dk + i] *", 0),
    ("dl_fold_drop_base_decay", "double base_w = exp(Ln[i]);", "double base_w = 1.0;", 0),
    ("dl_drop_k_replay", "yk += ck[m] * bl[(long)m * dv + j];", "(void)0;", 0),
    ("dl_drop_q_replay", "yq += cq[m] * bl[(long)m * dv + j];", "(void)0;", 0),
    ("dl_drop_kappa", "o[j] = yq + kappa * bt[j];", "o[j] = yq;", 0),
    ("dl_snapshot_prev", "L[(long)n * dk + i] = Lnew[i];",
     "L[(long)n * dk + i] = Lnew[i] - log_decay(op, ld, sh, dk, i);", 0),
    ("dl_rwkv_read_new_decay", "wq[i] = exp(prev) * q[i];", "wq[i] = exp(Lnew[i]) * q[i];", 0),
    ("dl_no_log_decay_floor", "Lnew[i] = prev + (ell < ORC_MIN_LOG_DECAY ? ORC_MIN_LOG_DECAY : ell);",
     "Lnew[i] = prev + ell;", 0),
    ("dl_merge_one_early", "if (n + 1 == M)\n        fold_one(dk, dv, M, M, Xb, a, bl, L);",
     "if (n + 2 == M)\n        fold_one(dk, dv, M, n + 1, Xb, a, bl, L);", 0),
]


def _mutate(text, old, new, occ):
    pos = -1
    for _ in range(occ + 1):
        pos = text.index(old, pos + 1)
    return text[:pos] + new + text[pos + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new, occ):
    with open(SRC) as f:
        text = f.read()
    mutated = _mutate(text, old, new, occ)
    assert mutated != text
    src = os.path.join(tmp_path, f"{name}.c")
    with open(src, "w") as f:
        f.write(mutated)
    lib = build(src, os.path.join(tmp_path, f"lib{name}.so"))
    bad = Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            with np.errstate(invalid="ignore", over="ignore"):  # a broken oracle may emit NaN
                pin(bad)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passed every pin"
