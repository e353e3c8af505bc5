"""Plant plausible mistakes in a copy of the oracle; the pins must catch each.

Each mutant replaces one exact piece of haste_oracle.c (asserted to occur
exactly once), is compiled with gcc into a temporary directory, and is run
against every pin in oracle_pins.ALL_PINS.  A mutant that passes all pins
would mean the pins cannot tell that mistake from the definition.  CPU only.
"""

import os
import tempfile

import pytest

from oracle import oracle as O

from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(O.__file__), "haste_oracle.c")

FWD = "acc += bf16_to_double(h[b * H + idx[k * F + f]]) * bf16_to_double(W[l * F + f]);"
BWW = "acc += dz_at(dz16, dz64, b * L + l) * bf16_to_double(h[b * H + idx[k * F + f]]);"
BWH = "dh[b * H + idx[k * F + f]] += d * bf16_to_double(W[l * F + f]);"

MUTANTS = {
    "fwd_group_map_mod": ("        const int64_t k = l / G;\n        for (int64_t b = 0; b < B; ++b) {",
                          "        const int64_t k = l % K;\n        for (int64_t b = 0; b < B; ++b) {"),
    "fwd_slot_reversed": (FWD, FWD.replace("W[l * F + f]", "W[l * F + (F - 1 - f)]")),
    "fwd_ignores_index": (FWD, FWD.replace("h[b * H + idx[k * F + f]]", "h[b * H + f]")),
    "fwd_drops_last_slot": ("            for (int64_t f = 0; f < F; ++f)\n                acc += bf16_to_double(h",
                            "            for (int64_t f = 0; f < F - 1; ++f)\n                acc += bf16_to_double(h"),
    "bww_sign": (BWW, BWW.replace("acc +=", "acc -=")),
    "bww_slot0_only": (BWW, BWW.replace("idx[k * F + f]", "idx[k * F]")),
    "bww_drops_last_sample": ("            for (int64_t b = 0; b < B; ++b)\n                acc += dz_at",
                              "            for (int64_t b = 0; b < B - 1; ++b)\n                acc += dz_at"),
    "bww_transposed_dz": (BWW, BWW.replace("b * L + l", "(l % B) * L + (b % L)")),
    "bwh_overwrite": (BWH, BWH.replace("+=", "=")),
    "bwh_group_weight_row": (BWH, BWH.replace("W[l * F + f]", "W[k * F + f]")),
    "bwh_plain_column": (BWH, BWH.replace("dh[b * H + idx[k * F + f]]", "dh[b * H + f]")),
    "bce_label_sign": ("scale * (1.0 / (1.0 + exp(-z)) - yy)", "scale * (1.0 / (1.0 + exp(-z)) + yy)"),
    "bce_no_scale": ("scale * (1.0 / (1.0 + exp(-z)) - yy)", "(1.0 / (1.0 + exp(-z)) - yy)"),
    "bce_sigmoid_sign": ("scale * (1.0 / (1.0 + exp(-z)) - yy)", "scale * (1.0 / (1.0 + exp(z)) - yy)"),
    "loss_drops_softplus": ("+ log1p(exp(-fabs(z))) - yy * z", "- yy * z"),
    "loss_label_term_sign": ("+ log1p(exp(-fabs(z))) - yy * z", "+ log1p(exp(-fabs(z))) + yy * z"),
}


def _pins_fail(lib):
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib)
        except Exception:  # a wrong value, or an error a mutant's output triggers
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} must occur exactly once"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as fh:
            fh.write(src.replace(old, new))
        lib = O.load(O.build(src=path, out=os.path.join(d, f"lib{name}.so")))
        failed = _pins_fail(lib)
    assert failed, f"no pin detects mutant {name}"


def test_pristine_oracle_passes_all_pins():
    assert _pins_fail(O.load()) == []


# The dense head and the joint pass live in oracle.py (numpy): the same
# check, on mutated copies of that module.
PY_SRC = os.path.join(os.path.dirname(O.__file__), "oracle.py")
PY_MUTANTS = {
    "head_dw_from_logits": ('"dW": dZ.T @ hf', '"dW": Z.T @ hf'),
    "head_scale_twice": ("oracle_bce(Z, y_rowptr, y_col, scale, lib=lib)",
                         "oracle_bce(Z, y_rowptr, y_col, scale * scale, lib=lib)"),
    "head_dh_negated": ('"dh": dZ @ Wf', '"dh": -(dZ @ Wf)'),
    "joint_dh_tail_only": ('"dh": t["dh"] + hd["dh"]', '"dh": t["dh"]'),
    "joint_loss_head_only": ('"loss": t["loss"] + hd["loss"]', '"loss": hd["loss"]'),
    "joint_scales_swapped": ("yt_col, scale_tail, G, lib=lib)", "yt_col, scale_head, G, lib=lib)"),
    "rewire_grow_signed": ("grow[k] = np.abs(dense_grad).sum(axis=0)", "grow[k] = dense_grad.sum(axis=0)"),
    "rewire_grow_abs_after_sum": ("grow[k] = np.abs(dense_grad).sum(axis=0)",
                                  "grow[k] = np.abs(dense_grad.sum(axis=0))"),
    "rewire_prune_signed": ("prune = np.abs(wf).reshape(K, G, F).sum(axis=1)", "prune = wf.reshape(K, G, F).sum(axis=1)"),
    "rewire_drop_strongest": ("dropped = set(by_weight[:n_swap])", "dropped = set(by_weight[F - n_swap:])"),
    "rewire_grow_weakest": ("key=lambda j: (-grow[k, j], j))[:n_swap]", "key=lambda j: (grow[k, j], j))[:n_swap]"),
    "rewire_tie_high_id": ("key=lambda j: (-grow[k, j], j))[:n_swap]", "key=lambda j: (-grow[k, j], -j))[:n_swap]"),
    "rewire_no_regrow_of_dropped": ("candidates = [j for j in range(H) if j not in kept]",
                                    "candidates = [j for j in range(H) if j not in cols]"),
    "rewire_weights_stay_in_slot": ("W[k * G:(k + 1) * G, kept[c]]", "W[k * G:(k + 1) * G, f_new]"),
    "e4m3_ties_away": ("    q = np.rint(np.ldexp(a, 3 - E))", "    q = np.floor(np.ldexp(a, 3 - E) + 0.5)"),
    "e4m3_bias": ("    code_n = 8 * (E + 6) + q", "    code_n = 8 * (E + 7) + q"),
    "e4m3_subnormal_step": ("    code_s = np.rint(np.ldexp(a, 9))", "    code_s = np.rint(np.ldexp(a, 8))"),
    "e4m3_decode_mantissa": ("np.where(e == 0, m * 2.0 ** -9, (8.0 + m)", "np.where(e == 0, m * 2.0 ** -9, (7.0 + m)"),
    "w8_scale_inverted": ("scaled = _bf16_f64(W) * np.ldexp(1.0, -np.repeat(wexp, G)",
                          "scaled = _bf16_f64(W) * np.ldexp(1.0, 0 * np.repeat(wexp, G)"),
    "w8_exponent_one_high": ("    return np.clip(e, -120, 120).astype(np.int32)",
                             "    return np.clip(e + 1, -120, 120).astype(np.int32)"),
    "kmeans_argmax_last": ("    a = np.argmax(S, axis=1)", "    a = S.shape[1] - 1 - np.argmax(S[:, ::-1], axis=1)"),
    "kmeans_update_no_norm": ("        Mc[c] = mu / np.linalg.norm(mu)", "        Mc[c] = mu"),
    "kmeans_update_ignores_counts": ("        mu = (v[c] * Mc[c] + Ef[members].sum(axis=0)) / (v[c] + m)",
                                     "        mu = Ef[members].sum(axis=0) / m"),
    "group_seed_highest": ("            seed = free[0]\n            rest = free[1:]",
                           "            seed = free[-1]\n            rest = free[:-1]"),
    "group_farthest": ("key=lambda i: (-sims[i], rest[i])", "key=lambda i: (sims[i], rest[i])"),
    "group_unsorted_members": ("            chosen = sorted([seed] + [rest[i] for i in order])",
                               "            chosen = [seed] + [rest[i] for i in order]"),
    "emb_mean_not_normalized": ("    E[ok] = S[ok] / norm[ok, None]", "    E[ok] = S[ok] / np.asarray(n)[ok, None]"),
    "emb_drops_last_positive": ("        for p in range(rp[b], rp[b + 1]):\n            S[col[p]] += hf[b]",
                                "        for p in range(rp[b], rp[b + 1] - 1):\n            S[col[p]] += hf[b]"),
    "emb_entry_as_sample": ("            S[col[p]] += hf[b]", "            S[col[p]] += hf[p % hf.shape[0]]"),
    "emb_round_up": ("    q = np.rint(np.ldexp(m, 8))", "    q = np.ceil(np.ldexp(m, 8))"),
    "emb_zero_rows_kept": ("    ok = (np.asarray(n) > 0) & (norm > 0)", "    ok = norm >= 0"),
    "slot_order_no_deal": ("            perm[k, 8 * (p % R) + p // R] = f", "            perm[k, p] = f"),
    "slot_order_low_bits": ("        keys = [(int(idx[k, f]) >> 1) & 7 for f in range(F)]",
                            "        keys = [int(idx[k, f]) & 7 for f in range(F)]"),
    "slot_order_ties_reversed": ("key=lambda f: (keys[f], f))", "key=lambda f: (keys[f], -f))"),
    "slot_order_inverse_perm": ("            perm[k, 8 * (p % R) + p // R] = f", "            perm[k, f] = 8 * (p % R) + p // R"),
    "slot_order_weights_stay": ("        W_new = np.take_along_axis(W, np.repeat(perm, G, axis=0), axis=1)",
                                "        W_new = W.copy()"),
    "rewire_grown_keep_old_weight": (
        "            if c in kept:\n                W_new[k * G:(k + 1) * G, f_new] = W[k * G:(k + 1) * G, kept[c]]",
        "            W_new[k * G:(k + 1) * G, f_new] = W[k * G:(k + 1) * G, kept.get(c, f_new)]"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_head_mutant_is_caught(name, monkeypatch):
    import importlib.util

    old, new = PY_MUTANTS[name]
    src = open(PY_SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "oracle_mutant.py")
        with open(path, "w") as fh:
            fh.write(src.replace(old, new))
        spec = importlib.util.spec_from_file_location("oracle_mutant", path)
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        lib = O.load()
        monkeypatch.setattr(O, "oracle_head_step", mod.oracle_head_step)
        monkeypatch.setattr(O, "oracle_joint_step", mod.oracle_joint_step)
        for fn in ("oracle_rewire_scores", "oracle_rewire_select", "oracle_rewire", "e4m3_decode", "e4m3_encode",
                   "w8_group_exponent", "oracle_quantize_w8", "oracle_dequantize_w8", "oracle_kmeans_assign",
                   "oracle_kmeans_update", "oracle_group_greedy", "oracle_label_emb_accumulate",
                   "f64_to_bf16_bits", "oracle_label_emb_finalize", "oracle_label_emb", "oracle_order_slots"):
            monkeypatch.setattr(O, fn, getattr(mod, fn))
        failed = _pins_fail(lib)
    assert failed, f"mutant {name} passes every pin"
