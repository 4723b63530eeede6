"""Mutation check of the oracle's pins (CPU only; not collected by pytest).

Each mutant plants one plausible mistake (a dropped term, a wrong sign, index or
operand) in a temporary copy of the oracle and runs the CPU pin suite against it;
every mutant must make a pin fail.  A line that recurs (the softmax scale, the
S-before-F check of both stack drivers) is changed everywhere it occurs.  The repository's own oracle is never modified.

    python tests/mutate_oracle.py [mutant ...]      (all mutants when none is named)
"""
import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join("oracle", "indexcache_oracle.py")

MUTANTS = {
    # O1 score
    "drop_relu": ("return w_t @ np.maximum(y, 0.0)", "return w_t @ y"),
    "relu_neg": ("np.maximum(y, 0.0)", "np.maximum(-y, 0.0)"),
    "head_weight_T": ("return w_t @ np.maximum(y, 0.0)", "return np.maximum(y, 0.0).sum(0) * w_t.mean()"),
    "causal_excl": ("keys = k_I[: p + 1]", "keys = k_I[: p]"),
    "causal_plus": ("keys = k_I[: p + 1]", "keys = k_I[: p + 2]"),
    # O2 / O3 select and emit
    "tie_high": ('order = np.argsort(-scores, kind="stable")',
                 'order = (len(scores)-1-np.argsort(-scores[::-1], kind="stable"))'),
    "asc_select": ('order = np.argsort(-scores, kind="stable")', 'order = np.argsort(scores, kind="stable")'),
    "no_sort_out": ("chosen = np.sort(order[: min(k, n)])", "chosen = order[: min(k, n)]"),
    "pad_zero": ("out = np.full(k, -1, dtype=np.int32)", "out = np.full(k, 0, dtype=np.int32)"),
    "fp64_decision": ("return np.asarray(row, dtype=np.float64).astype(np.float32)",
                      "return np.asarray(row, dtype=np.float64)"),
    # O4 attention
    "kv_swap": ("K = kv[sel, 0, :]", "K = kv[sel, 1, :]"),
    "no_max_sub": ("logits = logits - logits.max(axis=1, keepdims=True)\n    p = np.exp(logits)",
                   "logits = logits - logits.max()\n    p = np.exp(logits)"),
    "scale_d": ("scale = 1.0 / math.sqrt(d) if scale is None else scale", "scale = 1.0 / d if scale is None else scale"),
    "no_norm": ("p = p / p.sum(axis=1, keepdims=True)", "p = p / p.sum()"),
    # O5 / O6 stack and decode
    "s_recompute": ("        elif cache is None:", "        elif False:"),
    "decode_pos": ("p = int(seq_len[b]) - 1", "p = int(seq_len[b])"),
    # fp8 codec
    "e4m3_bias": ("np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    "e4m3_sub": ("m / 8.0 * 2.0 ** -6", "m / 8.0 * 2.0 ** -7"),
    # overlap diagnostic
    "jaccard_union": ("out[r] = len(sa & sb) / (len(sa | sb) + 1e-8)", "out[r] = len(sa & sb) / (len(sa) + 1e-8)"),
    # distillation loss
    "kl_reverse": ("return float(np.sum(p[nz] * (np.log(p[nz]) - log_r[nz])))",
                   "return float(np.sum(np.exp(log_r[nz]) * (log_r[nz] - np.log(p[nz]))))"),
    "target_head_norm": ("a = a / a.sum(axis=1, keepdims=True)", "a = a / a.sum()"),
    "target_first_layer": ("total += a.sum(axis=0)", "total += a.sum(axis=0) if count == 0 else 0.0"),
    # dynamic refresh
    "refresh_inclusive": ("if hit < tau * own:", "if hit <= tau * own:"),
    "recall_inverted": ("recall[l] = hit / own", "recall[l] = own / max(hit, 1)"),
    "probe_from_zero": ("return np.arange((Lq - 1) % stride, Lq, stride)", "return np.arange(0, Lq, stride)"),
    "probe_no_pos0": ('lay["k_I"], pos0 + int(t))', 'lay["k_I"], int(t))'),
    "refresh_keeps_cache": ('                cache = indexer_topk(lay["q_I"], lay["w"], lay["k_I"], k, pos0)\n                refreshed[l] = True', '                refreshed[l] = True'),
    # codecs
    "bf16_shift": ("u32 = bits.astype(np.uint32) << np.uint32(16)", "u32 = bits.astype(np.uint32) << np.uint32(15)"),
    "e4m3_all_nan_top": ("return np.where((e == 15) & (m == 7), np.nan, val)", "return np.where(e == 15, np.nan, val)"),
    "e4m3_no_sign": ("val = np.where(s == 1, -mag, mag)", "val = mag"),
    # attention and distillation details
    "skip_key_zero": ("sel = idx_t[idx_t >= 0]", "sel = idx_t[idx_t > 0]"),
    "kl_unnormalised_r": ("log_r = log_r - math.log(np.exp(log_r).sum())", "log_r = log_r"),
    "target_layer_mean": ("count += a.shape[0]", "count += 1"),
    # query positions
    "stack_no_pos0": ('indexer_topk(lay["q_I"], lay["w"], lay["k_I"], k, pos0)', 'indexer_topk(lay["q_I"], lay["w"], lay["k_I"], k)'),
    "row_pos_fixed": ("indexer_scores_row(q_I[t], w[t], k_I, pos0 + t)", "indexer_scores_row(q_I[t], w[t], k_I, pos0)"),
    # decode
    "decode_first_cache": ('one = {"q": lay["q"][b][None], "kv": lay["kv"][b]}',
                           'one = {"q": lay["q"][b][None], "kv": lay["kv"][0]}'),
}


def main(names=None) -> int:
    src = open(os.path.join(ROOT, ORACLE)).read()
    missed = []
    for name, (old, new) in MUTANTS.items():
        if names and name not in names:
            continue
        if src.count(old) < 1:
            print(f"{name:20s} PATTERN NOT IN THE ORACLE")
            missed.append(name)
            continue
        tmp = tempfile.mkdtemp()
        try:
            repo = os.path.join(tmp, "r")
            shutil.copytree(ROOT, repo, ignore=shutil.ignore_patterns(".git", "_work", "gpurun_out", "_build",
                                                                      "__pycache__", "*.so"))
            with open(os.path.join(repo, ORACLE), "w") as f:
                f.write(src.replace(old, new))
            r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_oracle_pins.py", "-q", "-x", "-p",
                                "no:cacheprovider"], cwd=repo, capture_output=True, text=True)
        finally:
            shutil.rmtree(tmp)
        caught = r.returncode != 0
        if not caught:
            missed.append(name)
        print(f"{name:20s} {'caught' if caught else 'MISSED'}", flush=True)
    print("all mutants caught" if not missed else f"missed: {', '.join(missed)}")
    return 1 if missed else 0


if __name__ == "__main__":
    sys.exit(main(set(sys.argv[1:])))
