"""Mutation check of the oracle's pins (CPU only; not collected by pytest).

Each entry below is a plausible mistake in the oracle -- a dropped term, a
wrong comparison, an off-by-one mask, a reversed tie-break.  The script plants
one at a time in a scratch copy of the oracle and runs tests/test_oracle.py
against it; every mutation must make at least one pin fail.

    python tests/mutation_check.py            # all mutations (~2 minutes)
    python tests/mutation_check.py NAME ...   # selected ones
Exit status 1 if any mutation survives.
"""
import os, shutil, subprocess, sys, tempfile
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
MUTS = {
    "pooled_no_sqrt": ("L = block_means(k, blk) @ qm / math.sqrt(d)", "L = block_means(k, blk) @ qm"),
    "pooled_sum": ("qm = q_last.astype(np.float64).mean(axis=0)", "qm = q_last.astype(np.float64).sum(axis=0)"),
    "pe_cut_strict": ('kstar = int(np.searchsorted(csum, target, side="left")) + 1\n        kstar = min(kstar, vals.size)',
                      'kstar = int(np.searchsorted(csum, target, side="right")) + 1\n        kstar = min(kstar, vals.size)'),
    "coverage_strict": ('kstar = min(int(np.searchsorted(csum, target, side="left")) + 1, vals.size)',
                        'kstar = min(int(np.searchsorted(csum, target, side="right")) + 1, vals.size)'),
    "route_jsd_strict": ("return bool(float(j) >= float(np.float32(tau)))", "return bool(float(j) > float(np.float32(tau)))"),
    "route_strict": ("return bool(np.float32(c) >= np.float32(tau))", "return bool(np.float32(c) > np.float32(tau))"),
    "vs_ge": ("sel = p > thr\n    sel[0] = True\n    sel[nb - 1] = True\n    return _top_up(sel, p, min_blocks)\n\n\ndef median_floor_f32",
              "sel = p >= thr\n    sel[0] = True\n    sel[nb - 1] = True\n    return _top_up(sel, p, min_blocks)\n\n\ndef median_floor_f32"),
    "mu_nb_minus_1": ("return np.float32(t / np.float32(nb - 2))", "return np.float32(t / np.float32(nb - 1))"),
    "pe_no_sqrt": ("L = (qm @ km.T) / math.sqrt(d)", "L = (qm @ km.T)"),
    "slash_sign": ("a_s[:q + 1] += A[r, q::-1]", "a_s[:q + 1] += A[r, :q + 1]"),
    "cstruct_no_local": ("cols[max(n - w_local, 0):] = True", "pass"),
    "pe_tie_upper": ("order = np.lexsort((flat, -vals))", "order = np.lexsort((-flat, -vals))"),
    "attn_no_scale": ("s = (q[rows].astype(np.float64) @ k[cols].astype(np.float64).T) / math.sqrt(d)",
                      "s = (q[rows].astype(np.float64) @ k[cols].astype(np.float64).T)"),
    "median_even_upper": ("return np.float32(np.float32(r[m // 2 - 1] + r[m // 2]) * np.float32(0.5))", "return np.float32(r[m // 2 - 1])"),
    "proxy_mask_offby1": ("s[np.arange(n)[None, :] > pos[:, None]] = -np.inf", "s[np.arange(n)[None, :] >= pos[:, None]] = -np.inf"),
    "attn_mask_offby1": ("s[cols[None, :] > rows[:, None]] = -np.inf", "s[cols[None, :] >= rows[:, None]] = -np.inf"),
    "dense_mask_diag": ("s[np.triu(np.ones((n, n), bool), 1)] = -np.inf\n    s -= s.max(axis=1, keepdims=True)\n    e = np.exp(s)\n    return (e @ v",
                        "s[np.triu(np.ones((n, n), bool), 0)] = -np.inf\n    s -= s.max(axis=1, keepdims=True)\n    e = np.exp(s)\n    return (e @ v"),
    "jsd_log2": ("return float(np.sum(x[nz] * np.log(x[nz] / m[nz])))", "return float(np.sum(x[nz] * np.log2(x[nz] / m[nz])))"),
    "topup_tie_upper": ("order = sorted(rest, key=lambda i: (-float(p[i]), int(i)))", "order = sorted(rest, key=lambda i: (-float(p[i]), -int(i)))"),
    "slash_block_plus1": ("s |= set(int(qb - x) for x in ss[ss <= qb])", "s |= set(int(qb - x - 1) for x in ss[ss < qb])"),
    "pe_no_diag_anchor": ("mask[np.arange(nb), np.arange(nb)] = True", "pass"),
    "median_odd_idx": ("return np.float32(r[(m - 1) // 2])", "return np.float32(r[(m + 1) // 2])"),
    "cov_tie_upper": ("order = np.lexsort((idx, -vals))", "order = np.lexsort((-idx, -vals))"),
    "mu_no_clamp": ("t = np.float32(max(t, np.float32(0.0)))", "pass"),
    "pooled_no_max_all": ("e = np.exp(L - L.max())\n    return e / e.sum()", "e = np.exp(L)\n    return e / e.sum()"),
    "vertical_div": ("a_v = A.sum(axis=0) / b", "a_v = A.sum(axis=0) / n"),
}
sel = sys.argv[1:] or list(MUTS)
survivors = []
for name in sel:
    old, new = MUTS[name]
    d = tempfile.mkdtemp(prefix="mut_")
    for sub in ("oracle", "tests", "workloads"):
        shutil.copytree(os.path.join(ROOT, sub), os.path.join(d, sub), ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copy(os.path.join(ROOT, "pytest.ini"), d)
    p = os.path.join(d, "oracle", "crisp_oracle.py")
    s = open(p).read()
    assert s.count(old) == 1, (name, s.count(old))
    open(p, "w").write(s.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle.py"],
                       cwd=d, capture_output=True, text=True)
    last = [l for l in r.stdout.splitlines() if l.strip()][-1]
    failed = [l for l in r.stdout.splitlines() if l.startswith("FAILED")]
    print(f"{name:22s} {'CAUGHT' if r.returncode else 'SURVIVED'}  {failed[0] if failed else last}", flush=True)
    if not r.returncode:
        survivors.append(name)
    shutil.rmtree(d)
print(f"{len(sel) - len(survivors)} of {len(sel)} mutations caught" + (f"; survived: {survivors}" if survivors else ""))
sys.exit(1 if survivors else 0)
