"""Mutation check of the oracle's pins (CPU only; not collected by pytest).

Each entry below is one plausible slip in oracle/gqla_ref.py: an off-by-one
causal bound, a dropped term, a wrong group, page or slot index, a wrong
rounding rule, a merge without its maximum, a metric over the wrong operand.
For each slip (and each place its text occurs) the repository is copied to a
temporary directory, the slip is written into the copy's oracle, and the
not-gpu test suite runs there; a slip counts as caught when some test fails.
The repository itself is never modified.

    python tests/oracle_mutation_check.py

Two entries are expected to survive because they do not change any result:
a split range whose end lies past the context (the visible bound clips it),
and a sparse index equal to the context length passing the range filter (the
causal bound excludes it).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join("oracle", "gqla_ref.py")

# (name, text in the oracle, slipped text)
SLIPS = [
    ("causal bound one short", "return L - s_q + i + 1", "return L - s_q + i"),
    ("no causal bound", "return L - s_q + i + 1", "return L"),
    ("lse without the maximum", "return (e @ values) / z, m + math.log(z)", "return (e @ values) / z, math.log(z)"),
    ("softmax not normalised", "return (e @ values) / z, m + math.log(z)", "return (e @ values), m + math.log(z)"),
    ("rope term dropped", "s = (K[:n] @ q_nope[b, i, h] + KR[:n] @ q_rope[b, i, h]) * d.scale",
     "s = (K[:n] @ q_nope[b, i, h]) * d.scale"),
    ("scale dropped", "s = (K[:n] @ q_nope[b, i, h] + KR[:n] @ q_rope[b, i, h]) * d.scale",
     "s = (K[:n] @ q_nope[b, i, h] + KR[:n] @ q_rope[b, i, h])"),
    ("keys of group 0", "K = C @ w_uk[G]", "K = C @ w_uk[0]"),
    ("values from W_UK", "V = C @ w_uv[G]", "V = C @ w_uk[G]"),
    ("page from the slot", "page = int(block_table_row[t // d.bs])", "page = int(block_table_row[t % d.bs])"),
    ("slot off by one", "rows[t] = pages[page, t % d.bs]", "rows[t] = pages[page, (t + 1) % d.bs]"),
    ("up-projection of group 0", "out[bi, i, h] = o_lat @ w_uv[G]", "out[bi, i, h] = o_lat @ w_uv[0]"),
    ("head-to-group map", "            G = h // d.heads_per_group\n            for i in range(d.s_q):\n                n = visible",
     "            G = h % d.g\n            for i in range(d.s_q):\n                n = visible"),
    ("expansion not rounded", "k_view[...] = bf16_round(C @ w_uk[G])", "k_view[...] = C @ w_uk[G]"),
    ("V block over the K block", "return G * d.bs * (d.d_nope + d.d_v) + d.bs * d.d_nope + slot * d.d_v + j",
     "return G * d.bs * (d.d_nope + d.d_v) + slot * d.d_v + j"),
    ("rope offset one group early", "return d.g * d.bs * (d.d_nope + d.d_v) + slot * d.d_R + j",
     "return (d.g - 1) * d.bs * (d.d_nope + d.d_v) + slot * d.d_R + j"),
    ("rope view one group early", "    base = d.g * d.bs * (d.d_nope + d.d_v)\n    return page",
     "    base = (d.g - 1) * d.bs * (d.d_nope + d.d_v)\n    return page"),
    ("bf16 with 8 stored bits", "ulp = np.ldexp(1.0, e - 7)", "ulp = np.ldexp(1.0, e - 8)"),
    ("bf16 ties away from zero", "q = np.round(xf / ulp) * ulp", "q = np.floor(xf / ulp + 0.5) * ulp"),
    ("bf16 truncated", "q = np.round(xf / ulp) * ulp", "q = np.trunc(xf / ulp) * ulp"),
    ("sparse index L accepted (no effect)", "if 0 <= int(t) < L]", "if 0 <= int(t) <= L]"),
    ("sparse duplicates dropped", "sel = [int(t) for t in indices[b][G] if 0 <= int(t) < L]",
     "sel = sorted(set(int(t) for t in indices[b][G] if 0 <= int(t) < L))"),
    ("sparse without the causal bound", "vis = np.array([t < visible_tokens(L, i, d.s_q) for t in sel], dtype=bool)",
     "vis = np.array([t < L for t in sel], dtype=bool)"),
    ("split end past L (no effect)", "return [(lo, min(lo + split_tokens, L)) for lo in range(0, L, split_tokens)]",
     "return [(lo, lo + split_tokens) for lo in range(0, L, split_tokens)]"),
    ("merge weights without the maximum", "w = [0.0 if v == -np.inf else math.exp(v - m) for v in ls]",
     "w = [0.0 if v == -np.inf else math.exp(v) for v in ls]"),
    ("merge lse without the maximum", "lse[(b,) + idx] = m + math.log(z)", "lse[(b,) + idx] = math.log(z)"),
    ("merge as a plain mean", "                    acc += ws * part_out[(s,) + idx]",
     "                    acc += part_out[(s,) + idx]\n                    z = hi - lo"),
    ("latent partials without the visible bound", "n_hi = min(hi, visible_tokens(L, i, d.s_q))", "n_hi = hi"),
    ("metric over the output maximum", "max_ref = float(np.max(np.abs(ref))) if ref.size else 0.0",
     "max_ref = float(np.max(np.abs(got))) if ref.size else 0.0"),
    ("metric with a squared norm", "l2_err = float(np.linalg.norm(err.ravel()))", "l2_err = float(np.linalg.norm(err.ravel())) ** 2"),
]

SKIP_DIRS = {".git", "gpurun_out", "_work", "_build", "__pycache__", ".pytest_cache", "profiles"}


def run_copy(src_text: str, dst: str) -> bool:
    """Write src_text as the copy's oracle, run the not-gpu suite there; True if a test fails."""
    with open(os.path.join(dst, ORACLE), "w") as f:
        f.write(src_text)
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider", "tests"],
                       cwd=dst, capture_output=True, text=True)
    return r.returncode != 0


def main() -> int:
    original = open(os.path.join(ROOT, ORACLE)).read()
    survived = []
    total = 0
    with tempfile.TemporaryDirectory() as tmp:
        dst = os.path.join(tmp, "repo")
        shutil.copytree(ROOT, dst, ignore=lambda d, names: [n for n in names if n in SKIP_DIRS])
        if run_copy(original, dst):
            print("the unmutated suite fails in the copy; nothing to check")
            return 2
        for name, old, new in SLIPS:
            count = original.count(old)
            if count == 0:
                print(f"no such text: {name}")
                survived.append(name)
                continue
            start = 0
            for k in range(count):
                pos = original.index(old, start)
                start = pos + 1
                total += 1
                label = name if count == 1 else f"{name} (place {k + 1} of {count})"
                caught = run_copy(original[:pos] + new + original[pos + len(old):], dst)
                print(("caught   " if caught else "survived ") + label, flush=True)
                if not caught:
                    survived.append(label)
    print(f"{total - len(survived)} of {total} slips caught; survived: {survived}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
