"""Plant plausible mistakes in copies of the oracle; some pin must catch each.

CPU only.  Each case copies oracle/ into a temporary package, applies one
text substitution (a dropped term, a wrong sign, a wrong index or map, an
off-by-one mask), imports the copy under a fresh name and runs every pin in
tests/oracle_pins.py against it.  The case passes when at least one pin fails.
"""

import importlib.util
import os
import shutil
import sys

import pytest

import oracle_pins

ORACLE_DIR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")

MUTATIONS = [
    ("ring.py", "o * w_old[:, None] + o_b", "o + o_b", "drop rescale of o"),
    ("ring.py", "l * w_old + l_b * w_blk", "l + l_b * w_blk", "drop rescale of l"),
    ("ring.py", "np.exp(m - ref)", "np.exp(ref - m)", "wrong sign of rescale"),
    ("ring.py", "np.exp(m_b - ref)", "np.exp(ref - m_b)", "wrong sign of the block's weight"),
    ("ring.py", "e = np.exp(s - np.where(has, m_b, 0.0)[:, None])", "e = np.exp(s)",
     "block sums not taken against the block max"),
    ("ring.py", "m_new = np.maximum(m, m_b)", "m_new = m_b", "forget running max"),
    ("ring.py", "[(p - s) % N for s", "[(p + s) % N for s", "rotation direction"),
    ("ring.py", "lse = np.where(pos, m + np.log(safe_l)", "lse = np.where(pos, m - np.log(safe_l)", "lse sign"),
    ("ring.py", "vis = (kp[None, :] <= qp[:, None])", "vis = (kp[None, :] < qp[:, None])", "ring mask excludes diagonal"),
    ("ring.py", "g = h // G", "g = h % Hkv", "ring GQA head map"),
    ("ring.py", "out = np.where(pos[:, None], o / safe_l[:, None], 0.0)",
     "out = np.where(pos[:, None], o, 0.0)", "finalize skips division"),
    ("attention.py", "vis = kp[keys][None, :] <= qp[r0:r1, None]", "vis = kp[keys][None, :] < qp[r0:r1, None]",
     "full mask excludes diagonal"),
    ("attention.py", 'np.searchsorted(kp, last, side="right")', 'np.searchsorted(kp, last, side="left")',
     "causal key prefix drops the last visible key"),
    ("attention.py", "keys = np.flatnonzero(kp <= last)", "keys = np.flatnonzero(kp < last)",
     "causal key selection (unsorted keys) drops the last visible key"),
    ("attention.py", "scale = 1.0 / np.sqrt(D)\n    qp", "scale = 1.0 / D\n    qp", "wrong default scale"),
    ("attention.py", "g = h // G\n            for r0", "g = h % Hkv\n            for r0", "full GQA head map"),
    ("attention.py", "s = (q_rows @ k.T) * scale", "s = (q_rows @ k.T)", "scale dropped"),
    ("attention.py", "lse = np.where(seen, m_safe + np.log", "lse = np.where(seen, np.log", "lse drops max"),
    ("attention.py", "(e @ v) / np.where", "(e @ v) * np.where", "normaliser inverted"),
    ("layouts.py", "return p + a * N", "return p * N + a", "striped map"),
    ("layouts.py", "(2 * N - 1 - p) * c + (a - c)", "(N + p) * c + (a - c)", "zigzag second chunk"),
    ("layouts.py", "int((keys[None, :] <= qp[:, None]).sum())", "int((keys[None, :] < qp[:, None]).sum())",
     "pair count off by one"),
    ("merge.py", "l = la * wa + lb * wb", "l = la * wa + lb", "merge drops rescale of l_b"),
    ("merge.py", "o = oa * wa[..., None] + ob * wb[..., None]", "o = oa * wa[..., None] + ob * wa[..., None]",
     "merge weights o_b by side a"),
    ("merge.py", "m = np.maximum(ma, mb)", "m = ma", "merge keeps side a's max"),
    ("merge.py", "lse = np.where(seen, m + np.log", "lse = np.where(seen, np.log", "merged lse drops max"),
    ("merge.py", "wb = np.where(seen, _side_weight(lse_b, ref), 0.0)",
     "wb = np.where(seen, _side_weight(lse_b, m), 0.0)", "merged out weight not normalised"),
    ("merge.py", "return np.where(finite, np.exp(np.where(finite, x, 0.0) - np.where(finite, ref, 0.0)), 0.0)",
     "return np.where(finite, np.exp(np.where(finite, x, 0.0) - np.where(finite, ref, 0.0)), 1.0)",
     "empty side weighted 1"),
    ("vocab_ce.py", "log_z = [m + np.log(s)", "log_z = [np.log(s)", "vocab log-normaliser drops max"),
    ("vocab_ce.py", "own = (t >= start) & (t < start + V_loc)\n    pred",
     "own = (t >= start) & (t <= start + V_loc)\n    pred", "vocab shard owns next shard's first id"),
    ("vocab_ce.py", "s = np.exp(z - np.where(m == -np.inf, 0.0, m)[:, None])", "s = np.exp(z)",
     "vocab sum not shifted by max"),
    ("vocab_ce.py", "lse = np.logaddexp(lse, lz)", "lse = np.maximum(lse, lz)",
     "shards merged by max instead of log-sum-exp"),
    ("vocab_ce.py", "loss = lse - pred", "loss = lse + pred", "vocab loss target sign"),
    ("vocab_ce.py", "g[np.arange(N)[own], tg[own]] -= 1.0", "g[np.arange(N)[own], tg[own]] += 1.0",
     "gradient one-hot sign"),
    ("vocab_ce.py", "    return g * scale", "    return g", "gradient scale dropped"),
    ("vocab_ce.py", "return logsumexp(z, axis=1) - zt", "return logsumexp(z, axis=1) + zt",
     "per-row loss target sign"),
    ("vocab_ce.py", "    m = z.max(axis=1)\n    s = np.exp", "    m = z.mean(axis=1)\n    s = np.exp",
     "shard max replaced by mean"),
]


def _load_mutant(tmp_path, idx, fname, old, new):
    name = f"oracle_mutant_{idx}"
    dst = tmp_path / name
    shutil.copytree(ORACLE_DIR, dst, ignore=shutil.ignore_patterns("__pycache__"))
    path = dst / fname
    src = path.read_text()
    assert old in src, f"mutation target not found in {fname}: {old!r}"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(name, dst / "__init__.py",
                                                  submodule_search_locations=[str(dst)])
    mod = importlib.util.module_from_spec(spec)
    sys.modules[name] = mod
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("idx,mut", list(enumerate(MUTATIONS)), ids=[m[3] for m in MUTATIONS])
def test_mutation_is_caught(tmp_path, idx, mut):
    fname, old, new, _ = mut
    mod = _load_mutant(tmp_path, idx, fname, old, new)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # AssertionError, or the mutant crashing
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin caught the planted mistake: {mut[3]}"
