"""Planted mistakes: each plausible error in the oracle must fail one of its pins.

Every case rewrites one passage of a copy of `oracle/vsa2_oracle.py` in a
temporary directory and runs `tests/test_oracle.py` against that copy in a
subprocess (CPU only). The run must fail. A case whose passage no longer
appears in the oracle fails too: the plant has to follow the oracle when it
changes.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle", "vsa2_oracle.py")

# name: (passage, replacement, -k filter of the pins to run, or None for all)
PLANTS = {
    # router, Eq.(5)-(7)
    "router sums instead of averaging the G x G entries":
        ("out[n] = p_hat.reshape(g, nb, g).mean(axis=(0, 2))", "out[n] = p_hat.reshape(g, nb, g).sum(axis=(0, 2))", None),
    "router without the softmax scale":
        ("s = qr[i * g:(i + 1) * g] @ kr.T * _scale(d, scale)", "s = qr[i * g:(i + 1) * g] @ kr.T", None),
    "router with Q and K swapped":
        ("s = qr[i * g:(i + 1) * g] @ kr.T * _scale(d, scale)", "s = kr[i * g:(i + 1) * g] @ qr.T * _scale(d, scale)", None),
    # per-sequence TopK, Eq.(8)-(9)
    "TopK ties to the higher flat index":
        ("order = np.lexsort((np.arange(nb * nb), -flat))", "order = np.lexsort((-np.arange(nb * nb), -flat))", None),
    "TopK budget one short":
        ("    k = min(nb * topk, nb * nb)\n", "    k = min(nb * topk, nb * nb) - 1\n", None),
    # fine branch, Eq.(12), and its gradients
    "fine forward without the softmax scale":
        ("        s = q[qt] @ k[toks].T * sc\n        m = s.max", "        s = q[qt] @ k[toks].T\n        m = s.max", None),
    "fine backward with delta added":
        ("ds = p * (dp - (d_o[qt] * o).sum(axis=1, keepdims=True))",
         "ds = p * (dp + (d_o[qt] * o).sum(axis=1, keepdims=True))", None),
    "fine backward dK without the scale":
        ("dk[toks] += ds.T @ q[qt] * sc", "dk[toks] += ds.T @ q[qt]", None),
    "fine backward dV from dS":
        ("dv[toks] += p.T @ d_o[qt]", "dv[toks] += ds.T @ d_o[qt]", None),
    # coarse branch and gate, Eq.(1)-(4), (13)-(14)
    "gate without the tanh":
        ("g = np.tanh(np.asarray(x, np.float64) @ np.asarray(w_g, np.float64))",
         "g = np.asarray(x, np.float64) @ np.asarray(w_g, np.float64)", None),
    "merge subtracts the fine output":
        ("repeat_cubes(oc_hat, block) + np.asarray(o_f, np.float64)",
         "repeat_cubes(oc_hat, block) - np.asarray(o_f, np.float64)", None),
    "coarse backward with delta added":
        ("ds = p * (dp - (doc_hat * oc_hat).sum(axis=1, keepdims=True))",
         "ds = p * (dp + (doc_hat * oc_hat).sum(axis=1, keepdims=True))", None),
    # padded grids
    "window mean over all members":
        ("return np.where(cnt[:, None] > 0, tot / np.maximum(cnt, 1)[:, None], 0.0)",
         "return np.where(cnt[:, None] > 0, tot / ok.shape[1], 0.0)", "pad"),
    "missing windows kept as keys": ("        s[:, ~ex] = -np.inf\n", "", "pad"),
    "missing windows kept as query rows": ("        p_hat[~ex[i * g:(i + 1) * g]] = 0.0\n", "", "pad"),
    "pad keys in the fine branch":
        ("        yield qt, qt[ok[qt]], toks[ok[toks]]", "        yield qt, qt[ok[qt]], toks", "pad"),
    "pad rows taken as fine queries":
        ("        yield qt, qt[ok[qt]], toks[ok[toks]]", "        yield qt, qt, toks[ok[toks]]", "pad"),
    "coarse gradient spread over the whole block":
        ("np.repeat(t / n[None, :, None], block, axis=1)", "np.repeat(t / float(block), block, axis=1)", "pad"),
    "gate not zero on pad rows": ("        g[~np.asarray(valid, bool)] = 0.0\n", "        pass\n", "pad"),
    "dpre not zero on pad rows": ("        dpre[~np.asarray(valid, bool)] = 0.0\n", "        pass\n", "pad"),
    # 128-token blocks
    "unweighted mean of a block's two cubes":
        ("    tot = (cm * n[:, None]).reshape(-1, 2, cm.shape[1]).sum(axis=1)\n"
         "    return tot / n.reshape(-1, 2).sum(axis=1)[:, None]",
         "    return cm.reshape(-1, 2, cm.shape[1]).mean(axis=1)", "block128"),
    "router G taken from the cube":
        ("    g = block // (pool[0] * pool[1] * pool[2])", "    g = 64 // (pool[0] * pool[1] * pool[2])", "block128"),
    "coarse gradient spread per cube":
        ("    n = ok.reshape(-1, block).sum(axis=1)                               # real tokens per block",
         "    n = np.repeat(ok.reshape(-1, 64).sum(axis=1), block // 64)", "block128"),
    "x not padded to a multiple of 8":
        ("    mult = (4, 4, 4 * _check_block(block))", "    mult = (4, 4, 4)", "block128"),
    "fine key tiles of one cube":
        ("        toks = np.concatenate([_tokens_of(np.nonzero(mask[i])[0], block), text])",
         "        toks = np.concatenate([_tokens_of(np.nonzero(mask[i])[0]), text])", "block128"),
    "fine query tiles of one cube":
        ("        qt = _tokens_of([i], block)", "        qt = _tokens_of([i])", "block128"),
    # MMDiT text tokens
    "video queries skip the text keys":
        ("        toks = np.concatenate([_tokens_of(np.nonzero(mask[i])[0], block), text])",
         "        toks = _tokens_of(np.nonzero(mask[i])[0], block)", "text"),
    "text queries skip the video keys":
        ("        yield text, text, np.concatenate([allv[ok[:Lv]], text])", "        yield text, text, text", "text"),
    "text queries skip the text keys":
        ("        yield text, text, np.concatenate([allv[ok[:Lv]], text])", "        yield text, text, allv[ok[:Lv]]",
         "text"),
    "text pad rows taken as tokens":
        ("    ok[Lv:Lv + n_text] = True\n    return ok, Lv, np.arange(Lv, Lv + n_text)",
         "    ok[Lv:] = True\n    return ok, Lv, np.arange(Lv, L)", "text"),
    "gate applied to text rows":
        ("        o = o_f.copy()\n        o[:Lv] = merge(g[:, h], oc_hat, o_f[:Lv], block)",
         "        o = o_f.copy()\n        o[:Lv] = merge(g[:, h], oc_hat, o_f[:Lv], block)\n"
         "        o[Lv:] += oc_hat.mean(axis=0)", "text"),
    # the routed layer forward (router -> TopK -> fine branch)
    "routed forward with Q and K swapped":
        ("p_r = router_scores(q[h][:Lv], k[h][:Lv], grid, scale=scale, bf16_pooled=bf16_pooled, block=block)",
         "p_r = router_scores(k[h][:Lv], q[h][:Lv], grid, scale=scale, bf16_pooled=bf16_pooled, block=block)",
         "routed"),
    "routed forward without the bf16 router operands":
        ("p_r = router_scores(q[h][:Lv], k[h][:Lv], grid, scale=scale, bf16_pooled=bf16_pooled, block=block)",
         "p_r = router_scores(q[h][:Lv], k[h][:Lv], grid, scale=scale, bf16_pooled=False, block=block)",
         "routed"),
    "routed forward with a TopK per row":
        ("            m = topk_per_sequence(p_r, topk)[0]", "            m = topk_per_row(p_r, topk)[0]", "routed"),
    # the VSA router baseline
    "per-row TopK ties to the higher column":
        ("        order = np.lexsort((np.arange(nb), -scores[i]))", "        order = np.lexsort((-np.arange(nb), -scores[i]))",
         "per_row or coarse_scores"),
    "per-row budget not capped":
        ("    kr = min(topk, nb)\n", "    kr = topk - 1\n", "per_row or coarse_scores"),
    "coarse scores without the softmax":
        ("    return _softmax_rows(qc @ kc.T * _scale(d, scale))", "    return qc @ kc.T * _scale(d, scale)",
         "per_row or coarse_scores"),
    "coarse scores without the scale":
        ("    return _softmax_rows(qc @ kc.T * _scale(d, scale))", "    return _softmax_rows(qc @ kc.T)",
         "per_row or coarse_scores"),
}


@pytest.mark.parametrize("name", list(PLANTS))
def test_planted_mistake_fails_a_pin(name, tmp_path):
    passage, replacement, select = PLANTS[name]
    src = open(ORACLE).read()
    assert passage in src, f"the planted passage is no longer in the oracle: {name}"
    (tmp_path / "oracle").mkdir()
    (tmp_path / "oracle" / "__init__.py").write_text("")
    (tmp_path / "oracle" / "vsa2_oracle.py").write_text(src.replace(passage, replacement, 1))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    for f in ("conftest.py", "test_oracle.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    cmd = [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider", "tests/test_oracle.py"]
    if select:
        cmd += ["-k", select]
    env = dict(os.environ, PYTHONPATH=os.pathsep.join([str(tmp_path), ROOT]))
    r = subprocess.run(cmd, cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    last = (r.stdout.strip().splitlines() or [""])[-1]
    assert r.returncode == 1, f"{name}: the pins did not fail ({last})"
