"""Acceptance rule for commit decisions, from the oracle's fp64 values only.

A masked position's commit decision is *fragile* when the oracle's own values
put it within FRAGILE = 1e-4 of a tie; such positions are excluded from the
exact GPU-vs-oracle comparison and counted.  Three tests, counted apart:

  margin  conf_i - p2_i < 1e-4: the greedy token's probability is within 1e-4
          of the runner-up's.  Both sides take the argmax on the raw fp32
          logits, so the token itself is still compared exactly; these are
          counted only.
  rank    0 < k < |M| and conf_(k) - conf_(k+1) < 1e-4 (ranked by confidence
          desc, index asc): every position within 1e-4 of either boundary
          value may fall on either side of the top-k cut.
  tau     |conf_i - tau| < 1e-4: the threshold test may go either way.

Excluded = rank | tau.  Nothing here reads a GPU result.
"""

import numpy as np

import oracle
import synth

FRAGILE = 1e-4


def runner_up(logits_row):
    """p2 of one row: the probability of the best token other than the greedy one."""
    return oracle.confidence_row(logits_row)[3]


def fragile(conf64, p2, masked, k, tau):
    """dict(margin=set, rank=set, tau=set) of fragile masked positions of one request."""
    M = [i for i in range(len(masked)) if masked[i]]
    out = dict(margin=set(), rank=set(), tau=set())
    for i in M:
        if conf64[i] - p2[i] < FRAGILE:
            out["margin"].add(i)
        if abs(conf64[i] - tau) < FRAGILE:
            out["tau"].add(i)
    if 0 < k < len(M):
        order = sorted(M, key=lambda i: (-conf64[i], i))
        kth, nxt = conf64[order[k - 1]], conf64[order[k]]
        if kth - nxt < FRAGILE:
            out["rank"] = {i for i in M if abs(conf64[i] - kth) < FRAGILE or abs(conf64[i] - nxt) < FRAGILE}
    return out


def step_fragility(logits, masked, S, tau, ref):
    """Fragile sets of every request of one confidence + commit step, given the
    oracle's result ``ref`` on (logits, masked)."""
    n_req, D, _ = logits.shape
    res = []
    for r in range(n_req):
        m = masked[r].astype(bool)
        k = oracle.commit_k(D, S, int(m.sum()))
        p2 = np.full(D, np.nan)
        for i in np.flatnonzero(m):
            p2[i] = runner_up(logits[r, i])
        res.append(fragile(ref["conf"][r], p2, m, k, tau))
    return res


def block_loop_logits(p, cfg_seed):
    """Per-step logits of a block's denoising loop: the step's own logits first,
    then fresh draws from Generator(PCG64(4242 + config number))."""
    rng = np.random.Generator(np.random.PCG64(4242 + cfg_seed))

    def nxt(first):
        return first if first is not None else synth.fresh_logits(p, rng)
    return nxt


def counts(sets_per_req):
    c = dict(margin=0, rank=0, tau=0, excluded=0)
    for f in sets_per_req:
        for key in ("margin", "rank", "tau"):
            c[key] += len(f[key])
        c["excluded"] += len(f["rank"] | f["tau"])
    return c


def oracle_block_loop(step, cfg_id):
    """The oracle's whole block loop (DiffusionVL notes, cached block decoding):
    steps until nothing is masked, fresh seeded logits per step.  Returns the
    per-step list of (logits, masked_before, tokens_before, ref, fragile sets)."""
    p = step["params"]
    masked, tokens = step["masked"].copy(), step["tokens"].copy()
    nxt = block_loop_logits(p, cfg_id)
    logits = nxt(step["logits"])
    hist = []
    while masked.sum() > 0:
        ref = oracle.confidence_commit(logits, masked, tokens, p["S"], p["tau"])
        hist.append((logits, masked, tokens, ref, step_fragility(logits, masked, p["S"], p["tau"], ref)))
        masked, tokens = ref["masked"], ref["tokens"]
        logits = nxt(None)
        assert len(hist) <= p["S"] + 1
    return hist


def summarize(cfg_id):
    """Fragile counts of a config's first step and of its whole block loop."""
    step = synth.config_step(cfg_id)
    p = step["params"]
    hist = oracle_block_loop(step, cfg_id)
    first = counts(hist[0][4])
    first["decisions"] = int(step["masked"].sum())
    loop = dict(margin=0, rank=0, tau=0, excluded=0, decisions=0)
    for logits, mb, tb, ref, fr in hist:
        c = counts(fr)
        for key in ("margin", "rank", "tau", "excluded"):
            loop[key] += c[key]
        loop["decisions"] += int(mb.sum())
    loop["steps"] = len(hist)
    return dict(config=cfg_id, S=p["S"], tau=p["tau"], first_step=first, block_loop=loop)
