"""Tie-free DSA inputs: seeded draws from synth, with rows whose top-k boundary
is closer than the float32 error bound redrawn from their own sub-stream (the
tie judgement is the oracle's)."""
import numpy as np

import oracle
import synth


def make_tie_free(cfg, max_attempts=12):
    inp = synth.make_dsa(cfg)
    for attempt in range(1, max_attempts + 1):
        bad = [(b, t) for b in range(cfg.batch)
               for t in np.nonzero(~oracle.tie_free_rows(inp["qI"], inp["kI"], inp["w"], cfg.topk, batch=b))[0]]
        if not bad:
            return inp
        synth.redraw_dsa_rows(inp, bad, attempt)
    raise RuntimeError("could not make the DSA inputs tie-free")
