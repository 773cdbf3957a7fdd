"""pytest plugin for tests/test_oracle_mutants.py: loads a mutated oracle
library (MUTANT_LIB) or patches one planner step of the oracle
(MUTANT_PY) before the pin tests run.  Test infrastructure only."""
import os

import oracle

if os.environ.get("MUTANT_LIB"):
    oracle._LIB_PATH = os.environ["MUTANT_LIB"]

_mp = os.environ.get("MUTANT_PY")
if _mp == "floor_chunk":                       # rank chunk rows floor(dim0 / W) instead of ceil
    oracle._ceil_div = lambda a, b: a // b
elif _mp == "no_round16":                      # all-gather segments not 16-byte aligned
    oracle._round16 = lambda x: x
elif _mp in ("bucket_by_grad", "O_not_cumulative", "last_bucket_first"):
    _orig = oracle.plan

    def _plan(params, W):
        pl = _orig(params, W)
        if _mp == "bucket_by_grad":            # reduce dtype ignored: buckets by gradient dtype
            ps = [p if isinstance(p, oracle.ParamDesc) else oracle.ParamDesc(*p) for p in params]
            stripped = [oracle.ParamDesc(p.dim0, p.inner, p.grad_dtype, 0, p.storage_dtype, p.param_dtype) for p in ps]
            pl2 = _orig(stripped, W)
            pl2.params = ps
            return pl2
        if _mp == "O_not_cumulative":          # column offset = previous member's P, not the prefix sum
            for b in pl.buckets:
                b.O = [0 if k == 0 else b.P[k - 1] for k in range(len(b.P))]
        if _mp == "last_bucket_first":         # buckets out of first-appearance order
            pl.buckets = pl.buckets[::-1]
        return pl

    oracle.plan = _plan
