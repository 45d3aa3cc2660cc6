#!/bin/bash
# Plant mistakes in a scratch copy of the oracle (CPU only) and check that the
# pins in tests/test_oracle_pins.py catch each one.  Every line of the output
# should show a failing pytest run ("rc=1").
#
# Mutations, in order: gap-extend charged the open cost; gap open charged the
# extend cost only; kill on <= instead of <; range hull one short on the
# right; end-cell tie to the largest i; traceback prefers D over I; transition
# and transversion swapped; matrix clip one cell too low; local mode without
# the D term; gap state prefers "extended" over "opened here"; no revival of a
# diagonal from d-2; the matrix read transposed; N scored as the matrix's A
# entry instead of n_score; the range from d-2 one cell too wide on the left
# (scores, ends and CIGARs stay the same, only the canonical cell count
# grows); the rounds rule covering seeds whose columns leave the sequences.
# Optional arguments: the indexes of the mutations to run (default: all).
set -u
SRC=$(cd "$(dirname "$0")/.." && pwd)
W=${TMPDIR:-/tmp}/fz_oracle_mut
declare -a MUTS=(
 's/I = max2(add(load(b, b->I, i, j - 1), -E)/I = max2(add(load(b, b->I, i, j - 1), -OE)/'
 's/add(load(b, b->S, i - 1, j), -OE));/add(load(b, b->S, i - 1, j), -E));/'
 's/if (S == NEG || (thr != NEG \&\& S < thr))/if (S == NEG || (thr != NEG \&\& S <= thr))/'
 's/int64_t cl = (back == 1) ? pl : pl + 1, ch = ph + 1;/int64_t cl = (back == 1) ? pl : pl + 1, ch = ph;/'
 's/if (S > dbest) { dbest = S; dbest_i = i; }/if (S >= dbest) { dbest = S; dbest_i = i; }/'
 's/else if (Sv != NEG \&\& Sv == load(b, b->I, i, j)) st = ST_I;/else if (Sv != NEG \&\& Sv == load(b, b->D, i, j)) st = ST_D;/'
 's/if (a_purine == b_purine) return sc->transition;/if (a_purine != b_purine) return sc->transition;/'
 's/if (lo < d - s->n) lo = d - s->n;/if (lo < d - s->n - 1) lo = d - s->n - 1;/'
 's/int64_t S = max2(0, max2(H, max2(I, D)));/int64_t S = max2(0, max2(H, I));/'
 's/if (Iv != NEG \&\& Iv == add(load(b, b->S, i, j - 1), -OE)) st = ST_S;/if (Iv != NEG \&\& Iv == add(load(b, b->I, i, j - 1), -E)) {} else st = ST_S;/'
 's/for (int64_t back = 1; back <= 2 \&\& d - back >= 0; back++)/for (int64_t back = 1; back <= 1 \&\& d - back >= 0; back++)/'
 's/? sc->n_score : sc->sub\[a\]\[b\];/? sc->n_score : sc->sub[b][a];/'
 's/return (a == 4 || b == 4) ? sc->n_score : sc->sub\[a\]\[b\];/return sc->sub[a \& 3][b \& 3];/'
 's/int64_t cl = (back == 1) ? pl : pl + 1, ch = ph + 1;/int64_t cl = pl, ch = ph + 1;/'
 'PY:s/covered = inside and any(/covered = any(/'
)
SEL=("$@")
[ ${#SEL[@]} -eq 0 ] && SEL=("${!MUTS[@]}")
for k in "${SEL[@]}"; do
  rm -rf $W && mkdir -p $W && cp -r $SRC/oracle $SRC/tests $SRC/smith_waterman_dp_amd $W/
  rm -f $W/oracle/libfz_oracle.so
  m="${MUTS[$k]}"; f=fz_oracle.c
  # a mutation prefixed PY: applies to the oracle's Python part
  if [ "${m:0:3}" = "PY:" ]; then m="${m:3}"; f=__init__.py; fi
  sed -i "$m" $W/oracle/$f
  if cmp -s $SRC/oracle/$f $W/oracle/$f; then echo "mut $k: NOT APPLIED"; continue; fi
  (cd $W && timeout 600 python -m pytest tests/test_oracle_pins.py -x -q -p no:cacheprovider > $W/log 2>&1)
  rc=$?
  echo "mut $k: pytest rc=$rc $(grep -E 'passed|failed' $W/log | tail -1)"
done
