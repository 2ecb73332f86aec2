#!/bin/bash
# Run the CPU test suite (no GPU) with the oracle built under AddressSanitizer
# and UndefinedBehaviorSanitizer.  The sanitizer runtime must be loaded before
# the interpreter, hence the preload; leak checking is off because the
# interpreter itself never frees some of its allocations.
set -euo pipefail
cd "$(dirname "$0")/.."
export DSPARK_ORACLE_SANITIZE=1
python -c "import oracle; oracle.build(force=True)"
LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
    python -m pytest tests -q -m "not gpu" -p no:cacheprovider "$@"
