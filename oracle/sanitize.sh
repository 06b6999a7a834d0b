#!/usr/bin/env bash
# Build the CPU oracle with AddressSanitizer and UndefinedBehaviorSanitizer
# (host code only) and run the oracle's own tests against that build.
# Usage, from the repository root:  bash oracle/sanitize.sh
set -euo pipefail
cd "$(dirname "$0")/.."
out=oracle/libmoe_oracle_asan.so
gcc -O1 -g -fno-omit-frame-pointer -fsanitize=address,undefined -fno-sanitize-recover=undefined \
    -fopenmp -fPIC -shared -o "$out" oracle/moe_oracle.c -lm
preload="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
LD_PRELOAD="$preload" ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1 \
    MOE_ORACLE_LIB="$PWD/$out" python -m pytest tests/test_oracle_schedule.py tests/test_oracle_float.py \
    tests/test_oracle_mx.py tests/test_oracle_ring.py tests/test_oracle_shared.py -q -p no:cacheprovider "$@"
