#!/bin/bash
# The CPU test suite with the host code under AddressSanitizer and UBSan: the
# oracle (oracle/tqref.c) and the library's host C++ (argument validation,
# plans, codebook solver) are rebuilt with -fsanitize=address,undefined and
# loaded in place of the ordinary builds (TQ_SANITIZE=1). CPU only: kernels
# are not instrumented and no test here launches one.
set -euo pipefail
cd "$(dirname "$0")/.."
python -m kv_cache_vector_03_amd.build --sanitize
export TQ_SANITIZE=1
export ASAN_OPTIONS=detect_leaks=0:abort_on_error=1
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
export LD_PRELOAD="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
exec python -m pytest tests -m "not gpu" -x -q -p no:cacheprovider "$@"
