#!/bin/bash
# CPU sanitizer runs (no GPU is used):
#  1. the oracle built with address, undefined-behaviour and leak sanitizers,
#     driven through every entry point by oracle_harness.c (leaks checked);
#  2. the whole CPU test suite (pytest -m "not gpu") against that oracle
#     build (gcc's runtime preloaded; leak checks off: the interpreter's own
#     allocations live until exit);
#  3. the ABI tests against a build of libspecverify.so whose host code
#     (argument validation, workspace planning, launch sequencing) carries
#     the address and undefined-behaviour sanitizers (clang's runtime
#     preloaded); device code is built as usual.
# Usage: tests/sanitize/run_sanitizers.sh [build-dir]   (from anywhere)
set -euo pipefail
ROOT="$(cd "$(dirname "$0")/../.." && pwd)"
OUT="${1:-$ROOT/tests/sanitize/_build}"
mkdir -p "$OUT"
cd "$ROOT"
SAN="-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer"

echo "== 1. oracle harness (ASan + UBSan + LSan)"
gcc -O1 -g -std=c11 $SAN -Wall -Wextra -o "$OUT/oracle_harness" tests/sanitize/oracle_harness.c \
    oracle/oracle.c -lm -lpthread
ASAN_OPTIONS=detect_leaks=1:abort_on_error=1 "$OUT/oracle_harness"

echo "== 2. CPU test suite against the sanitized oracle (ASan + UBSan)"
gcc -O1 -g -std=c11 -fPIC -shared $SAN -o "$OUT/liboracle_san.so" oracle/oracle.c -lm -lpthread
GCC_RT="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
SPEC_ORACLE_LIB="$OUT/liboracle_san.so" LD_PRELOAD="$GCC_RT" \
    ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
    python -m pytest tests -m "not gpu" -x -q -p no:cacheprovider

echo "== 3. ABI tests against libspecverify.so with sanitized host code (ASan + UBSan)"
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
"$HIPCC" -O1 -g -std=c++17 -fPIC -shared --offload-arch=gfx950 \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer \
    -I include -I exact_draft_verification_amd/csrc -o "$OUT/libspecverify_san.so" \
    exact_draft_verification_amd/csrc/api.hip exact_draft_verification_amd/csrc/chain.hip \
    exact_draft_verification_amd/csrc/tree.hip exact_draft_verification_amd/csrc/outcome.hip \
    exact_draft_verification_amd/csrc/treebuild.hip exact_draft_verification_amd/csrc/treestoch.hip \
    2> >(grep -v packed-fp32-ops >&2)
CLANG_RT="$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
SPEC_VERIFY_LIB="$OUT/libspecverify_san.so" LD_PRELOAD="$CLANG_RT" \
    ASAN_OPTIONS=detect_leaks=0:abort_on_error=1 UBSAN_OPTIONS=print_stacktrace=1:halt_on_error=1 \
    python -m pytest tests/test_abi.py -x -q -p no:cacheprovider
echo "== all sanitizer runs passed"
