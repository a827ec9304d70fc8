#!/bin/bash
# CPU-side sanitizer runs (no GPU needed):
#  1. the fp64 oracle built with gcc's AddressSanitizer and
#     UndefinedBehaviorSanitizer (any report aborts), under the whole CPU
#     test suite;
#  2. the C ABI's host-side argument validation built with clang's
#     AddressSanitizer and UndefinedBehaviorSanitizer on the host code only
#     (device code unchanged), under tests/test_abi.py.
# Usage, from anywhere: bash tests/sanitize.sh
set -euo pipefail
cd "$(dirname "$0")/.."
mkdir -p _build
python -c 'import oracle; oracle.build(sanitize=True)'
SPEC_ORACLE_SANITIZE=1 ASAN_OPTIONS=detect_leaks=0 \
    LD_PRELOAD="$(gcc -print-file-name=libasan.so) $(gcc -print-file-name=libubsan.so)" \
    python -m pytest tests -q -m "not gpu" -p no:cacheprovider
hipcc --offload-arch=gfx950 -O1 -g -std=c++17 -fPIC -shared \
    -Xclang -target-feature -Xclang -packed-fp32-ops \
    -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
    -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer \
    -I include -o _build/libspec_san.so speculative_decoding_spec_amd/csrc/*.hip
ASAN_RT="$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)"
SPEC_LIB_PATH=_build/libspec_san.so ASAN_OPTIONS=detect_leaks=0 LD_PRELOAD="$ASAN_RT" \
    python -m pytest tests/test_abi.py tests/test_workspace_cache.py -q -p no:cacheprovider
echo "sanitizer runs clean"
