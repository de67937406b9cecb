#!/bin/bash
# AddressSanitizer and UndefinedBehaviorSanitizer runs of the host code:
#  1. the oracle (oracle/oracle.c, built with gcc) under the CPU test suite;
#  2. the C-ABI library's host code (every hipcc compile and the link get
#     -Xarch_host -fsanitize=...; the gfx950 device code is built as usual)
#     under the ABI host tests (argument checks, workspace sizes, error
#     paths, the allocation-free entry point's limits) and the host tests of
#     pass planning (phase links and the schedule of whole stacks).
# Everything is built in a scratch copy of the sources (SV_SAN_DIR, default
# /tmp/sv_sanitize), so the in-tree builds are untouched.  gcc's and clang's
# sanitizer runtimes cannot share a process, so the two parts run in
# separate pytest processes; a preload already in the environment is kept,
# after the sanitizer runtime.
set -euo pipefail
R=$(cd "$(dirname "$0")/.." && pwd)
D=${SV_SAN_DIR:-/tmp/sv_sanitize}
rm -rf "$D/src"
mkdir -p "$D/src"
(cd "$R" && tar --exclude=./_work --exclude=./gpurun_out --exclude=./_build --exclude=./.git -cf - .) | tar -xf - -C "$D/src"
cd "$D/src"
export ASAN_OPTIONS=detect_leaks=0:halt_on_error=1:verify_asan_link_order=0
export UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1
PRE=${LD_PRELOAD:-}

echo "== oracle with gcc ASan + UBSan, CPU tests"
gcc -O1 -g -std=c11 -ffp-contract=off -fno-fast-math -fsanitize=address,undefined -fno-sanitize-recover=undefined \
    -fno-omit-frame-pointer -fPIC -shared -pthread -o oracle/liboracle.so oracle/oracle.c -lm
GCC_RT="$(gcc -print-file-name=libasan.so):$(gcc -print-file-name=libubsan.so)"
LD_PRELOAD="$GCC_RT${PRE:+:$PRE}" python -m pytest tests -q -m "not gpu" -p no:cacheprovider \
    --deselect tests/test_abi_host.py --deselect tests/test_schedule_host.py

echo "== library host code with clang ASan + UBSan"
python - <<'PY'
import sys
sys.path.insert(0, ".")
from speculative_decoding_verification_amd import _build
host = []
for f in ("-fsanitize=address", "-fsanitize=undefined", "-fno-sanitize-recover=undefined",
          "-fno-omit-frame-pointer", "-g"):
    host += ["-Xarch_host", f]
link = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-shared-libsan"]
print(_build.build(verbose=True, extra=host, link_extra=link))
PY
# the oracle again without sanitizers: gcc's runtime is not in this process
python -c "import sys; sys.path.insert(0, '.'); import oracle; oracle.build(force=True)"
CLANG_RT=$(ls /opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
LD_PRELOAD="$CLANG_RT${PRE:+:$PRE}" python -m pytest tests/test_abi_host.py tests/test_schedule_host.py -q \
    -p no:cacheprovider
echo "sanitizer runs passed"
