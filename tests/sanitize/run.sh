#!/bin/bash
# Host-side AddressSanitizer + UndefinedBehaviorSanitizer run of the CPU tests that exercise
# native code without a GPU: the C ABI's argument checks and workspace queries
# (tests/test_abi.py) and the fp64 oracle against its pins (tests/test_oracle_pins.py).
# Device code is compiled as usual; only the host code carries the sanitizers.  Builds go to
# a temporary directory; nothing in the tree is replaced.
#   usage: tests/sanitize/run.sh
set -euo pipefail
ROOT=$(cd "$(dirname "$0")/../.." && pwd)
OUT=$(mktemp -d /tmp/ssm_sanitize.XXXXXX)
HIPCC=${HIPCC:-/opt/rocm/bin/hipcc}
CLANG=${CLANG:-/opt/rocm/lib/llvm/bin/clang}
RT=$("$CLANG" -print-file-name=libclang_rt.asan-x86_64.so)
[ -f "$RT" ] || RT=$(ls /opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so | head -1)
SAN="-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-omit-frame-pointer -Xarch_host -fno-sanitize-recover=all"
echo "== host-sanitized HIP library -> $OUT"
objs=(); pids=()
for src in abi bwd conv init_state pool recurrent ssd vdecay; do
  $HIPCC -O1 -g -std=c++17 -fPIC --offload-arch=gfx950 -Xclang -target-feature -Xclang -packed-fp32-ops \
    $SAN -c "$ROOT/ssm_sequence_models_amd/csrc/$src.hip" -o "$OUT/$src.o" &
  objs+=("$OUT/$src.o"); pids+=($!)
done
for p in "${pids[@]}"; do wait "$p"; done
$HIPCC -shared -fPIC --offload-arch=gfx950 -shared-libsan $SAN "${objs[@]}" -o "$OUT/libssm_mi355x.so"
echo "== sanitized oracle"
"$CLANG" -O1 -g -std=c11 -fPIC -shared -ffp-contract=off -fsanitize=address,undefined \
  -fno-sanitize-recover=all -fno-omit-frame-pointer -shared-libsan \
  "$ROOT/oracle/ssm_oracle.c" -o "$OUT/libssm_oracle.so" -lm
echo "== tests under the sanitizers"
cd "$ROOT"
# --capture=sys: a sanitizer report is written to file descriptor 2 just before the abort, so
# it must not be held in pytest's fd-level capture.
set +e
LD_PRELOAD="$RT" ASAN_OPTIONS=detect_leaks=0:halt_on_error=1:abort_on_error=1 \
  UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \
  SSM_LIB_PATH="$OUT/libssm_mi355x.so" ORACLE_LIB_PATH="$OUT/libssm_oracle.so" \
  python -m pytest tests/test_abi.py tests/test_oracle_pins.py -v -m "not gpu" -p no:cacheprovider --capture=sys
rc=$?; rm -rf "$OUT"; exit $rc
