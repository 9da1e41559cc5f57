#!/bin/bash
# Sanitizer build of the host code: the libwqmm runtime (its host half; the
# device code is compiled as usual) and the CPU oracle, with AddressSanitizer
# and UndefinedBehaviorSanitizer, linked with the unmodified kernel objects into
# one instrumented test program.  usage: build.sh OUTDIR
set -euo pipefail
HERE=$(cd "$(dirname "$0")" && pwd)
ROOT=$(cd "$HERE/../.." && pwd)
PKG=$ROOT/weight_only_quantized_matmul_amd
OUT=$1
mkdir -p "$OUT"
SAN="-fsanitize=address,undefined -fno-sanitize-recover=all -fno-omit-frame-pointer"
CLANG=/opt/rocm/llvm/bin/clang
# runtime: HIP source; sanitizers on the host pass only
/opt/rocm/bin/hipcc -x hip --offload-arch=gfx950 -O1 -g -fPIC -std=c++17 -I "$ROOT/include" -I "$PKG/csrc" \
  -Xclang -target-feature -Xclang -packed-fp32-ops \
  -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -Xarch_host -fno-sanitize-recover=all -Xarch_host -fno-omit-frame-pointer \
  -c "$PKG/csrc/runtime.cpp" -o "$OUT/runtime_san.o"
$CLANG $SAN -O1 -g -std=c11 -ffp-contract=off -c "$ROOT/oracle/oracle.c" -o "$OUT/oracle_san.o"
$CLANG $SAN -O1 -g -std=c11 -I "$ROOT/include" -c "$HERE/sanitize_main.c" -o "$OUT/main_san.o"
# kernel objects as built by the package build (device code plus host launch stubs)
KOBJ=$(ls "$PKG"/_build/*.hip.o)
/opt/rocm/llvm/bin/clang++ $SAN -o "$OUT/sanitize_main" "$OUT/main_san.o" "$OUT/runtime_san.o" "$OUT/oracle_san.o" \
  $KOBJ -L/opt/rocm/lib -lamdhip64 -Wl,-rpath,/opt/rocm/lib -lm
echo "$OUT/sanitize_main"
