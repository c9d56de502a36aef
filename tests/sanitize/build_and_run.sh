#!/bin/bash
# Builds liblora with AddressSanitizer and UndefinedBehaviorSanitizer on its
# host code only (each -fsanitize= behind -Xarch_host; the GPU code is built
# as usual and never runs here), links it with tests/sanitize/abi_driver.cpp
# and runs the driver on the CPU.  Usage: build_and_run.sh <output directory>
set -euo pipefail
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(cd "$HERE/../.." && pwd)"
OUT="$1"
mkdir -p "$OUT"
CSRC="$ROOT/lora_linear_fwd_amd/csrc"
HIPCC="${HIPCC:-/opt/rocm/bin/hipcc}"
FLAGS=(--offload-arch=gfx950 -O1 -g -std=c++17 -I "$ROOT/include" -I "$CSRC"
       -Xclang -target-feature -Xclang -packed-fp32-ops
       -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined
       -Xarch_host -fno-sanitize-recover=undefined -Xarch_host -fno-omit-frame-pointer)
objs=()
for src in api.cpp gemm_nt.hip gemm_nt_q4.hip gemm_nn.hip gemm_nn_q4.hip gemm_nt_q4dq.hip gemm_nn_q4dq.hip; do
  o="$OUT/${src%.*}.o"
  "$HIPCC" "${FLAGS[@]}" -x hip -c "$CSRC/$src" -o "$o" &
  objs+=("$o")
done
wait
"$HIPCC" "${FLAGS[@]}" -x c++ -c "$HERE/abi_driver.cpp" -o "$OUT/abi_driver.o"
"$HIPCC" --offload-arch=gfx950 -Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined \
  -o "$OUT/abi_driver" "$OUT/abi_driver.o" "${objs[@]}"
ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=print_stacktrace=1 "$OUT/abi_driver"
