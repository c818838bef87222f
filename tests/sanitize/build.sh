#!/bin/bash
# Host-only build of libgc's C ABI layer (api.cpp) with AddressSanitizer and
# UndefinedBehaviorSanitizer, linked against launch stubs (no GPU code, no HIP
# runtime): tests/sanitize/abi_fuzz, run by tests/test_host_sanitize.py.
#   usage: tests/sanitize/build.sh OUTPUT
set -e
HERE="$(cd "$(dirname "$0")" && pwd)"
ROOT="$(dirname "$(dirname "$HERE")")"
ROCM="${ROCM_PATH:-/opt/rocm}"
g++ -std=c++17 -O1 -g -fsanitize=address,undefined -fno-sanitize-recover=undefined -fno-omit-frame-pointer \
    -D__HIP_PLATFORM_AMD__ -I"$ROOT/include" -I"$ROOT/collective_communication_reduction_amd/csrc" -I"$HERE" \
    -I"$ROCM/include" \
    "$ROOT/collective_communication_reduction_amd/csrc/api.cpp" "$HERE/launch_stubs.cpp" "$HERE/abi_fuzz.cpp" \
    -o "$1"
