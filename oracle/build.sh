#!/bin/sh
# Builds the CPU oracle shared library (test infrastructure only).
set -e
cd "$(dirname "$0")"
gcc -O2 -fopenmp -fPIC -shared -std=c11 -Wall -Wextra -o liboracle.so moe_oracle.c -lm
