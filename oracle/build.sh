#!/bin/sh
# Builds the CPU oracle (test infrastructure) as a shared library with gcc.
set -e
cd "$(dirname "$0")"
gcc -O2 -std=c11 -fPIC -shared -fopenmp -Wall -Wextra -o libbsa_oracle.so bsa_oracle.c -lm
