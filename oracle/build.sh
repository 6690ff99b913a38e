#!/bin/sh
# Builds the CPU oracle (test infrastructure) as oracle/liboracle.so.
set -e
cd "$(dirname "$0")"
gcc -O2 -fopenmp -fPIC -shared -std=c11 -Wall -Wextra -o liboracle.so oracle.c -lm
