// Work partition map of the decode kernels (which compute it in assembly with
// the same formulas) and the combine kernel.
//
// The rows of the whole batch are cut into 64-row units (one cache page each),
// sequence after sequence: sequence b owns units [u0(b), u0(b) + units(b)),
// units(b) = max(1, ceil(seq_len[b] / 64)) (a sequence with no row still owns
// one unit, so that its empty result gets written).  Partition p of P covers
// units [start(p), start(p+1)) with start(p) = floor(p * U / P), U the total.
// A partition therefore sees at most two sequences that are cut across
// partitions: the one it starts in (partial slot 0) and the one it ends in
// (partial slot 1).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace mla {

__device__ __forceinline__ int units_of_len(int len) { return len > 64 ? (len + 63) >> 6 : 1; }

// parts = 2^log2_parts, so the division is a shift
__device__ __forceinline__ int part_start(int p, int total_units, int log2_parts) {
  return (int)(((long long)p * total_units) >> log2_parts);
}

// The partition whose range holds unit u: the largest p with start(p) <= u.
__device__ __forceinline__ int part_of_unit(int u, int total_units, int parts) {
  return (int)((((long long)u + 1) * parts - 1) / total_units);
}

}  // namespace mla
