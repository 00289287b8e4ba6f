// Work partition map of the decode kernels (which compute it in assembly with
// the same formulas) and the combine kernel.
//
// The rows of the whole batch are cut into 64-row units (one cache page each),
// sequence after sequence: sequence b owns units [u0(b), u0(b) + units(b)),
// units(b) = max(1, ceil(seq_len[b] / 64)) (a sequence with no row still owns
// one unit, so that its empty result gets written).  Besides its units every
// sequence weighs kSegWeight units of fixed cost (its start, its last output,
// its epilogue), placed before its units: unit u of sequence b has the
// weighted position pos(u) = u + (b + 1) kSegWeight.  Partition p of P takes
// the units whose positions fall in [start(p), start(p+1)),
// start(p) = floor(p * W / P), W = total units + batch * kSegWeight, so that
// partitions that hold more sequence boundaries get fewer units.  A
// partition's units are consecutive; it sees at most two sequences that are
// cut across partitions: the one it starts in (partial slot 0) and the one it
// ends in (partial slot 1).
#pragma once
#include <stdint.h>
#include <hip/hip_runtime.h>

namespace mla {

constexpr int kSegWeight = 3;

__device__ __forceinline__ int units_of_len(int len) { return len > 64 ? (len + 63) >> 6 : 1; }

// parts = 2^log2_parts, so the division is a shift
__device__ __forceinline__ int part_start(int p, int total_weight, int log2_parts) {
  return (int)(((long long)p * total_weight) >> log2_parts);
}

// The partition whose position range holds position x: the largest p with start(p) <= x.
__device__ __forceinline__ int part_of_pos(int x, int total_weight, int parts) {
  return (int)((((long long)x + 1) * parts - 1) / total_weight);
}

}  // namespace mla
