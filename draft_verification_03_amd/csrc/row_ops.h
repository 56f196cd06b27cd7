// row_ops.h -- one wave streaming one bf16 logits row: coalesced 16-byte loads of kU vectors
// per lane per trip, masking of a partial last vector, and the row argmax.
#pragma once

#include "spec_device.h"

namespace specv {

constexpr int kU = 4;  // vectors per row per lane per trip

// Loads kU vectors of one row for this lane; vectors past the row read as -inf.
__device__ __forceinline__ void load_trip(const uint4* __restrict__ row, int v0, int nvec,
                                          int lane, uint4 d[kU]) {
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int v = v0 + u * kWave + lane;
    if (v < nvec) d[u] = row[v];
    else d[u] = make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
  }
}

// Masks the logits of the last, partial vector (V not a multiple of 8) to -inf.
__device__ __forceinline__ void mask_tail(uint4 d[kU], int v0, int nvec, int V, int lane) {
  const int rem = V & 7;
  if (rem == 0) return;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int v = v0 + u * kWave + lane;
    if (v == nvec - 1) {
      uint32_t w[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (e >= rem) {
          if (e & 1) w[e >> 1] = (w[e >> 1] & 0x0000FFFFu) | 0xFF800000u;
          else w[e >> 1] = (w[e >> 1] & 0xFFFF0000u) | 0x0000FF80u;
        }
      }
      d[u] = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }
}

// ----------------------------------------------------------------------------------------
// Greedy rows: argmax with the lowest index on ties.
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ int row_argmax(const uint4* __restrict__ row, int nvec, int V,
                                          int lane) {
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  for (int v0 = 0; v0 < nvec; v0 += kU * kWave) {
    uint4 d[kU];
    load_trip(row, v0, nvec, lane, d);
    mask_tail(d, v0, nvec, V, lane);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float x[8];
      unpack8(d[u], x);
      const float vm = max8(x);
      if (vm > bv) {  // this lane's vectors come in increasing index order
        int e = 7;
#pragma unroll
        for (int j = 7; j >= 0; --j)
          if (x[j] == vm) e = j;
        bv = vm;
        bi = (v0 + u * kWave + lane) * 8 + e;
      }
    }
  }
  wave_argmax(bv, bi);
  return bi == 0x7FFFFFFF ? 0 : bi;
}

}  // namespace specv
