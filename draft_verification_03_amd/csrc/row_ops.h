// row_ops.h -- one wave streaming one bf16 logits row: coalesced 16-byte loads of kU vectors
// per lane per trip, masking of a partial last vector, and the row argmax.
#pragma once

#include "spec_device.h"

namespace specv {

constexpr int kU = 4;  // vectors per row per lane per trip

// Loads kU vectors of one row for this lane; vectors past the row read as -inf. A full trip
// (every trip but possibly the last) loads from a uniform base with the lane's offset and an
// immediate per vector: no predication and no per-load address arithmetic.
__device__ __forceinline__ void load_trip(const uint4* __restrict__ row, int v0, int nvec,
                                          int lane, uint4 d[kU]) {
  const uint4* base = row + v0;
  if (v0 + kU * kWave <= nvec) {
#pragma unroll
    for (int u = 0; u < kU; ++u) d[u] = base[u * kWave + lane];
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * kWave + lane;
      d[u] = (v < nvec) ? base[u * kWave + lane]
                        : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
    }
  }
}

// Masks the logits of the last, partial vector (V not a multiple of 8) to -inf; only the
// last trip of a row can hold it.
__device__ __forceinline__ void mask_tail(uint4 d[kU], int v0, int nvec, int V, int lane) {
  const int rem = V & 7;
  if (rem == 0 || v0 + kU * kWave < nvec) return;
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
// Greedy rows: argmax with the lowest index on ties. Loads are double-buffered; the lane's
// best is only revisited when a trip holds a larger value (rare after the first trips).
// ----------------------------------------------------------------------------------------
__device__ __forceinline__ void argmax_trip(uint4 d[kU], int v0, int nvec, int V, int lane,
                                            float& bv, int& bi) {
  mask_tail(d, v0, nvec, V, lane);
  float vm[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    float x[8];
    unpack8(d[u], x);
    vm[u] = max8(x);
  }
  static_assert(kU == 4, "trip max below assumes four vectors per trip");
  const float tm = vmax3(vmax3(vm[0], vm[1], vm[2]), vm[3], vm[3]);
  if (tm > bv) {  // this lane's earliest occurrence of tm in the trip
    int found = 0x7FFFFFFF;
#pragma unroll
    for (int u = kU - 1; u >= 0; --u) {
      if (vm[u] == tm) {
        float x[8];
        unpack8(d[u], x);
        int e = 7;
#pragma unroll
        for (int j = 7; j >= 0; --j)
          if (x[j] == tm) e = j;
        found = (v0 + u * kWave + lane) * 8 + e;
      }
    }
    bv = tm;
    bi = found;
  }
}

// Argmax of vectors [cv0, cv1) of a row (cv0 a multiple of the trip): the wave's largest
// value and its lowest index.
__device__ __forceinline__ void row_argmax_range(const uint4* __restrict__ row, int cv0,
                                                 int cv1, int nvec, int V, int lane, float& v,
                                                 int& i) {
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  constexpr int kStep = kU * kWave;
  uint4 a[kU], b[kU];
  load_trip(row, cv0, cv1, lane, a);
  for (int v0 = cv0; v0 < cv1; v0 += 2 * kStep) {
    const int v1 = v0 + kStep;
    if (v1 < cv1) load_trip(row, v1, cv1, lane, b);
    argmax_trip(a, v0, nvec, V, lane, bv, bi);
    if (v1 >= cv1) break;
    if (v1 + kStep < cv1) load_trip(row, v1 + kStep, cv1, lane, a);
    argmax_trip(b, v1, nvec, V, lane, bv, bi);
  }
  wave_argmax(bv, bi);
  v = bv;
  i = bi == 0x7FFFFFFF ? cv0 * 8 : bi;
}

__device__ __forceinline__ int row_argmax(const uint4* __restrict__ row, int nvec, int V,
                                          int lane) {
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  constexpr int kStep = kU * kWave;
  uint4 a[kU], b[kU];
  load_trip(row, 0, nvec, lane, a);
  for (int v0 = 0; v0 < nvec; v0 += 2 * kStep) {
    const int v1 = v0 + kStep;
    if (v1 < nvec) load_trip(row, v1, nvec, lane, b);
    argmax_trip(a, v0, nvec, V, lane, bv, bi);
    if (v1 >= nvec) break;
    if (v1 + kStep < nvec) load_trip(row, v1 + kStep, nvec, lane, a);
    argmax_trip(b, v1, nvec, V, lane, bv, bi);
  }
  wave_argmax(bv, bi);
  return bi == 0x7FFFFFFF ? 0 : bi;
}

}  // namespace specv
