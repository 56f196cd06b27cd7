// row_ops.h -- one wave streaming one bf16 logits row: coalesced 16-byte loads of kU vectors
// per lane per trip, masking of a partial last vector, and the row argmax.
#pragma once

#include "spec_device.h"

namespace specv {

constexpr int kU = 4;  // vectors per row per lane per trip

// One 16-byte vector of a logits row, loaded with the nontemporal hint: the row streams
// read each row once, and they run faster with it than with plain loads.
__device__ __forceinline__ uint4 ld_row(const uint4* p) {
  typedef uint32_t v4u __attribute__((ext_vector_type(4)));
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Loads kU vectors of one row for this lane; vectors past the row read as -inf. A full trip
// (every trip but possibly the last) loads from a uniform base with the lane's offset and an
// immediate per vector: no predication and no per-load address arithmetic.
__device__ __forceinline__ void load_trip(const uint4* __restrict__ row, int v0, int nvec,
                                          int lane, uint4 d[kU]) {
  const uint4* base = row + v0;
  if (v0 + kU * kWave <= nvec) {
#pragma unroll
    for (int u = 0; u < kU; ++u) d[u] = ld_row(base + u * kWave + lane);
  } else {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int v = v0 + u * kWave + lane;
      d[u] = (v < nvec) ? ld_row(base + u * kWave + lane)
                        : make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u);
    }
  }
}

// Loads one full trip (every vector exists): no predication.
__device__ __forceinline__ void load_full(const uint4* __restrict__ row, int v0, int lane,
                                          uint4 d[kU]) {
  const uint4* base = row + v0;
#pragma unroll
  for (int u = 0; u < kU; ++u) d[u] = ld_row(base + u * kWave + lane);
}

// Spare load target: a claim past a row's full trips loads these 4 KB instead (data never
// used), so that the row streams' loads are all issued unconditionally.
static __device__ uint4 g_spare_trip[kU * kWave];

// Streams the full trips of a row that this wave claims from a counter shared by the
// workgroup's waves (one LDS atomic per trip, issued before the consume so that its latency
// hides behind it), DEPTH trips of loads in flight: a wave that runs faster takes more trips,
// so the waves of a row finish together. The wave that claims index nfull also streams the
// row's partial trip, if there is one. consume(d, v0, maybe_last) takes a trip of
// kU vectors per lane starting at vector v0; maybe_last is true where it may hold vector nvec - 1.
template <int DEPTH, typename F>
__device__ __forceinline__ void stream_row_claimed(const uint4* __restrict__ row, int nvec,
                                                   int lane, int* ctr, F&& consume) {
  constexpr int kStep = kU * kWave;
  const int nfull = nvec / kStep;
  // A claim is issued by lane 0 and read back (readfirstlane) only where it is needed, so
  // that the consume between the two hides the atomic's latency.
  auto claim_issue = [&]() {
    int t = 0;
    if (lane == 0) t = atomicAdd(ctr, 1);
    return t;  // the claim in lane 0
  };
  auto claim = [&]() { return __builtin_amdgcn_readfirstlane(claim_issue()); };
  auto src = [&](int t) { return t < nfull ? row + t * kStep : g_spare_trip; };
  bool partial = false;  // this wave claimed index nfull
  uint4 buf[DEPTH][kU];
  int tc[DEPTH];
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) {
    tc[s] = claim();
    partial |= tc[s] == nfull;
    load_full(src(tc[s]), 0, lane, buf[s]);
  }
  // Each wave's claims grow and its buffers hold them in claim order (tc[0] < tc[1] < ...):
  // once tc[0] is past the full trips, so are the others.
  while (tc[0] < nfull) {
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) {
      const int tq = claim_issue();
      if (tc[s] < nfull) consume(buf[s], tc[s] * kStep, tc[s] == nfull - 1);
      const int tn = __builtin_amdgcn_readfirstlane(tq);
      partial |= tn == nfull;
      load_full(src(tn), 0, lane, buf[s]);
      __builtin_amdgcn_sched_barrier(0);  // the reload issues before the next trip's waits
      tc[s] = tn;
    }
  }
  if (partial && nfull * kStep < nvec) {
    uint4 d[kU];
    load_trip(row, nfull * kStep, nvec, lane, d);
    consume(d, nfull * kStep, true);
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

}  // namespace specv
