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

// Loads one full trip (every vector exists): no predication.
__device__ __forceinline__ void load_full(const uint4* __restrict__ row, int v0, int lane,
                                          uint4 d[kU]) {
  const uint4* base = row + v0;
#pragma unroll
  for (int u = 0; u < kU; ++u) d[u] = base[u * kWave + lane];
}

// Streams vectors [0, nvec) of a row through consume(d, v0, maybe_last), one trip of kU
// vectors per lane at a time, with DEPTH trips of loads in flight. The steady-state loop
// loads full trips only, unpredicated, so that the compiler can keep the younger trips'
// loads outstanding while it consumes the oldest; the last few full trips and the partial
// trip follow it. maybe_last is true only where the trip may hold vector nvec - 1.
template <int DEPTH, typename F>
__device__ __forceinline__ void stream_row(const uint4* __restrict__ row, int nvec, int lane,
                                           F&& consume) {
  constexpr int kStep = kU * kWave;
  const int nfull = nvec / kStep;
  int t = 0;
  if (nfull >= DEPTH) {
    uint4 buf[DEPTH][kU];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) load_full(row, s * kStep, lane, buf[s]);
    // Issue priority falls with progress (quarters of the row): of the waves sharing a SIMD,
    // the one furthest behind is served first, which narrows the spread of finish times.
    __builtin_amdgcn_s_setprio(3);
    for (; t + 2 * DEPTH <= nfull; t += DEPTH) {  // trips t .. t+DEPTH-1; none is the last
      const int lvl = (4 * t) / nfull;
      if (lvl == 1) __builtin_amdgcn_s_setprio(2);
      else if (lvl == 2) __builtin_amdgcn_s_setprio(1);
      else if (lvl == 3) __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        consume(buf[s], (t + s) * kStep, false);
        load_full(row, (t + s + DEPTH) * kStep, lane, buf[s]);
      }
    }
    // DEPTH .. 2*DEPTH-1 full trips remain; the first DEPTH of them are loaded
#pragma unroll
    for (int s = 0; s < 2 * DEPTH - 1; ++s) {
      if (t + s < nfull) {
        consume(buf[s % DEPTH], (t + s) * kStep, true);
        if (t + s + DEPTH < nfull) load_full(row, (t + s + DEPTH) * kStep, lane, buf[s % DEPTH]);
      }
    }
    t = nfull;
    __builtin_amdgcn_s_setprio(0);
  }
  for (; t * kStep < nvec; ++t) {  // short rows, and the partial trip
    uint4 d[kU];
    load_trip(row, t * kStep, nvec, lane, d);
    consume(d, t * kStep, true);
  }
}

// Streams the trips first, first + step, first + 2*step, ... of a row (a trip is kU vectors
// per lane at kU * kWave vectors apart from the next trip) through consume(d, v0,
// maybe_last), with DEPTH of this wave's trips of loads in flight: the waves of a workgroup
// pass first = 0 .. step-1 and together cover the row once, each wave's stream a regular
// stride of full trips (unpredicated loads) plus, for one of them, the row's partial trip.
// Issue priority falls with the wave's progress, as in stream_row.
template <int DEPTH, typename F>
__device__ __forceinline__ void stream_row_strided(const uint4* __restrict__ row, int nvec,
                                                   int lane, int first, int step, F&& consume) {
  constexpr int kStep = kU * kWave;
  const int nfull = nvec / kStep;
  const int nf = first < nfull ? (nfull - 1 - first) / step + 1 : 0;  // this wave's full trips
  auto v0_of = [&](int i) { return (first + i * step) * kStep; };
  int i = 0;
  if (nf >= DEPTH) {
    uint4 buf[DEPTH][kU];
#pragma unroll
    for (int s = 0; s < DEPTH; ++s) load_full(row, v0_of(s), lane, buf[s]);
    const int q1 = nf / 4, q2 = nf / 2, q3 = (3 * nf) / 4;
    __builtin_amdgcn_s_setprio(3);
    for (; i + 2 * DEPTH <= nf; i += DEPTH) {  // trips i .. i+DEPTH-1; none is the row's last
      if (i >= q3) __builtin_amdgcn_s_setprio(0);
      else if (i >= q2) __builtin_amdgcn_s_setprio(1);
      else if (i >= q1) __builtin_amdgcn_s_setprio(2);
#pragma unroll
      for (int s = 0; s < DEPTH; ++s) {
        consume(buf[s], v0_of(i + s), false);
        load_full(row, v0_of(i + s + DEPTH), lane, buf[s]);
        __builtin_amdgcn_sched_barrier(0);  // the reload issues before the next trip's waits
      }
    }
    // DEPTH .. 2*DEPTH-1 full trips remain; the first DEPTH of them are loaded
#pragma unroll
    for (int s = 0; s < 2 * DEPTH - 1; ++s) {
      if (i + s < nf) {
        consume(buf[s % DEPTH], v0_of(i + s), true);
        if (i + s + DEPTH < nf) load_full(row, v0_of(i + s + DEPTH), lane, buf[s % DEPTH]);
      }
    }
    i = nf;
    __builtin_amdgcn_s_setprio(0);
  }
  for (; i < nf; ++i) {  // fewer than DEPTH full trips
    uint4 d[kU];
    load_full(row, v0_of(i), lane, d);
    consume(d, v0_of(i), true);
  }
  if (nfull * kStep < nvec && nfull >= first && (nfull - first) % step == 0) {  // partial trip
    uint4 d[kU];
    load_trip(row, nfull * kStep, nvec, lane, d);
    consume(d, nfull * kStep, true);
  }
}

// Spare load target: a claim past a row's full trips loads these 4 KB instead (data never
// used), so that the row streams' loads are all issued unconditionally.
static __device__ uint4 g_spare_trip[kU * kWave];

// Streams the full trips of a row that this wave claims from a counter shared by the
// workgroup's waves (one LDS atomic per trip, issued before the consume so that its latency
// hides behind it), DEPTH trips of loads in flight: a wave that runs faster takes more trips,
// so the waves of a row finish together. The wave that claims index nfull also streams the
// row's partial trip, if there is one. consume(d, v0, maybe_last) as in stream_row.
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

__device__ __forceinline__ int row_argmax(const uint4* __restrict__ row, int nvec, int V,
                                          int lane) {
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF;
  stream_row<2>(row, nvec, lane, [&](uint4* d, int v0, bool) {
    argmax_trip(d, v0, nvec, V, lane, bv, bi);
  });
  wave_argmax(bv, bi);
  return bi == 0x7FFFFFFF ? 0 : bi;
}

}  // namespace specv
