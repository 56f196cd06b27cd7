// spec_device.h -- device helpers shared by the gfx950 kernels of libspecv: bf16 unpacking,
// order-preserving bf16 keys, the Philox4x32-10 uniform stream and wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kWave = 64;

// ---- bf16 ----------------------------------------------------------------------------------
// A dword holds two bf16 logits; each is the top half of an IEEE binary32, so the
// conversion is exact: the low element is shifted up, the high element masked.
__device__ __forceinline__ float bf_lo(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const uint4& d, float x[8]) {
  x[0] = bf_lo(d.x); x[1] = bf_hi(d.x);
  x[2] = bf_lo(d.y); x[3] = bf_hi(d.y);
  x[4] = bf_lo(d.z); x[5] = bf_hi(d.z);
  x[6] = bf_lo(d.w); x[7] = bf_hi(d.w);
}

// max of three in one v_max3_f32. Written as one instruction because the compiler's fmaxf
// must first canonicalise operands that come from bit casts (IEEE NaN quieting), which
// doubles the cost of a max reduction over unpacked logits. Logits are never NaN (the ABI
// says so), where v_max3_f32 and fmaxf agree.
__device__ __forceinline__ float vmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float max8(const float x[8]) {
  return vmax3(vmax3(x[0], x[1], x[2]), vmax3(x[3], x[4], x[5]), vmax3(x[6], x[7], x[7]));
}

// Order-preserving 16-bit key of a bf16 value (larger float <=> larger key), with -0 folded
// onto +0 so that keys compare exactly like the floats they encode. Used for threshold
// searches over the distinct logit values of a row.
__device__ __forceinline__ uint32_t key_of_bits(uint32_t b16) {
  b16 = (b16 == 0x8000u) ? 0u : b16;
  return (b16 & 0x8000u) ? (~b16 & 0xFFFFu) : (b16 | 0x8000u);
}
__device__ __forceinline__ uint32_t key_of(float bf_value) {
  return key_of_bits(__float_as_uint(bf_value) >> 16);
}
__device__ __forceinline__ float value_of_key(uint32_t key) {
  uint32_t b16 = (key & 0x8000u) ? (key & 0x7FFFu) : (~key & 0xFFFFu);
  return __uint_as_float(b16 << 16);
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ----------------------------------
// Counter (id, pos, purpose, 0), key (seed low word, seed high word); ten rounds of the
// 4x32 S-box with the Weyl key schedule. Only the first output word is used.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint32_t a0 = 0xD2511F53u * c0, h0 = __umulhi(0xD2511F53u, c0);
    const uint32_t a1 = 0xCD9E8D57u * c2, h1 = __umulhi(0xCD9E8D57u, c2);
    const uint32_t n0 = h1 ^ c1 ^ k0;
    const uint32_t n2 = h0 ^ c3 ^ k1;
    c0 = n0;
    c1 = a1;
    c2 = n2;
    c3 = a0;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// u = (word0 >> 8) * 2^-24: a 24-bit dyadic in [0, 1), exact in fp32.
__device__ __forceinline__ float uniform24(uint32_t seed_lo, uint32_t seed_hi, uint32_t id,
                                           uint32_t pos, uint32_t purpose) {
  return (float)(philox_word0(id, pos, purpose, 0u, seed_lo, seed_hi) >> 8) *
         (1.0f / 16777216.0f);
}

// ---- wave64 reductions -------------------------------------------------------------------
// XOR butterflies: every lane combines the same two operands at every level, so every lane
// ends with bit-identical results (fp addition is commutative), and the order is fixed, so
// results are reproducible run to run.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Wave maximum through DPP moves (quad permutes, half-row and row mirrors, row broadcasts
// 15 and 31), read back from lane 63: no LDS traffic. Lanes a masked DPP row does not write
// keep their own value, which leaves the maximum unchanged.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_max_step(float v) {
  const int o = __builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROW_MASK,
                                            0xF, false);
  return vmax3(v, __int_as_float(o), __int_as_float(o));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = dpp_max_step<0xB1>(v);         // quad_perm [1,0,3,2]
  v = dpp_max_step<0x4E>(v);         // quad_perm [2,3,0,1]
  v = dpp_max_step<0x141>(v);        // row_half_mirror
  v = dpp_max_step<0x140>(v);        // row_mirror
  v = dpp_max_step<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max_step<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// DPP move with 0 for lanes that have no source (row edges, rows outside ROW_MASK).
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_or_zero(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, false);
}
// Wave sum through DPP (the same tree as wave_max_dpp), read back from lane 63; fixed order.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(dpp_or_zero<0xB1>(__float_as_int(v)));        // quad_perm [1,0,3,2]
  v += __int_as_float(dpp_or_zero<0x4E>(__float_as_int(v)));        // quad_perm [2,3,0,1]
  v += __int_as_float(dpp_or_zero<0x141>(__float_as_int(v)));       // row_half_mirror
  v += __int_as_float(dpp_or_zero<0x140>(__float_as_int(v)));       // row_mirror
  v += __int_as_float(dpp_or_zero<0x142, 0xA>(__float_as_int(v)));  // row_bcast:15
  v += __int_as_float(dpp_or_zero<0x143, 0xC>(__float_as_int(v)));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
// Inclusive prefix sum over the wave through DPP: shifts by 1, 2, 4, 8 inside each row of 16
// lanes, then the row totals carried by row broadcasts 15 and 31.
__device__ __forceinline__ int wave_incl_scan_dpp(int v) {
  v += dpp_or_zero<0x111>(v);       // row_shr:1
  v += dpp_or_zero<0x112>(v);       // row_shr:2
  v += dpp_or_zero<0x114>(v);       // row_shr:4
  v += dpp_or_zero<0x118>(v);       // row_shr:8
  v += dpp_or_zero<0x142, 0xA>(v);  // row_bcast:15
  v += dpp_or_zero<0x143, 0xC>(v);  // row_bcast:31
  return v;
}
__device__ __forceinline__ float wave_incl_scan_dpp_f(float v) {
  v += __int_as_float(dpp_or_zero<0x111>(__float_as_int(v)));
  v += __int_as_float(dpp_or_zero<0x112>(__float_as_int(v)));
  v += __int_as_float(dpp_or_zero<0x114>(__float_as_int(v)));
  v += __int_as_float(dpp_or_zero<0x118>(__float_as_int(v)));
  v += __int_as_float(dpp_or_zero<0x142, 0xA>(__float_as_int(v)));
  v += __int_as_float(dpp_or_zero<0x143, 0xC>(__float_as_int(v)));
  return v;
}
// The same for 64-bit values (the two halves moved separately, added with carry).
__device__ __forceinline__ uint64_t dpp_add_u64_step(uint64_t v, uint32_t lo, uint32_t hi) {
  return v + (((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ uint64_t wave_incl_scan_dpp_u64(uint64_t v) {
#define SPECV_SCAN_STEP(CTRL, MASK)                                                          \
  v = dpp_add_u64_step(v, (uint32_t)dpp_or_zero<CTRL, MASK>((int)(uint32_t)v),              \
                       (uint32_t)dpp_or_zero<CTRL, MASK>((int)(uint32_t)(v >> 32)));
  SPECV_SCAN_STEP(0x111, 0xF)
  SPECV_SCAN_STEP(0x112, 0xF)
  SPECV_SCAN_STEP(0x114, 0xF)
  SPECV_SCAN_STEP(0x118, 0xF)
  SPECV_SCAN_STEP(0x142, 0xA)
  SPECV_SCAN_STEP(0x143, 0xC)
#undef SPECV_SCAN_STEP
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, o, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), o, kWave);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}
__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
  return v;
}
// (value, index) maximum: larger value wins, the lower index on equal values.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, kWave);
    int oi = __shfl_xor(i, o, kWave);
    if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
  }
}
// Inclusive prefix sum over the wave (Hillis-Steele; fixed order).
__device__ __forceinline__ float wave_incl_scan(float v, int lane) {
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    float t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

}  // namespace specv
