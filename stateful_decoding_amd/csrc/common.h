// Device-side building blocks shared by the gfx950 kernels: element types, 16-byte vector
// loads, MFMA wrappers and wave/block reductions. Wavefronts are 64 lanes; every kernel in
// this library runs 256-thread (4-wave) workgroups.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rlt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWave = 64;

// Self-timing of a launch (clk != NULL): every workgroup writes the GPU's constant-rate clock
// to its own slot pair, clk[2 blockIdx] when it starts and clk[2 blockIdx + 1] when all its
// waves are done; the host takes the earliest start and the latest end. No two workgroups
// write the same address and nothing is queued around the launch.
struct LaunchClock {
  unsigned long long* clk;
  __device__ __forceinline__ void start() const {
    if (clk && threadIdx.x == 0) clk[2 * blockIdx.x] = wall_clock64();
  }
  __device__ __forceinline__ void stop() const {
    if (clk) {
      __syncthreads();
      if (threadIdx.x == 0) clk[2 * blockIdx.x + 1] = wall_clock64();
    }
  }
};

// Elements of T in one 16-byte vector.
template <typename T> struct Vec16;
template <> struct Vec16<float> { static constexpr int N = 4; };
template <> struct Vec16<bf16> { static constexpr int N = 8; };

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
// The same load with the non-temporal policy, for rows streamed once per launch (the attention
// kernels' keys and values, hundreds of megabytes per token): they then do not push data that is
// reused soon, such as the projections' weights shared by the row groups, out of the caches.
// Measured on the 140M-scale batch of 256: 66 -> 59 us per memory-attention launch and 1.62 ->
// 1.52 s per 1024-token run.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Widen one 16-byte vector of T to float.
__device__ __forceinline__ void unpack(u32x4 raw, float (&out)[8]) {  // bf16 -> float
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(raw[i] << 16);
    out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void unpack(u32x4 raw, float (&out)[4]) {  // float -> float
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(raw[i]);
}

template <typename T> __device__ __forceinline__ T to_elem(float x);
template <> __device__ __forceinline__ float to_elem<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 to_elem<bf16>(float x) { return (bf16)x; }

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<bf16>(bf16 x) { return (float)x; }

// ---- MFMA operand fragments -------------------------------------------------------------
// One lane's share of a 16x32 (rows x k) operand tile: 8 consecutive k values of one row.
// Lane l holds row (l % 16), k = 8 * (l / 16) + [0, 8). The A and B operands use the same
// lane -> k assignment, so every product pairs matching k.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = __builtin_bit_cast(bf16x8, ld16(p)); }
  __device__ __forceinline__ void zero() { v = __builtin_bit_cast(bf16x8, u32x4{0, 0, 0, 0}); }
  __device__ __forceinline__ void from_raw(const u32x4* r) { v = __builtin_bit_cast(bf16x8, r[0]); }
  __device__ __forceinline__ void from_f32(const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = (bf16)x[i];
  }
};
template <> struct Frag<float> {
  float v[8];
  __device__ __forceinline__ void load(const float* p) {
    u32x4 a = ld16(p), b = ld16(p + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.f;
  }
  __device__ __forceinline__ void from_raw(const u32x4* r) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(r[0][i]);
      v[4 + i] = __uint_as_float(r[1][i]);
    }
  }
  __device__ __forceinline__ void from_f32(const float (&x)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[i];
  }
};

// Element offset of (row, k) in a [rows][K] operand stored in MFMA fragment order: for every
// 16-row tile and 32-wide k-step, the 64 lanes' 8 consecutive k values lie contiguously (1 KB
// in bf16), so one wave load of a fragment reads whole cache lines. A row range that starts
// on a multiple of 16 begins at the same offset as in row-major order (row * K).
__host__ __device__ __forceinline__ int64_t frag_off(int64_t row, int k, int ksteps) {
  return ((((row >> 4) * ksteps + (k >> 5)) << 6) + (row & 15) + (((k & 31) >> 3) << 4)) * 8 +
         (k & 7);
}

// acc(16x16, fp32) += A(16x32) * B(32x16). Output layout: lane l holds rows 4*(l/16)+i,
// i = 0..3, of column l % 16.
__device__ __forceinline__ void mfma_16x16x32(f32x4& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}
// fp32 operands: eight 16x16x4 steps; step i multiplies element i of every lane, i.e.
// k = 8*(l/16) + i across the four lane groups, so the eight steps cover all 32 k.
__device__ __forceinline__ void mfma_16x16x32(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[i], b.v[i], acc, 0, 0, 0);
}

// ---- reductions ----------------------------------------------------------------------------
// Lane move within rows of 16 lanes (DPP; ctrl: 0x00-0xff quad permutation, 0x140 mirror of the
// row, 0x141 mirror of each half row).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, true));
}
// Sum over aligned groups of G lanes (G a power of two up to 64): DPP moves inside rows of 16,
// cross-row shuffles beyond. Each step adds a partner that holds the other half-group's sum,
// so every lane of a group ends with the same value.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_move<0xb1>(v);   // quad permutation [1, 0, 3, 2]
  if constexpr (G >= 4) v += dpp_move<0x4e>(v);   // quad permutation [2, 3, 0, 1]
  if constexpr (G >= 8) v += dpp_move<0x141>(v);  // lane i <-> 7 - i within 8
  if constexpr (G >= 16) v += dpp_move<0x140>(v); // lane i <-> 15 - i within 16
  if constexpr (G >= 32) v += __shfl_xor(v, 16, 64);
  if constexpr (G >= 64) v += __shfl_xor(v, 32, 64);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
// Block-wide reductions over 256 threads; `red` is 4 floats of LDS. Every thread gets the
// result. Contains two barriers.
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  float r = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) red[w] = v;
  __syncthreads();
  float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  return r;
}

// 1 / (1 + e^-x) with the hardware reciprocal (about 1 ulp; an IEEE division costs about ten
// vector instructions more); e^-x = inf gives 0, e^-x = 0 gives 1
__device__ __forceinline__ float sigmoidf_(float x) {
  return __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

}  // namespace rlt
