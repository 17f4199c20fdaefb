// Single-query multi-head attention of the decoder step on gfx950.
//
// Both attentions of a decoder block are bandwidth work: one query per (sequence, head)
// against n key/value rows that are read exactly once. One workgroup takes one (sequence,
// head[, memory partition]) and streams its rows with 16-byte loads: hd/8 (bf16) or hd/4
// (fp32) lanes share one row, so every wave load covers whole, contiguous rows. Scores go to
// LDS, the softmax is max-subtracted, and values are accumulated in fp32.
//
// Self-attention reads the per-layer ring cache (window = current token + W-1 past entries,
// "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", architecture section).
// Cross-attention reads memory entries 1..t of the layer's group (prefix restriction, same
// section); long prefixes are split over several workgroups whose partial (max, sum, output)
// triples are merged by the last one to finish, so one launch does the whole attention.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace rlt {

template <typename T, int HD>
struct Geo {
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int LPR = HD / VEC;              // lanes per row
  static constexpr int RPW = kWave / LPR;           // rows per wave load
  static constexpr int RPB = RPW * (kThreads / kWave);
  static_assert(LPR >= 1 && LPR <= kWave && HD % VEC == 0, "unsupported head size");
};

// Attention of one query over rows [0, n) of K/V (row stride HD). Leaves the unnormalised
// output sum_j p_j v_j in o_lds[4*HD + i], and returns the running max and sum of p in
// m_out / l_out (p_j = exp(s_j - max)). s_lds holds >= n floats. Every thread participates.
template <typename T, int HD, int U>
__device__ void attend_rows(const float* __restrict__ q, const T* __restrict__ K,
                            const T* __restrict__ V, int n, float scale, float* s_lds,
                            float* red, float* o_lds, float& m_out, float& l_out) {
  using G = Geo<T, HD>;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int sub = lane % G::LPR, r = lane / G::LPR;
  float qv[G::VEC];
#pragma unroll
  for (int i = 0; i < G::VEC; ++i) qv[i] = q[sub * G::VEC + i] * scale;

  float mloc = -INFINITY;
  for (int base = 0; base < n; base += G::RPB * U) {
    u32x4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * G::RPB + wave * G::RPW + r;
      raw[u] = row < n ? ld16(K + (int64_t)row * HD + sub * G::VEC) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[G::VEC];
      unpack(raw[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < G::VEC; ++i) dot += qv[i] * kf[i];
#pragma unroll
      for (int o = G::LPR / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, kWave);
      const int row = base + u * G::RPB + wave * G::RPW + r;
      if (row < n) {
        if (sub == 0) s_lds[row] = dot;
        mloc = fmaxf(mloc, dot);
      }
    }
  }
  const float m = block_max(mloc, red);
  float lsum = 0.f;
  for (int j = tid; j < n; j += kThreads) {
    const float p = __expf(s_lds[j] - m);
    s_lds[j] = p;
    lsum += p;
  }
  const float l = block_sum(lsum, red);

  float acc[G::VEC];
#pragma unroll
  for (int i = 0; i < G::VEC; ++i) acc[i] = 0.f;
  for (int base = 0; base < n; base += G::RPB * U) {
    u32x4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * G::RPB + wave * G::RPW + r;
      raw[u] = row < n ? ld16(V + (int64_t)row * HD + sub * G::VEC) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * G::RPB + wave * G::RPW + r;
      const float p = row < n ? s_lds[row] : 0.f;
      float vf[G::VEC];
      unpack(raw[u], vf);
#pragma unroll
      for (int i = 0; i < G::VEC; ++i) acc[i] += p * vf[i];
    }
  }
  // sum over the row slots of the wave (lanes sharing `sub`), then over the four waves
#pragma unroll
  for (int o = G::LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int i = 0; i < G::VEC; ++i) acc[i] += __shfl_xor(acc[i], o, kWave);
  if (r == 0) {
#pragma unroll
    for (int i = 0; i < G::VEC; ++i) o_lds[wave * HD + sub * G::VEC + i] = acc[i];
  }
  __syncthreads();
  if (tid < HD) o_lds[4 * HD + tid] = (o_lds[tid] + o_lds[HD + tid]) + (o_lds[2 * HD + tid] + o_lds[3 * HD + tid]);
  __syncthreads();
  m_out = m;
  l_out = l;
}

// Self-attention: one workgroup per (sequence, head). The ring slots [0, n_valid) hold the
// window (the current token was written by the QKV projection).
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_self(const float* __restrict__ q,
                                                        const T* __restrict__ ring_k,
                                                        const T* __restrict__ ring_v,
                                                        T* __restrict__ out, int H, int W,
                                                        int n_valid, float scale) {
  __shared__ float s_lds[kMaxWindow];
  __shared__ float red[4];
  __shared__ float o_lds[5 * HD];
  const int bh = blockIdx.x, b = bh / H, hh = bh - b * H, d = H * HD;
  const int64_t off = (int64_t)bh * W * HD;
  float m, l;
  attend_rows<T, HD, 4>(q + (int64_t)b * d + hh * HD, ring_k + off, ring_v + off, n_valid, scale,
                        s_lds, red, o_lds, m, l);
  if (threadIdx.x < HD) out[(int64_t)b * d + hh * HD + threadIdx.x] = to_elem<T>(o_lds[4 * HD + threadIdx.x] / l);
}

// Cross-attention over memory entries [0, t): item = ((b * H + h) * nsplit + split); split
// covers entries [split * chunk, min(t, (split + 1) * chunk)).
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attn_cross(
    const float* __restrict__ qc, const T* __restrict__ mk, const T* __restrict__ mv,
    int64_t cap, T* __restrict__ out, float* __restrict__ part, int* __restrict__ cnt, int H,
    int t, int chunk, int nsplit, float scale) {
  __shared__ float s_lds[kMaxChunk];
  __shared__ float red[4];
  __shared__ float o_lds[5 * HD];
  __shared__ int last;
  const int item = blockIdx.x;
  const int bh = item / nsplit, split = item - bh * nsplit;
  const int b = bh / H, hh = bh - b * H, d = H * HD;
  const int j0 = split * chunk;
  const int n = min(t - j0, chunk);
  const int64_t off = ((int64_t)bh * cap + j0) * HD;
  float m, l;
  attend_rows<T, HD, 4>(qc + (int64_t)b * d + hh * HD, mk + off, mv + off, n, scale, s_lds, red,
                        o_lds, m, l);
  T* o = out + (int64_t)b * d + hh * HD;
  if (nsplit == 1) {
    if (threadIdx.x < HD) o[threadIdx.x] = to_elem<T>(o_lds[4 * HD + threadIdx.x] / l);
    return;
  }
  constexpr int PS = HD + 2;
  float* pb = part + (int64_t)bh * kMaxSplit * PS;
  if (threadIdx.x == 0) {
    pb[split * PS] = m;
    pb[split * PS + 1] = l;
  }
  if (threadIdx.x < HD) pb[split * PS + 2 + threadIdx.x] = o_lds[4 * HD + threadIdx.x];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const int prev = __hip_atomic_fetch_add(cnt + bh, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    last = prev == nsplit - 1;
  }
  __syncthreads();
  if (!last) return;
  __threadfence();
  if (threadIdx.x < HD) {
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, pb[s * PS]);
    float L = 0.f, acc = 0.f;
    for (int s = 0; s < nsplit; ++s) {
      const float w = __expf(pb[s * PS] - M);
      L += w * pb[s * PS + 1];
      acc += w * pb[s * PS + 2 + threadIdx.x];
    }
    o[threadIdx.x] = to_elem<T>(acc / L);
  }
  if (threadIdx.x == 0) cnt[bh] = 0;
}

template <typename T>
static inline T* elem(void* base, int64_t off) {
  return static_cast<T*>(base) + off;
}

template <typename T, int HD>
static hipError_t self_t(const Dims& D, int B, int l, const StateBufs& S, int n_valid,
                         hipStream_t st) {
  const int64_t layer = (int64_t)B * D.H * D.W * HD;
  hipLaunchKernelGGL((k_attn_self<T, HD>), dim3(B * D.H), dim3(kThreads), 0, st, S.q,
                     elem<T>(S.ring_k, l * layer), elem<T>(S.ring_v, l * layer),
                     static_cast<T*>(S.o), D.H, D.W, n_valid, 1.f / sqrtf((float)HD));
  return hipGetLastError();
}

// Partition of t memory entries: enough workgroups to fill the chip (about 2048), at least
// 64 entries each, at most kMaxSplit partitions of at most kMaxChunk entries.
static void cross_split(int64_t t, int bh, int& chunk, int& nsplit) {
  const int want = (int)std::max<int64_t>(1, (2048 + bh - 1) / bh);
  int64_t c = (t + want - 1) / want;
  c = std::max<int64_t>(c, 64);
  c = std::max<int64_t>(c, (t + kMaxSplit - 1) / kMaxSplit);
  c = std::min<int64_t>(c, std::max<int64_t>(t, 1));
  chunk = (int)c;
  nsplit = (int)((t + c - 1) / c);
}

template <typename T, int HD>
static hipError_t cross_t(const Dims& D, int B, int l, const StateBufs& S, const MemBufs& M,
                          int64_t t, hipStream_t st) {
  int chunk, nsplit;
  cross_split(t, B * D.H, chunk, nsplit);
  if (chunk > kMaxChunk || nsplit > kMaxSplit) return hipErrorInvalidValue;
  const int g = D.G == 1 ? 0 : l;
  const int64_t grp = (int64_t)g * B * D.H * M.capacity * HD;
  hipLaunchKernelGGL((k_attn_cross<T, HD>), dim3(B * D.H * nsplit), dim3(kThreads), 0, st, S.qc,
                     elem<T>(M.k, grp), elem<T>(M.v, grp), M.capacity, static_cast<T*>(S.o),
                     S.part, S.cnt, D.H, (int)t, chunk, nsplit, 1.f / sqrtf((float)HD));
  return hipGetLastError();
}

#define RLT_HD_DISPATCH(fn, ...)                                              \
  switch (D.hd) {                                                              \
    case 32: return D.dtype == RLT_BF16 ? fn<bf16, 32>(__VA_ARGS__) : fn<float, 32>(__VA_ARGS__);   \
    case 64: return D.dtype == RLT_BF16 ? fn<bf16, 64>(__VA_ARGS__) : fn<float, 64>(__VA_ARGS__);   \
    case 128: return D.dtype == RLT_BF16 ? fn<bf16, 128>(__VA_ARGS__) : fn<float, 128>(__VA_ARGS__); \
    default: return hipErrorInvalidValue;                                      \
  }

hipError_t attn_self(const Dims& D, int B, int l, const StateBufs& S, int n_valid,
                     hipStream_t st) {
  RLT_HD_DISPATCH(self_t, D, B, l, S, n_valid, st)
}

hipError_t attn_cross(const Dims& D, int B, int l, const StateBufs& S, const MemBufs& M,
                      int64_t t, hipStream_t st) {
  RLT_HD_DISPATCH(cross_t, D, B, l, S, M, t, st)
}

}  // namespace rlt
