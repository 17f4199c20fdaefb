// Single-query multi-head attention of the decoder step on gfx950.
//
// Both attentions of a decoder block are bandwidth work: one query per (sequence, head)
// against n key/value rows that are read exactly once. One workgroup takes one (sequence,
// head) and streams its key and value rows together with 16-byte loads: hd/8 (bf16) or
// hd/4 (fp32) lanes share one row, so every wave load covers whole, contiguous rows. The
// softmax is computed online in fp32 (running max, sum and output per row slot), so there is
// no score buffer and no limit on n; partial states meet in registers and LDS, never in
// global memory, so workgroups never wait on each other.
//
// Self-attention reads the per-layer ring cache (window = current token + W-1 past entries,
// "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", architecture section).
// Cross-attention reads memory entries 1..t of the layer's group (prefix restriction, same
// section).
#include <math.h>

#include "common.h"
#include "internal.h"

namespace rlt {

template <typename T, int HD>
struct Geo {
  static constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte load
  static constexpr int LPR = HD / VEC;              // lanes per row
  static constexpr int RPW = kWave / LPR;           // row slots per wave
  static_assert(LPR >= 1 && LPR <= kWave && HD % VEC == 0, "unsupported head size");
};

// Running softmax state of one row slot: max m, sum l of exp(s - m), acc = sum exp(s - m) v.
// Merging two states rescales both to the larger max; an empty state has m = -inf, l = 0.
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float mo, float lo,
                                            const float* acco, int n) {
  const float mn = fmaxf(m, mo);
  const float a = m == -INFINITY ? 0.f : __expf(m - mn);
  const float b = mo == -INFINITY ? 0.f : __expf(mo - mn);
  l = l * a + lo * b;
  for (int i = 0; i < n; ++i) acc[i] = acc[i] * a + acco[i] * b;
  m = mn;
}

// One workgroup of NW waves per (sequence, head): softmax attention of one query over the
// rows [0, n) of a contiguous [rows][HD] key block and value block, in a single pass; n comes
// from the sequence's own position, so sequences of one batch may be at different tokens. Each row
// slot (LPR lanes) walks its rows with a running softmax state, U rows at a time with one
// rescale per batch; slots merge through lane shuffles, waves through LDS. The query is q[b]
// (fp32, head hh), K/V blocks start at K + bh * bh_stride; the output row o[b] (dtype) is
// written in MFMA fragment order, as the output projection reads it.
template <typename T, int HD, int NW, int U>
__device__ __forceinline__ void attend(const float* __restrict__ q, const T* __restrict__ K,
                                       const T* __restrict__ V, int64_t bh_stride,
                                       const int64_t* __restrict__ pos, int64_t t_uniform,
                                       int window, int H, float scale, T* __restrict__ out) {
  using G = Geo<T, HD>;
  constexpr int RPB = G::RPW * NW;  // rows per block per batch step
  __shared__ float lds_m[NW], lds_l[NW];
  __shared__ float lds_acc[NW][HD];
  const int bh = blockIdx.x, b = bh / H, hh = bh - b * H, d = H * HD;
  // rows attended: the memory prefix 1..t+1 of this sequence, or its window of
  // min(t + 1, W) ring slots (t = tokens the sequence has processed before this step)
  const int64_t tb = (t_uniform >= 0 ? t_uniform : pos[b]) + 1;
  const int n = window > 0 ? (int)(tb < window ? tb : window) : (int)tb;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int sub = lane % G::LPR, slot = lane / G::LPR;
  const T* Kb = K + (int64_t)bh * bh_stride + sub * G::VEC;
  const T* Vb = V + (int64_t)bh * bh_stride + sub * G::VEC;
  float qv[G::VEC];
  const float* qp = q + (int64_t)b * d + hh * HD + sub * G::VEC;
#pragma unroll
  for (int i = 0; i < G::VEC; ++i) qv[i] = qp[i] * scale;

  float m = -INFINITY, l = 0.f, acc[G::VEC];
#pragma unroll
  for (int i = 0; i < G::VEC; ++i) acc[i] = 0.f;
  const int first = wave * G::RPW + slot;
  for (int base = 0; base < n; base += RPB * U) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * RPB + first;
      const bool ok = row < n;
      kr[u] = ok ? ld16(Kb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
      vr[u] = ok ? ld16(Vb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
    }
    float sc[U];
    float mb = m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[G::VEC];
      unpack(kr[u], kf);
      float dot = 0.f;
#pragma unroll
      for (int i = 0; i < G::VEC; ++i) dot += qv[i] * kf[i];
#pragma unroll
      for (int o = G::LPR / 2; o >= 1; o >>= 1) dot += __shfl_xor(dot, o, kWave);
      const bool ok = base + u * RPB + first < n;
      sc[u] = ok ? dot : -INFINITY;
      mb = fmaxf(mb, sc[u]);
    }
    if (mb == -INFINITY) continue;  // this slot had no rows in the batch
    const float c = m == -INFINITY ? 0.f : __expf(m - mb);
    l *= c;
#pragma unroll
    for (int i = 0; i < G::VEC; ++i) acc[i] *= c;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float p = sc[u] == -INFINITY ? 0.f : __expf(sc[u] - mb);
      float vf[G::VEC];
      unpack(vr[u], vf);
      l += p;
#pragma unroll
      for (int i = 0; i < G::VEC; ++i) acc[i] += p * vf[i];
    }
    m = mb;
  }
  // merge the row slots of the wave (lanes sharing `sub`)
#pragma unroll
  for (int o = G::LPR; o < kWave; o <<= 1) {
    const float mo = __shfl_xor(m, o, kWave), lo = __shfl_xor(l, o, kWave);
    float ao[G::VEC];
#pragma unroll
    for (int i = 0; i < G::VEC; ++i) ao[i] = __shfl_xor(acc[i], o, kWave);
    merge_state(m, l, acc, mo, lo, ao, G::VEC);
  }
  if (slot == 0) {
    if (sub == 0) {
      lds_m[wave] = m;
      lds_l[wave] = l;
    }
#pragma unroll
    for (int i = 0; i < G::VEC; ++i) lds_acc[wave][sub * G::VEC + i] = acc[i];
  }
  __syncthreads();
  if (tid < HD) {
    float M = lds_m[0], L = lds_l[0], A = lds_acc[0][tid];
    for (int w = 1; w < NW; ++w) merge_state(M, L, &A, lds_m[w], lds_l[w], &lds_acc[w][tid], 1);
    out[frag_off(b, hh * HD + tid, d / 32)] = to_elem<T>(A / L);
  }
}

// The two uses get kernels of their own, so that traces tell them apart. clk != NULL: a timed
// launch (LaunchClock).
template <typename T, int HD, int NW, int U>
__device__ __forceinline__ void attend_timed(const float* q, const T* K, const T* V,
                                             int64_t bh_stride, const int64_t* pos,
                                             int64_t t_uniform, int window, int H, float scale,
                                             T* out, unsigned long long* clk) {
  const LaunchClock lc{clk};
  lc.start();
  attend<T, HD, NW, U>(q, K, V, bh_stride, pos, t_uniform, window, H, scale, out);
  lc.stop();
}
template <typename T, int HD, int NW, int U>
__global__ __launch_bounds__(NW * kWave) void k_attend_window(
    const float* q, const T* K, const T* V, int64_t bh_stride, const int64_t* pos,
    int64_t t_uniform, int window, int H, float scale, T* out, unsigned long long* clk) {
  attend_timed<T, HD, NW, U>(q, K, V, bh_stride, pos, t_uniform, window, H, scale, out, clk);
}
template <typename T, int HD, int NW, int U>
__global__ __launch_bounds__(NW * kWave) void k_attend_memory(
    const float* q, const T* K, const T* V, int64_t bh_stride, const int64_t* pos,
    int64_t t_uniform, int window, int H, float scale, T* out, unsigned long long* clk) {
  attend_timed<T, HD, NW, U>(q, K, V, bh_stride, pos, t_uniform, window, H, scale, out, clk);
}

template <typename T>
static inline T* elem(void* base, int64_t off) {
  return static_cast<T*>(base) + off;
}

// Waves per workgroup: enough workgroups x waves to keep the chip streaming.
template <typename T, int HD, bool MEMORY>
static hipError_t attend_t(int BH, const float* q, const T* K, const T* V, int64_t bh_stride,
                           const int64_t* pos, int64_t t_uniform, int window, int H, T* out,
                           const Exec& st) {
  const float scale = 1.f / sqrtf((float)HD);
  const int nw = BH >= 1024 ? 4 : BH >= 512 ? 8 : 16;
#define RLT_ATTEND(NW)                                                                     \
  return launch(MEMORY ? k_attend_memory<T, HD, NW, 4> : k_attend_window<T, HD, NW, 4>,   \
                dim3(BH), dim3(NW * kWave), st, q, K, V, bh_stride, pos, t_uniform, window, \
                H, scale, out, st.clk)
  if (nw == 4) RLT_ATTEND(4);
  if (nw == 8) RLT_ATTEND(8);
  RLT_ATTEND(16);
#undef RLT_ATTEND
}

template <typename T, int HD>
static hipError_t self_t(const Dims& D, int B, int l, const StateBufs& S, const Exec& st) {
  const int64_t layer = (int64_t)S.Bt * D.H * D.W * HD;
  return attend_t<T, HD, false>(B * D.H, S.q, elem<T>(S.ring_k, l * layer),
                                elem<T>(S.ring_v, l * layer), (int64_t)D.W * HD, S.pos, S.t_uniform, D.W, D.H,
                                static_cast<T*>(S.o), st);
}

template <typename T, int HD>
static hipError_t cross_t(const Dims& D, int B, int l, const StateBufs& S, const MemBufs& M,
                          const Exec& st) {
  const int g = D.G == 1 ? 0 : l;
  const int64_t grp = (int64_t)g * M.Bt * D.H * M.capacity * HD;
  return attend_t<T, HD, true>(B * D.H, S.qc, elem<T>(M.k, grp), elem<T>(M.v, grp),
                               M.capacity * HD, S.pos, S.t_uniform, 0, D.H,
                               static_cast<T*>(S.o), st);
}

#define RLT_HD_DISPATCH(fn, ...)                                              \
  switch (D.hd) {                                                              \
    case 32: return D.dtype == RLT_BF16 ? fn<bf16, 32>(__VA_ARGS__) : fn<float, 32>(__VA_ARGS__);   \
    case 64: return D.dtype == RLT_BF16 ? fn<bf16, 64>(__VA_ARGS__) : fn<float, 64>(__VA_ARGS__);   \
    case 128: return D.dtype == RLT_BF16 ? fn<bf16, 128>(__VA_ARGS__) : fn<float, 128>(__VA_ARGS__); \
    default: return hipErrorInvalidValue;                                      \
  }

hipError_t attn_self(const Dims& D, int B, int l, const StateBufs& S, const Exec& st) {
  RLT_HD_DISPATCH(self_t, D, B, l, S, st)
}

hipError_t attn_cross(const Dims& D, int B, int l, const StateBufs& S, const MemBufs& M,
                      const Exec& st) {
  RLT_HD_DISPATCH(cross_t, D, B, l, S, M, st)
}

}  // namespace rlt
