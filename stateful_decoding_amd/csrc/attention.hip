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

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace rlt {

// Rows per lane slot loaded per batch, and the largest grid of an attention launch (0: one
// workgroup per item).
#ifndef RLT_ATTN_U
#define RLT_ATTN_U 6
#endif
#ifndef RLT_ATTN_CAP
#define RLT_ATTN_CAP 0
#endif
#ifndef RLT_SPLIT_LIMIT
#define RLT_SPLIT_LIMIT kMaxSplits
#endif
constexpr int kAttnU = RLT_ATTN_U;
constexpr int64_t kAttnCap = RLT_ATTN_CAP;
constexpr int kSplitLimit = RLT_SPLIT_LIMIT;

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

// One batch of U rows per row slot: scores, one rescale of the running state to the batch's
// max, then the weighted values. Rows past n (score -inf) contribute nothing.
template <typename T, int HD, int U>
__device__ __forceinline__ void step_batch(const u32x4* kr, const u32x4* vr, int base, int RPB,
                                           int first, int n, const float* qv, float& m,
                                           float& l, float* acc) {
  using G = Geo<T, HD>;
  float sc[U];
  float mb = m;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float kf[G::VEC];
    unpack(kr[u], kf);
    float dot = 0.f;
#pragma unroll
    for (int i = 0; i < G::VEC; ++i) dot += qv[i] * kf[i];
    dot = group_sum<G::LPR>(dot);
    const bool ok = base + u * RPB + first < n;
    sc[u] = ok ? dot : -INFINITY;
    mb = fmaxf(mb, sc[u]);
  }
  if (mb == -INFINITY) return;  // this slot had no rows in the batch
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

// NW waves per (sequence, head, part): softmax attention of one query over the rows of a
// contiguous [rows][HD] key block and value block, in a single pass. The sequence attends rows
// [0, n), n from its own position, so sequences of one batch may be at different tokens; with
// `parts` > 1 (gridDim.x = sequences x heads x parts) workgroup p takes the p-th of `parts`
// contiguous slices of those rows. Each row slot (LPR lanes) walks its rows with a running
// softmax state, U rows at a time with one rescale per batch; slots merge through lane
// shuffles, waves through LDS. The query is q[b] (fp32, head hh), K/V blocks start at
// K + bh * bh_stride. One part: the output row o[b] (dtype) is written in MFMA fragment order,
// as the output projection reads it. Several parts: the unnormalised output, the max and the
// sum of the slice go to part[(bh * parts + p) * (HD + 2)] (an empty slice leaves max -inf,
// sum 0) for k_attend_merge.
// qssq != NULL: q[b] is unnormalised and is scaled by 1/sqrt(sum(qssq[b]) / d + eps), the
// 1/rms of the residual stream whose 32-column sums of squares qssq[b] holds.
template <typename T, int HD, int NW, int U, bool NTL = true>
__device__ __forceinline__ void attend(const float* __restrict__ q, const T* __restrict__ K,
                                       const T* __restrict__ V, int64_t bh_stride,
                                       const int64_t* __restrict__ pos, int64_t t_uniform,
                                       int window, int H, float scale, T* __restrict__ out,
                                       int parts, float* __restrict__ part,
                                       const float* __restrict__ qssq, float eps, int item) {
  using G = Geo<T, HD>;
  constexpr int RPB = G::RPW * NW;  // rows per block per batch step
  __shared__ float lds_m[NW], lds_l[NW];
  __shared__ float lds_acc[NW][HD];
  const int bh = item / parts, pi = item - bh * parts;
  const int b = bh / H, hh = bh - b * H, d = H * HD;
  // rows attended: the memory prefix 1..t+1 of this sequence, or its window of
  // min(t + 1, W) ring slots (t = tokens the sequence has processed before this step)
  const int64_t tb = (t_uniform >= 0 ? t_uniform : pos[b]) + 1;
  const int nb = window > 0 ? (int)(tb < window ? tb : window) : (int)tb;
  const int chunk = (nb + parts - 1) / parts;
  const int lo = min(nb, pi * chunk), n = min(nb, lo + chunk) - lo;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int sub = lane % G::LPR, slot = lane / G::LPR;
  const T* Kb = K + (int64_t)bh * bh_stride + (int64_t)lo * HD + sub * G::VEC;
  const T* Vb = V + (int64_t)bh * bh_stride + (int64_t)lo * HD + sub * G::VEC;
  float qv[G::VEC];
  const float* qp = q + (int64_t)b * d + hh * HD + sub * G::VEC;
  float qs = scale;
  if (qssq) {
    const int nch = d / 32;  // <= 512 chunks
    float ss = 0.f;
    for (int c = lane; c < nch; c += kWave) ss += qssq[(int64_t)b * nch + c];
    qs *= rsqrtf(wave_sum(ss) / (float)d + eps);
  }
#pragma unroll
  for (int i = 0; i < G::VEC; ++i) qv[i] = qp[i] * qs;

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
      if constexpr (NTL) {
        kr[u] = ok ? ld16_stream(Kb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
        vr[u] = ok ? ld16_stream(Vb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
      } else {
        kr[u] = ok ? ld16(Kb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
        vr[u] = ok ? ld16(Vb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
      }
    }
    step_batch<T, HD, U>(kr, vr, base, RPB, first, n, qv, m, l, acc);
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
    if (parts == 1) {
      out[frag_off(b, hh * HD + tid, d / 32)] = to_elem<T>(A / L);
    } else {
      float* pp = part + (int64_t)item * (HD + 2);
      pp[tid] = A;
      if (tid == 0) {
        pp[HD] = M;
        pp[HD + 1] = L;
      }
    }
  }
}

// Merge of the `parts` partial softmax states of each (sequence, head) in part order; thread
// (bh, j) writes output element j of head hh of row b in fragment order.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_attend_merge(const float* __restrict__ part,
                                                            int parts, int BH, int H,
                                                            T* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)BH * HD) return;
  const int bh = (int)(i / HD), j = (int)(i - (int64_t)bh * HD);
  const int b = bh / H, hh = bh - b * H;
  const float* pp = part + (int64_t)bh * parts * (HD + 2);
  float M = -INFINITY, L = 0.f, A = 0.f;
  for (int p = 0; p < parts; ++p, pp += HD + 2)
    merge_state(M, L, &A, pp[HD], pp[HD + 1], pp + j, 1);
  out[frag_off(b, hh * HD + j, H * HD / 32)] = to_elem<T>(A / L);
}

// The two uses get kernels of their own, so that traces tell them apart. clk != NULL: a timed
// launch (LaunchClock).
// Workgroup g takes the items g, g + gridDim.x, ... of the items = sequences x heads x parts
// (one each unless the launch caps its grid).
template <typename T, int HD, int NW, int U, bool NTL>
__device__ __forceinline__ void attend_timed(const float* q, const T* K, const T* V,
                                             int64_t bh_stride, const int64_t* pos,
                                             int64_t t_uniform, int window, int H, float scale,
                                             T* out, int parts, float* part, const float* qssq,
                                             float eps, int items, unsigned long long* clk) {
  const LaunchClock lc{clk};
  lc.start();
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    attend<T, HD, NW, U, NTL>(q, K, V, bh_stride, pos, t_uniform, window, H, scale, out, parts,
                              part, qssq, eps, item);
    if (item + (int)gridDim.x < items) __syncthreads();  // LDS is reused by the next item
  }
  lc.stop();
}
template <typename T, int HD, int NW, int U>
__global__ __launch_bounds__(NW * kWave) void k_attend_window(
    const float* q, const T* K, const T* V, int64_t bh_stride, const int64_t* pos,
    int64_t t_uniform, int window, int H, float scale, T* out, int parts, float* part,
    const float* qssq, float eps, int items, unsigned long long* clk) {
  attend_timed<T, HD, NW, U, true>(q, K, V, bh_stride, pos, t_uniform, window, H, scale, out,
                                   parts, part, qssq, eps, items, clk);
}
template <typename T, int HD, int NW, int U, bool NTL>
__global__ __launch_bounds__(NW * kWave) void k_attend_memory(
    const float* q, const T* K, const T* V, int64_t bh_stride, const int64_t* pos,
    int64_t t_uniform, int window, int H, float scale, T* out, int parts, float* part,
    const float* qssq, float eps, int items, unsigned long long* clk) {
  attend_timed<T, HD, NW, U, NTL>(q, K, V, bh_stride, pos, t_uniform, window, H, scale, out,
                                  parts, part, qssq, eps, items, clk);
}

template <typename T>
static inline T* elem(void* base, int64_t off) {
  return static_cast<T*>(base) + off;
}

// Waves per workgroup: enough workgroups x waves to keep the chip streaming. With parts > 1
// the slices' partial states are merged by a second launch (untimed: the clock stamps, when
// attached, time the streaming launch).
template <typename T, int HD, bool MEMORY>
static hipError_t attend_t(int BH, const float* q, const T* K, const T* V, int64_t bh_stride,
                           const int64_t* pos, int64_t t_uniform, int window, int H, T* out,
                           int parts, float* part, const float* qssq, float eps,
                           const Exec& st, bool stream = true) {
  const float scale = 1.f / sqrtf((float)HD);
  const int64_t items = (int64_t)BH * parts;
  if (parts < 1 || parts > kMaxSplits || items > INT32_MAX) return hipErrorInvalidValue;
  const int64_t blocks = attn_blocks(items);
  // Waves per workgroup from the number of items (sequence-head pairs x parts): few waves per
  // workgroup stream best once there are many workgroups. One box, against the earlier 4 / 8 /
  // 16 waves from 1024 / 512 / fewer items: 50M-scale batch of 64 (512 pairs) 263.5 -> 255.3 ms
  // per run and 48-layer batch of 32 (512 pairs) 5.24 -> 5.04 s over its first 1024 tokens with
  // 4 waves (16 waves: 317.7 ms, 5.54 s); long-context batch of 16 (192 pairs) 6.96 -> 6.71 s
  // with 8 waves (4 waves: 7.31 s).
  const int nw = items >= 512 ? 4 : items >= 128 ? 8 : 16;
  hipError_t e = hipSuccess;
#define RLT_ATTEND(NW)                                                                     \
  e = launch(!MEMORY ? k_attend_window<T, HD, NW, kAttnU>                                  \
             : stream ? k_attend_memory<T, HD, NW, kAttnU, true>                           \
                      : k_attend_memory<T, HD, NW, kAttnU, false>,                         \
             dim3((unsigned)blocks), dim3(NW * kWave), st, q, K, V, bh_stride, pos, t_uniform, \
             window, H, scale, out, parts, part, qssq, eps, (int)items, st.clk)
  if (nw == 4) RLT_ATTEND(4);
  else if (nw == 8) RLT_ATTEND(8);
  else RLT_ATTEND(16);
#undef RLT_ATTEND
  if (e != hipSuccess || parts == 1) return e;
  const int64_t threads = (int64_t)BH * HD;
  return launch(k_attend_merge<T, HD>, dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                dim3(kThreads), Exec(st.st), (const float*)part, parts, BH, H, out);
}

bool memory_streams(const Dims& D, int Bt, int64_t t_max) {
  // Layers that share one memory (G = 1) read the same prefix once per layer and token: while
  // the whole batch's prefix fits in half of the 256 MB memory-side cache, ordinary loads let
  // the later layers find it there. Otherwise (a memory per layer, or a longer prefix) each
  // row is read once before hundreds of megabytes of others, and non-temporal loads keep the
  // projections' weights cached instead. Measured: the 50M-scale batch of 64 (128 MiB of
  // memory at 1024 tokens) 281 -> 273 ms per run; the long-context batch of 16 (403 MB)
  // 7.61 s with ordinary loads throughout against 7.38 s non-temporal.
  const double bytes = (double)Bt * (double)(t_max + 1) * 2.0 * D.d * (double)D.es;
  return !(D.G == 1 && bytes <= (double)(128 << 20));
}

int64_t attn_blocks(int64_t items) {
  return kAttnCap > 0 && items > kAttnCap ? kAttnCap : items;
}

int cross_splits(const Dims& D, int B, int64_t t_max) {
  // Only batches with fewer sequence-head pairs than half the compute units are split: from 128
  // pairs up, 16-wave workgroups already stream the prefix at 5.7-5.9 TB/s (long-context and
  // 48-layer workloads), and the merge launch would only lengthen the chain of dependent
  // launches. Below that, about 256 workgroups in all, and at least 256 entries per slice.
  const int64_t bh = (int64_t)B * D.H, n = t_max + 1;
  if (bh >= 128) return 1;
  int64_t parts = (256 + bh - 1) / bh;
  parts = std::min<int64_t>(parts, n / 256);
  return (int)std::max<int64_t>(1, std::min<int64_t>(parts, kSplitLimit));
}

template <typename T, int HD>
static hipError_t self_t(const Dims& D, int B, int l, const StateBufs& S, const Exec& st) {
  const int64_t layer = (int64_t)S.Bt * D.H * D.W * HD;
  return attend_t<T, HD, false>(B * D.H, S.q, elem<T>(S.ring_k, l * layer),
                                elem<T>(S.ring_v, l * layer), (int64_t)D.W * HD, S.pos,
                                S.t_uniform, D.W, D.H, static_cast<T*>(S.o), 1, nullptr,
                                nullptr, 0.f, st);
}

template <typename T, int HD>
static hipError_t cross_t(const Dims& D, int B, int l, const StateBufs& S, const MemBufs& M,
                          const Exec& st, bool q_unnormalised) {
  const int g = D.G == 1 ? 0 : l;
  const int64_t grp = (int64_t)g * M.Bt * D.H * M.capacity * HD;
  return attend_t<T, HD, true>(B * D.H, S.qc, elem<T>(M.k, grp), elem<T>(M.v, grp),
                               M.capacity * HD, S.pos, S.t_uniform, 0, D.H,
                               static_cast<T*>(S.o), cross_splits(D, B, S.t_max), S.part,
                               q_unnormalised ? S.ssq : nullptr, D.eps, st,
                               memory_streams(D, M.Bt, S.t_max));
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
                      const Exec& st, bool q_unnormalised) {
  RLT_HD_DISPATCH(cross_t, D, B, l, S, M, st, q_unnormalised)
}

}  // namespace rlt
