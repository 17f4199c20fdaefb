// Support kernels: weight packing, state reset, snapshot export/import, and the decoder-step
// sequencing (one launch per phase, all on the caller's stream).
#include <math.h>

#include <algorithm>

#include "common.h"
#include "internal.h"

namespace rlt {

// ---- weight packing: dst row row(n) = column n of src [K][N], MFMA fragment order ----------
template <typename T>
__global__ __launch_bounds__(kThreads) void k_pack_transpose(const T* __restrict__ src, int K,
                                                             int N, T* __restrict__ dst,
                                                             int64_t row_base, int grp,
                                                             int grp_stride) {
  __shared__ T tile[32][33];
  const int k0 = blockIdx.y * 32, n0 = blockIdx.x * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int k = k0 + r, n = n0 + tx;
    if (k < K && n < N) tile[r][tx] = src[(int64_t)k * N + n];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int n = n0 + r, k = k0 + tx;
    if (k < K && n < N) {
      const int64_t row = row_base + (int64_t)(n / grp) * grp_stride + n % grp;
      dst[frag_off(row, k, K / 32)] = tile[tx][r];
    }
  }
}

hipError_t launch_pack_transpose(int dtype, const void* src, int K, int N, void* dst,
                                 int64_t row_base, int grp, int grp_stride, hipStream_t st) {
  const dim3 grid((N + 31) / 32, (K + 31) / 32);
  if (dtype == RLT_BF16)
    hipLaunchKernelGGL(k_pack_transpose<bf16>, grid, dim3(kThreads), 0, st,
                       static_cast<const bf16*>(src), K, N, static_cast<bf16*>(dst), row_base,
                       grp, grp_stride);
  else
    hipLaunchKernelGGL(k_pack_transpose<float>, grid, dim3(kThreads), 0, st,
                       static_cast<const float*>(src), K, N, static_cast<float*>(dst), row_base,
                       grp, grp_stride);
  return hipGetLastError();
}

// ---- reset: s = s*, positions 0 ----------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void k_reset(float* __restrict__ s,
                                                    const float* __restrict__ s_star, int d,
                                                    int64_t n_s, int64_t* __restrict__ pos,
                                                    int B) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n_s) s[i] = s_star[i % d];
  if (i < B) pos[i] = 0;
}

hipError_t launch_reset(const Dims& D, int B, const Packed& P, const StateBufs& S,
                        hipStream_t st) {
  const int64_t n_s = (int64_t)B * D.d;
  hipLaunchKernelGGL(k_reset, dim3((unsigned)((n_s + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, S.s, P.s_star, D.d, n_s, S.pos, B);
  return hipGetLastError();
}

__global__ __launch_bounds__(kThreads) void k_set_pos(int64_t* __restrict__ pos, int B, int64_t t) {
  const int i = blockIdx.x * kThreads + threadIdx.x;
  if (i < B) pos[i] = t;
}

hipError_t launch_set_positions(int64_t* pos, int B, int64_t t, hipStream_t st) {
  hipLaunchKernelGGL(k_set_pos, dim3((unsigned)((B + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     st, pos, B, t);
  return hipGetLastError();
}

// ---- snapshots: ring [L][B][H][W][hd] <-> canonical [L][B][W-1][d], oldest first ----------
// Row b retains its tokens t-n .. t-1 (0-based), t = pos[b], n = min(t, W-1), token tau in slot
// tau % W; canonical entries beyond n are zero on export.
template <typename T, bool EXPORT>
__global__ __launch_bounds__(kThreads) void k_snapshot(T* __restrict__ ring_k,
                                                       T* __restrict__ ring_v,
                                                       T* __restrict__ can_k,
                                                       T* __restrict__ can_v, int B, int H,
                                                       int hd, int W,
                                                       const int64_t* __restrict__ pos,
                                                       int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int d = H * hd, keep = W - 1;
  const int c = (int)(i % d);
  int64_t rest = i / d;
  const int e = (int)(rest % keep);
  rest /= keep;
  const int b = (int)(rest % B);
  const int l = (int)(rest / B);
  const int hh = c / hd, dd = c % hd;
  const int64_t t = pos[b];
  const int n_valid = (int)(t < keep ? t : keep);
  if (e >= n_valid) {
    if (EXPORT) {
      if (can_k) can_k[i] = to_elem<T>(0.f);
      if (can_v) can_v[i] = to_elem<T>(0.f);
    }
    return;
  }
  const int64_t tau = t - n_valid + e;
  const int64_t r = ((((int64_t)l * B + b) * H + hh) * W + (int)(tau % W)) * hd + dd;
  if (EXPORT) {
    if (can_k) can_k[i] = ring_k[r];
    if (can_v) can_v[i] = ring_v[r];
  } else {
    ring_k[r] = can_k[i];
    ring_v[r] = can_v[i];
  }
}

template <typename T, bool EXPORT>
static hipError_t snapshot_t(const Dims& D, int B, const StateBufs& S, void* k, void* v,
                             hipStream_t st) {
  const int keep = D.W - 1;
  const int64_t total = (int64_t)D.L * B * keep * D.d;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL((k_snapshot<T, EXPORT>), dim3((unsigned)((total + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, st, static_cast<T*>(S.ring_k), static_cast<T*>(S.ring_v),
                     static_cast<T*>(k), static_cast<T*>(v), B, D.H, D.hd, D.W,
                     (const int64_t*)S.pos, total);
  return hipGetLastError();
}

hipError_t launch_export(const Dims& D, int B, const StateBufs& S, float* s, void* k, void* v,
                         hipStream_t st) {
  if (s) {
    hipError_t e = hipMemcpyAsync(s, S.s, sizeof(float) * (size_t)B * D.d,
                                  hipMemcpyDeviceToDevice, st);
    if (e != hipSuccess) return e;
  }
  if (!k && !v) return hipSuccess;
  return D.dtype == RLT_BF16 ? snapshot_t<bf16, true>(D, B, S, k, v, st)
                             : snapshot_t<float, true>(D, B, S, k, v, st);
}

hipError_t launch_import_caches(const Dims& D, int B, const StateBufs& S, const void* k,
                                const void* v, hipStream_t st) {
  return D.dtype == RLT_BF16
             ? snapshot_t<bf16, false>(D, B, S, const_cast<void*>(k), const_cast<void*>(v), st)
             : snapshot_t<float, false>(D, B, S, const_cast<void*>(k), const_cast<void*>(v), st);
}

hipError_t launch_import(const Dims& D, int B, const StateBufs& S, int64_t t, const float* s,
                         const void* k, const void* v, hipStream_t st) {
  hipError_t e = hipMemcpyAsync(S.s, s, sizeof(float) * (size_t)B * D.d, hipMemcpyDeviceToDevice,
                                st);
  if (e != hipSuccess) return e;
  if ((e = launch_set_positions(S.pos, B, t, st)) != hipSuccess) return e;
  return launch_import_caches(D, B, S, k, v, st);
}

// ---- row groups -----------------------------------------------------------------------------
StateBufs state_rows(const Dims& D, const StateBufs& S, int b0) {
  StateBufs v = S;
  const int64_t d = D.d;
  v.s += b0 * d;
  v.h += b0 * d;
  v.q += b0 * d;
  v.qc += b0 * d;
  v.hg = static_cast<char*>(S.hg) + b0 * d * D.es;
  v.ssq += b0 * (d / 32);
  v.o = static_cast<char*>(S.o) + b0 * d * D.es;
  v.act = static_cast<char*>(S.act) + (int64_t)b0 * D.F * D.es;
  v.hb = static_cast<char*>(S.hb) + b0 * d * D.es;
  v.pos += b0;
  v.part += (int64_t)b0 * D.H * kMaxSplits * (D.hd + 2);
  if (S.active) v.active += b0;
  const int64_t ring_row = (int64_t)D.H * D.W * D.hd * D.es;
  v.ring_k = static_cast<char*>(S.ring_k) + b0 * ring_row;
  v.ring_v = static_cast<char*>(S.ring_v) + b0 * ring_row;
  return v;
}

MemBufs memory_rows(const Dims& D, const MemBufs& M, int b0) {
  MemBufs v = M;
  const int64_t row = (int64_t)D.H * M.capacity * D.hd * D.es;
  v.k = static_cast<char*>(M.k) + b0 * row;
  v.v = static_cast<char*>(M.v) + b0 * row;
  return v;
}

// ---- kernel timing ---------------------------------------------------------------------------
// Sets `pairs` clock slot pairs to (max, 0), so that a workgroup that left no stamps shows.
__global__ void k_clock_clear(unsigned long long* __restrict__ p, int64_t pairs) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < pairs;
       i += (int64_t)gridDim.x * blockDim.x) {
    p[2 * i] = ~0ull;
    p[2 * i + 1] = 0ull;
  }
}

hipError_t Profiler::clear_clock(hipStream_t st) const {
  if (!clk_buf || clk_cap <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((clk_cap + 255) / 256, 4096);
  hipLaunchKernelGGL(k_clock_clear, dim3((unsigned)blocks), dim3(256), 0, st, clk_buf, clk_cap);
  return hipGetLastError();
}

hipError_t Profiler::arm(int kind, double bytes, double flops, Exec& x, int64_t grid) {
  if (!on(kind)) return hipSuccess;
  if (clk_buf && grid > 0) {
    if (clk_used + grid > clk_cap) {
      ++clk_dropped;  // reported by rlt_profile_end
      return hipSuccess;
    }
    x.clk = clk_buf + 2 * clk_used;
    recs.push_back(Rec{kind, -1, clk_used, grid, bytes, flops});
    clk_used += grid;
    return hipSuccess;
  }
  while (events.size() < used + 2) {
    hipEvent_t e;
    hipError_t err = hipEventCreate(&e);
    if (err != hipSuccess) return err;
    events.push_back(e);
  }
  x.start = events[used];
  x.stop = events[used + 1];
  recs.push_back(Rec{kind, (int)used, -1, 0, bytes, flops});
  used += 2;
  return hipSuccess;
}

void Profiler::destroy() {
  for (hipEvent_t e : events) (void)hipEventDestroy(e);
  events.clear();
  recs.clear();
  used = 0;
  mask = 0;
}

// ---- one decoder step ------------------------------------------------------------------------
// Algorithmic bytes and flops of each kernel: every operand read once, every result written
// once (weights es bytes per element, fp32 activations 4, dtype activations es).
hipError_t launch_step(const Dims& D, int B, const Packed& P, const StateBufs& S,
                       const MemBufs& M, const void* e_t, int64_t e_ld, int64_t t0, float* out,
                       int64_t out_ld, hipStream_t st, Profiler* prof) {
  hipError_t e;
  const double b = B, d = D.d, F = D.F, es = (double)D.es;
  const double act32 = b * d * 4, actd = b * d * es;
  // `call` launches one kernel on Exec x.
  // the attention kernels (one workgroup per sequence and head, times the parts of a split
  // memory prefix) can time themselves
  const int64_t self_grid = attn_blocks((int64_t)B * D.H);
  const int64_t cross_grid = attn_blocks((int64_t)B * D.H * cross_splits(D, B, t0));
#define RLT_TIMED(kind, bytes, flops, call)                                                 \
  do {                                                                                      \
    Exec x(st);                                                                             \
    const int64_t grid = kind == RLT_K_SELF_ATTN ? self_grid                                \
                         : kind == RLT_K_CROSS_ATTN ? cross_grid : 0;                        \
    if (prof && (e = prof->arm(kind, bytes, flops, x, grid)) != hipSuccess) return e;       \
    if ((e = (call)) != hipSuccess) return e;                                               \
  } while (0)
  RLT_TIMED(RLT_K_GATE, 2 * d * d * es + actd + 2 * act32, 4 * b * d * d,
            gemm_gate(D, B, P, S, e_t, e_ld, x));
  const int n_valid = (int)(t0 + 1 < D.W ? t0 + 1 : D.W);
  const double t = (double)(t0 + 1);
  for (int l = 0; l < D.L; ++l) {
    const bool last = l == D.L - 1;
    RLT_TIMED(RLT_K_QKV, 3 * d * d * es + 2 * act32 + 2 * actd, 6 * b * d * d,
              gemm_qkv(D, B, l, P, S, x));
    RLT_TIMED(RLT_K_SELF_ATTN, n_valid * b * 2 * d * es + act32 + actd, 4 * b * d * n_valid,
              attn_self(D, B, l, S, x));
    // self-attention output fused with the cross-attention query (one launch; the memory
    // attention applies the query's 1/rms)
    RLT_TIMED(RLT_K_SELF_OUT, 3 * d * d * es + 2 * actd + 3 * act32, 2 * b * d * d * 3,
              gemm_self_out_cq(D, B, l, P, S, x));
    RLT_TIMED(RLT_K_CROSS_ATTN, t * b * 2 * d * es + act32 + actd, 4 * b * d * t,
              attn_cross(D, B, l, S, M, x, true));
    RLT_TIMED(RLT_K_CROSS_OUT, d * d * es + actd + 2 * act32, 2 * b * d * d,
              gemm_residual(D, B, l, 1, P, S, false, nullptr, 0, x));
    RLT_TIMED(RLT_K_FFN_UP, 2 * F * d * es + act32 + b * F * es, 4 * b * d * F,
              gemm_w13(D, B, l, P, S, x));
    RLT_TIMED(RLT_K_FFN_DOWN, F * d * es + b * F * es + 2 * act32 + (last && out ? act32 : 0),
              2 * b * d * F,
              gemm_residual(D, B, l, 2, P, S, last, last ? out : nullptr, out_ld, x));
  }
#undef RLT_TIMED
  return hipSuccess;
}

}  // namespace rlt
