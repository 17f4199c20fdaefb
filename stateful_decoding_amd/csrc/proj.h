// Projection building blocks shared by the decoder-step kernels and the backward pass: the
// split-K decoder-step GEMM (k_proj) and the register-tiled token GEMM (k_gemm_tokens), with
// the operand loaders and epilogue scaffolding they are instantiated with.
//
// Every projection is C[M][N] = A[M][K] * W[K][N] with M = batch rows (or batch*tokens), W packed
// output-major (W^T, k contiguous) in MFMA fragment order so that one lane's operand is a single
// 16-byte load for bf16. The operand A is produced on the fly by a loader and the result is
// consumed by an epilogue, so intermediates do not round-trip through HBM.
#pragma once

#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.h"
#include "internal.h"

namespace rlt {

// ---- operand loaders ------------------------------------------------------------------------
// Two-phase interface so that a whole batch of loads is in flight before any of it is used:
//   issue(rt, row, step, lane, r)  raw 16-byte loads of one lane's fragment: row tile rt
//                                  (fragment-ordered operands) or row `row` (row-major ones),
//                                  k-step `step` (k = 32 step + 8 (lane / 16) + [0, 8))
//   issue_shared(step, r)          raw loads shared by every fragment of the k-step (none)
//   make(r, sh)                    the MFMA fragment from the raw data
// rt and row are always valid (callers clamp; rows past M are never stored).
// RMSNorm consumers (kNorm) read hg = h * gamma, written in the working dtype by whichever
// kernel produced h, and scale each output row by 1/rms(h) (a per-row scalar, so it commutes
// with the product); the producer also left the partial sums of h^2 the scale needs.

template <typename T>
struct AFrag {  // A = a [M][K] matrix of T in MFMA fragment order (ksteps = K / 32)
  static constexpr bool kNorm = false;
  static constexpr int kPer = sizeof(T) == 2 ? 1 : 2, kShared = 0;
  const T* a;
  int ksteps;
  int M;
  __device__ void issue(int rt, int, int step, int lane, u32x4* r) const {
    const T* p = a + ((((int64_t)rt * ksteps + step) << 6) + lane) * 8;
    r[0] = ld16(p);
    if constexpr (kPer == 2) r[1] = ld16(p + 4);
  }
  __device__ void issue_shared(int, u32x4*) const {}
  __device__ Frag<T> make(const u32x4* r, const u32x4*) const {
    Frag<T> f;
    f.from_raw(r);
    return f;
  }
};

template <typename T>
struct ATokens {  // A row (b, i) = e[b * e_seq + i], rows of d elements, n tokens per sequence
  static constexpr bool kNorm = false;
  const T* e;
  int64_t e_seq;
  int M, n, d;
  __device__ Frag<T> load(int row, int k, float&) const {
    Frag<T> f;
    if (row < M) {
      const int b = row / n, i = row - b * n;
      f.load(e + ((int64_t)b * e_seq + i) * d + k);
    } else {
      f.zero();
    }
    return f;
  }
};

template <typename T>
struct AGate {  // A = [e_t ; alpha * s] (K = 2d); a 32-wide k-step never straddles d
  static constexpr bool kNorm = false;
  static constexpr int kPer = 2, kShared = 0;
  const T* e;
  int64_t lde;
  const float* s;
  float alpha;
  int M, d;
  __device__ void issue(int, int row, int step, int lane, u32x4* r) const {
    const int k = step * 32 + (lane >> 4) * 8;
    if (k < d) {
      const T* p = e + (int64_t)row * lde + k;
      r[0] = ld16(p);
      r[1] = sizeof(T) == 2 ? r[0] : ld16(p + 4);
    } else {
      const float* p = s + (int64_t)row * d + (k - d);
      r[0] = ld16(p);
      r[1] = ld16(p + 4);
    }
  }
  __device__ void issue_shared(int, u32x4*) const {}
  // the k of this fragment is not known here, so make() is told which half it is in
  __device__ Frag<T> make_half(const u32x4* r, bool first) const {
    Frag<T> f;
    if (first) {
      f.from_raw(r);
    } else {
      float a4[4], b4[4], x[8];
      unpack(r[0], a4);
      unpack(r[1], b4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[i] = alpha * a4[i];
        x[4 + i] = alpha * b4[i];
      }
      f.from_f32(x);
    }
    return f;
  }
};

// ---- epilogues ------------------------------------------------------------------------------
// store() consumes a finished [BM][BN] fp32 tile held in LDS (row stride ld) whose element
// (r, c) is output (r0 + r, c0 + c); thread tid takes elements tid, tid + NT, ... so
// consecutive threads take consecutive columns. prefetch() runs before the main loop and loads
// into registers (Pre) whatever store() will read from global memory, so those loads overlap
// the operand loads instead of adding a round trip at the end.

template <int E>
struct Pre {
  float a[E], b[E], c[E];
};

template <class D>
struct EpiTile {
  template <int NT, int BM, int BN, int E>
  __device__ void prefetch(Pre<E>&, int, int) const {}
  template <int NT, int BM, int BN, int E>
  __device__ void store(float* tile, int ld, int r0, int c0, const Pre<E>&) const {
    for (int i = threadIdx.x; i < BM * BN; i += NT) {
      const int r = i / BN, c = i - r * BN;
      static_cast<const D*>(this)->op(r0 + r, c0 + c, tile[r * ld + c]);
    }
  }
};

// ROWS = false: every row writes ring slot `slot`; ROWS = true: row r writes slot pos[r] % W and
// rows outside `active` keep their ring (ragged steps).
struct EpiStoreF32 : EpiTile<EpiStoreF32> {
  float* out;
  int64_t ld;
  int M;
  __device__ void op(int row, int col, float v) const {
    if (row < M) out[(int64_t)row * ld + col] = v;
  }
};

// Epilogues that produce a new residual stream h also prepare the operand of the next
// RMSNorm: hg = h * gamma_next in the working dtype and fragment order, and the sums of h^2
// over each 32-column chunk of every row (ssq[row][col / 32]); both are skipped when hg is
// NULL (the last block writes s, whose next use is the gate). D::value(row, col, v) stores h
// and returns it.
template <class AL> struct is_gate : std::false_type {};
template <typename T> struct is_gate<AGate<T>> : std::true_type {};

// Loaders whose output tiles skip a leading part of K provide kstart(first output column).
template <class AL, class = void> struct has_kstart : std::false_type {};
template <class AL>
struct has_kstart<AL, std::void_t<decltype(std::declval<const AL&>().kstart(0))>>
    : std::true_type {};

// ---- decoder-step projections: split-K over the waves of a block --------------------------------
//
// A block owns a BM x BN output tile (BM = 16 FM, BN = 16 FN) and NW waves; its K range is cut
// into NW contiguous parts, one per wave. Each wave issues the loads of up to U k-steps before
// any of their MFMAs (a scheduling barrier keeps the batch together); the launcher picks NW so
// that one batch usually covers a wave's whole part, i.e. one memory round trip per block. The
// NW partial tiles are summed in LDS in wave order, so results do not depend on timing, and
// blocks never communicate.
template <typename T, int FM, int FN, int NW, int U, class AL, class EP>
__global__ __launch_bounds__(NW * kWave) void k_proj(int N, int K, const T* __restrict__ Wt,
                                                     AL al, EP ep) {
  constexpr int BM = 16 * FM, BN = 16 * FN, LD = BN + 1, NT = NW * kWave;
  __shared__ float red[NW * BM * LD];
  __shared__ float rinv[BM];
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int r0 = tm * BM, c0 = tn * BN;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  // 1/rms inputs: NT / BM lanes per row load that row's chunk sums now, add them at the end
  constexpr int LPRR = NT / BM, QMAX = 8;
  float sq[QMAX];
  int nq = 0;
  if constexpr (AL::kNorm) {
    const int row = min(r0 + tid / LPRR, al.M - 1), part = tid % LPRR;
    const int q = (al.nchunk + LPRR - 1) / LPRR;
    nq = min(q, QMAX);
    const float* p = al.ssq + (int64_t)row * al.nchunk;
#pragma unroll
    for (int j = 0; j < QMAX; ++j) {
      const int ch = part + j * LPRR;
      sq[j] = j < nq && ch < al.nchunk ? p[ch] : 0.f;
    }
  }
  constexpr int EPT = (BM * BN + NT - 1) / NT;
  Pre<EPT> pre;
  ep.template prefetch<NT, BM, BN>(pre, r0, c0);

  // k-steps (of 32) of this wave, out of the tile's [k0, ksteps)
  const int ksteps = K / 32;
  int k0 = 0;
  if constexpr (has_kstart<AL>::value) k0 = al.kstart(c0);
  const int kn = ksteps - k0;
  const int per_w = (kn + NW - 1) / NW;
  const int kb = k0 + min(kn, wave * per_w), ke = k0 + min(kn, (wave + 1) * per_w);

  const T* bp[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) bp[f] = Wt + ((((int64_t)(c0 / 16 + f) * ksteps) << 6) + lane) * 8;
  int arow[FM], art[FM];
  const int last_rt = (al.M - 1) / 16;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    arow[i] = min(r0 + 16 * i + (lane & 15), al.M - 1);
    art[i] = min(tm * FM + i, last_rt);
  }
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // raw 16-byte loads of one k-step: FM A fragments, the shared part, FN B fragments
  constexpr int NA = AL::kPer, NS = AL::kShared, NB = sizeof(T) == 2 ? 1 : 2;
  constexpr int PS = FM * NA + NS + FN * NB;
  auto issue = [&](int step, u32x4* r) {
#pragma unroll
    for (int i = 0; i < FM; ++i) al.issue(art[i], arow[i], step, lane, r + i * NA);
    al.issue_shared(step, r + FM * NA);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const T* p = bp[j] + step * 512;
      r[FM * NA + NS + j * NB] = ld16(p);
      if constexpr (NB == 2) r[FM * NA + NS + j * NB + 1] = ld16(p + 4);
    }
  };
  auto consume = [&](int step, const u32x4* r) {
    Frag<T> a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      if constexpr (is_gate<AL>::value) a[i] = al.make_half(r + i * NA, step * 32 < al.d);
      else a[i] = al.make(r + i * NA, r + FM * NA);
    }
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j].from_raw(r + FM * NA + NS + j * NB);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_16x16x32(acc[i][j], a[i], b[j]);
  };
  for (int st = kb; st < ke; st += U) {
    const int n = min(U, ke - st);
    u32x4 raw[U][PS];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n) issue(st + u, raw[u]);
    __builtin_amdgcn_sched_barrier(0);  // keep the whole batch of loads ahead of its uses
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (u < n) consume(st + u, raw[u]);
  }

  if constexpr (AL::kNorm) {
    // chunks beyond QMAX per lane (very wide rows) are added here, in the same lane order
    const int row = min(r0 + tid / LPRR, al.M - 1), part = tid % LPRR;
    float v = 0.f;
#pragma unroll
    for (int j = 0; j < QMAX; ++j) v += sq[j];
    for (int ch = part + QMAX * LPRR; ch < al.nchunk; ch += LPRR) v += al.ssq[(int64_t)row * al.nchunk + ch];
#pragma unroll
    for (int o = 1; o < LPRR; o <<= 1) v += __shfl_xor(v, o, kWave);
    if (tid % LPRR == 0) rinv[tid / LPRR] = rsqrtf(v / (float)al.K + al.eps);
  }
  // the wave partials -> LDS, summed into red[0 .. BM*LD) and scaled by 1/rms
  float* mine = red + wave * BM * LD;
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        mine[(16 * i + (lane >> 4) * 4 + e) * LD + 16 * j + (lane & 15)] = acc[i][j][e];
  __syncthreads();
  for (int i = tid; i < BM * BN; i += NT) {
    const int r = i / BN, o = r * LD + (i % BN);
    float v = red[o];
#pragma unroll
    for (int w = 1; w < NW; ++w) v += red[w * BM * LD + o];
    if constexpr (AL::kNorm) v *= rinv[r];
    red[o] = v;
  }
  __syncthreads();
  ep.template store<NT, BM, BN>(red, LD, r0, c0, pre);
}

// ---- memory projection: register tiles, no split ------------------------------------------------
// Many rows (B x tokens): each wave owns FM x FN 16x16 tiles of a WM x WN wave grid and walks
// all of K.
template <typename T, int WM, int WN, int FM, int FN, class AL, class EP>
__global__ __launch_bounds__(kThreads) void k_gemm_tokens(int N, int K, const T* __restrict__ Wt,
                                                   AL al, EP ep) {
  static_assert(WM * WN == kThreads / kWave, "four waves per workgroup");
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = wave / WN, wn = wave - wm * WN;
  const int rw = tm * BM + wm * 16 * FM;
  const int cw = tn * BN + wn * 16 * FN;
  const int kl = (lane >> 4) * 8;
  const int ksteps = K / 32;
  const T* bp[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) bp[f] = Wt + ((((int64_t)(cw / 16 + f) * ksteps) << 6) + lane) * 8;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += 32) {
    Frag<T> a[FM], b[FN];
    float unused = 0.f;
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = al.load(rw + 16 * i + (lane & 15), k0 + kl, unused);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j].load(bp[j] + (k0 / 32) * 512);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_16x16x32(acc[i][j], a[i], b[j]);
  }
  ep.template tile<FM, FN>(acc, rw + (lane >> 4) * 4, cw, lane);
}

// Batched products: product z (blockIdx.y) shifts its operand loader and its epilogue with an
// overload of batch_at found by argument-dependent lookup; this default is for loaders and
// epilogues of single products, where only z = 0 occurs.
template <class X>
__device__ __forceinline__ X batch_at(const X& x, int) {
  return x;
}

// The same product for bf16 with 128 x 128 workgroup tiles staged through LDS: every k-step's
// 8 A fragments (from the loader) and 8 B fragments are fetched once per workgroup, one 16-byte
// load per thread and operand pair, into one of two LDS buffers while the other is multiplied;
// each wave then reads its 4 + 4 fragments from LDS (64 x 64 per wave). The next k-step's loads
// are issued before the current one's MFMAs. Every output element accumulates its k-steps in
// the same order with the same instruction as k_gemm_tokens, so the results are identical.
// blockIdx.y = z selects product z of a batch: W at Wt + z wt_stride, batch_at(al / ep, z).
template <class AL, class EP>
__global__ __launch_bounds__(kThreads) void k_gemm_tokens_lds(int N, int K,
                                                             const bf16* __restrict__ Wt,
                                                             int64_t wt_stride, AL al_, EP ep_) {
  constexpr int FM = 4, FN = 4, BM = 128, BN = 128;
  const int z = blockIdx.y;
  const AL al = batch_at(al_, z);
  const EP ep = batch_at(ep_, z);
  Wt += z * wt_stride;
  __shared__ __attribute__((aligned(16))) u32x4 as[2][8][kWave];
  __shared__ __attribute__((aligned(16))) u32x4 bs[2][8][kWave];
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = wave / 2, wn = wave % 2;
  const int ksteps = K / 32, kl = (lane >> 4) * 8;
  // this thread stages fragments wave and wave + 4 of A (row tiles) and of B (column tiles)
  int arow[2];
  const bf16* bp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    arow[u] = tm * BM + (wave + 4 * u) * 16 + (lane & 15);
    bp[u] = Wt + ((((int64_t)(tn * 8 + wave + 4 * u) * ksteps) << 6) + lane) * 8;
  }
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ra[2], rb[2];
  float unused = 0.f;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    ra[u] = __builtin_bit_cast(u32x4, al.load(arow[u], kl, unused).v);
    rb[u] = ld16(bp[u]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    as[0][wave + 4 * u][lane] = ra[u];
    bs[0][wave + 4 * u][lane] = rb[u];
  }
  __syncthreads();
  for (int s = 0; s < ksteps; ++s) {
    const int cur = s & 1;
    if (s + 1 < ksteps) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        ra[u] = __builtin_bit_cast(u32x4, al.load(arow[u], (s + 1) * 32 + kl, unused).v);
        rb[u] = ld16(bp[u] + (s + 1) * 512);
      }
    }
    Frag<bf16> a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i].from_raw(&as[cur][wm * 4 + i][lane]);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j].from_raw(&bs[cur][wn * 4 + j][lane]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_16x16x32(acc[i][j], a[i], b[j]);
    if (s + 1 < ksteps) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        as[cur ^ 1][wave + 4 * u][lane] = ra[u];
        bs[cur ^ 1][wave + 4 * u][lane] = rb[u];
      }
    }
    __syncthreads();
  }
  ep.template tile<FM, FN>(acc, tm * BM + wm * 64 + (lane >> 4) * 4, tn * BN + wn * 64, lane);
}

// Tile shape of the register-tiled token GEMM: (WM, WN, FM, FN).
struct Shape {
  int wm, wn, fm, fn;
};
constexpr Shape kBig{2, 2, 2, 2};  // 64 x 64

// C = A W over M rows: bf16 products whose N is a multiple of 128 and that still make at least
// 1024 workgroups of 128 x 128 (four per compute unit) take the LDS-staged kernel, the rest the
// register-tiled one with (WM, WN, FM, FN) tiles, which makes four times as many workgroups.
template <typename T, int WM, int WN, int FM, int FN, class AL, class EP>
static hipError_t run_gemm(int M, int N, int K, const void* Wt, const AL& al, const EP& ep,
                           const Exec& st) {
  if (K % 32 != 0 || M <= 0) return hipErrorInvalidValue;
  if constexpr (std::is_same<T, bf16>::value) {
    const int64_t blocks = (int64_t)((M + 127) / 128) * (N / 128);
    if (N % 128 == 0 && blocks >= 1024) {
      if (blocks > INT32_MAX) return hipErrorInvalidValue;
      return launch(k_gemm_tokens_lds<AL, EP>, dim3((unsigned)blocks), dim3(kThreads), st, N, K,
                    static_cast<const bf16*>(Wt), (int64_t)0, al, ep);
    }
  }
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  const int64_t blocks = (int64_t)((M + BM - 1) / BM) * (N / BN);
  if (N % BN != 0 || blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
  return launch(k_gemm_tokens<T, WM, WN, FM, FN, AL, EP>, dim3((unsigned)blocks), dim3(kThreads),
                st, N, K, static_cast<const T*>(Wt), al, ep);
}

// `batch` products of M x N x K in one launch of the LDS-staged kernel (bf16, N a multiple of
// 128): product z reads W at Wt + z wt_stride and batch_at(al / ep, z).
template <class AL, class EP>
static hipError_t run_gemm_batched(int M, int N, int K, int batch, const bf16* Wt,
                                   int64_t wt_stride, const AL& al, const EP& ep, const Exec& st) {
  const int64_t blocks = (int64_t)((M + 127) / 128) * (N / 128);
  if (K % 32 != 0 || M <= 0 || N % 128 != 0 || batch < 1 || batch > 65535 || blocks <= 0 ||
      blocks > INT32_MAX)
    return hipErrorInvalidValue;
  return launch(k_gemm_tokens_lds<AL, EP>, dim3((unsigned)blocks, (unsigned)batch),
                dim3(kThreads), st, N, K, Wt, wt_stride, al, ep);
}

template <typename T, int FM, int FN, int NW, class AL, class EP>
static void launch_proj(int64_t tiles, int N, int K, const T* W, const AL& al, const EP& ep,
                        const Exec& st) {
  constexpr int PS = FM * AL::kPer + AL::kShared + FN * (sizeof(T) == 2 ? 1 : 2);
  constexpr int U = 24 / PS < 1 ? 1 : 24 / PS > 6 ? 6 : 24 / PS;  // <= 96 VGPRs of raw loads
  (void)launch(k_proj<T, FM, FN, NW, U, AL, EP>, dim3((unsigned)tiles), dim3(NW * kWave), st, N,
               K, W, al, ep);
}

// Decoder-step projection with tile FM x FN: enough waves per block that each wave's share of K
// fits one batch of loads, and more waves when there are few tiles.
template <typename T, int FM, int FN, class AL, class EP>
static hipError_t run_proj(int M, int N, int K, const void* Wt, const AL& al, const EP& ep,
                           const Exec& st) {
  constexpr int BM = 16 * FM, BN = 16 * FN;
  constexpr int PS = FM * AL::kPer + AL::kShared + FN * (sizeof(T) == 2 ? 1 : 2);
  constexpr int U = 24 / PS < 1 ? 1 : 24 / PS > 6 ? 6 : 24 / PS;
  if (N % BN != 0 || K % 32 != 0) return hipErrorInvalidValue;
  const int64_t tiles = (int64_t)((M + BM - 1) / BM) * (N / BN);
  if (tiles <= 0 || tiles > INT32_MAX) return hipErrorInvalidValue;
  const int ksteps = K / 32;
  constexpr int kMaxNW = FM * FN <= 2 ? 16 : 8;  // 1024-thread blocks only for the small tile
  int nw = 4;
  while (nw < kMaxNW && (ksteps + nw - 1) / nw > U) nw *= 2;
  // Few tiles: the most waves, so that each compute unit has more loads in flight. Below 128
  // rows the batch runs as one row group and the launch has the chip to itself, so this pays
  // from 256 tiles and 16 k-steps down (one box: long-context batch of 16 7.39 -> 6.96 s per
  // run, 50M-scale batch of 64 273 -> 264 ms); at 128 rows per group the other group's
  // attention shares the compute units, and the same rule cost the 140M-scale run 2.4%.
  const bool few = M < 128 ? tiles < 256 && ksteps >= 16 : tiles < 128 && ksteps >= 32;
  if (few) nw = kMaxNW;
  const T* W = static_cast<const T*>(Wt);
  if (nw == 4) launch_proj<T, FM, FN, 4>(tiles, N, K, W, al, ep, st);
  else if (nw == 8) launch_proj<T, FM, FN, 8>(tiles, N, K, W, al, ep, st);
  else if constexpr (kMaxNW == 16) launch_proj<T, FM, FN, 16>(tiles, N, K, W, al, ep, st);
  return hipGetLastError();
}

// Largest tile that still gives enough blocks to fill the chip.
template <typename T, class AL, class EP>
static hipError_t run_step_gemm(int M, int N, int K, const void* Wt, const AL& al, const EP& ep,
                                const Exec& st) {
  auto blocks = [&](int bm, int bn) { return (int64_t)((M + bm - 1) / bm) * (N / bn); };
  if (N % 64 == 0 && blocks(32, 64) >= 320) return run_proj<T, 2, 4>(M, N, K, Wt, al, ep, st);
  if (blocks(32, 32) >= 320) return run_proj<T, 2, 2>(M, N, K, Wt, al, ep, st);
  return run_proj<T, 1, 2>(M, N, K, Wt, al, ep, st);
}

template <typename T>
static inline T* elem(void* base, int64_t off) {
  return static_cast<T*>(base) + off;
}
template <typename T>
static inline const T* elem(const void* base, int64_t off) {
  return static_cast<const T*>(base) + off;
}

}  // namespace rlt
