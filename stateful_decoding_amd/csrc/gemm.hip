// Batched projections of the decoder step and the memory projection on gfx950 MFMA.
//
// Every projection is C[M][N] = A[M][K] * W[K][N] with M = batch rows (or batch*tokens for
// the memory projection), W packed output-major (W^T, k contiguous) so that one lane's MFMA
// operand is a single 16-byte load for bf16. The operand A is produced on the fly by a
// loader (plain rows, RMSNorm of the fp32 residual stream, or the gate's [e_t ; alpha s]
// concatenation) and the result is consumed by an epilogue (query/key/value scatter into
// the ring cache, residual add, SiLU-gated product, gate merge, memory layout scatter), so
// no intermediate round-trips through HBM.
//
// Tiling: 4 waves per workgroup in a WM x WN grid; each wave owns FM x FN tiles of 16x16 and
// walks K in steps of 32 (v_mfma_f32_16x16x32_bf16; eight v_mfma_f32_16x16x4_f32 for fp32).
#include "common.h"
#include "internal.h"

namespace rlt {

// ---- operand loaders ------------------------------------------------------------------------

template <typename T>
struct ARows {  // A = rows of a [M][lda] matrix of T
  const T* a;
  int64_t lda;
  int M;
  __device__ void prepare(int, int, float*) {}
  __device__ Frag<T> load(int row, int k) const {
    Frag<T> f;
    if (row < M) f.load(a + (int64_t)row * lda + k);
    else f.zero();
    return f;
  }
};

template <typename T>
struct ATokens {  // A row (b, i) = e[b * e_seq + i], rows of d elements, n tokens per sequence
  const T* e;
  int64_t e_seq;
  int M, n, d;
  __device__ void prepare(int, int, float*) {}
  __device__ Frag<T> load(int row, int k) const {
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
struct ANorm {  // A = gamma * h / sqrt(mean(h^2) + eps), h fp32 [M][K]
  const float* h;
  const float* gamma;
  float eps;
  int M, K;
  int row0;
  const float* rinv;
  // Inverse RMS of rows [r0, r0 + nrows) into lds (one wave per row).
  __device__ void prepare(int r0, int nrows, float* lds) {
    const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
    for (int r = wave; r < nrows; r += kThreads / kWave) {
      const int row = r0 + r;
      float ss = 0.f;
      if (row < M) {
        const float* hr = h + (int64_t)row * K;
        for (int k = lane * 4; k < K; k += kWave * 4) {
          float x[4];
          unpack(ld16(hr + k), x);
          ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
        }
      }
      ss = wave_sum(ss);
      if (lane == 0) lds[r] = row < M ? rsqrtf(ss / (float)K + eps) : 0.f;
    }
    __syncthreads();
    row0 = r0;
    rinv = lds;
  }
  __device__ Frag<T> load(int row, int k) const {
    Frag<T> f;
    if (row >= M) {
      f.zero();
      return f;
    }
    const float* hr = h + (int64_t)row * K + k;
    float x[8];
    float a4[4], b4[4];
    unpack(ld16(hr), a4);
    unpack(ld16(hr + 4), b4);
    float ga[4], gb[4];
    unpack(ld16(gamma + k), ga);
    unpack(ld16(gamma + k + 4), gb);
    const float r = rinv[row - row0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a4[i] * r * ga[i];
      x[4 + i] = b4[i] * r * gb[i];
    }
    f.from_f32(x);
    return f;
  }
};

template <typename T>
struct AGate {  // A = [e_t ; alpha * s] (K = 2d)
  const T* e;
  int64_t lde;
  const float* s;
  float alpha;
  int M, d;
  __device__ void prepare(int, int, float*) {}
  __device__ Frag<T> load(int row, int k) const {
    Frag<T> f;
    if (row >= M) {
      f.zero();
    } else if (k < d) {
      f.load(e + (int64_t)row * lde + k);
    } else {
      const float* sr = s + (int64_t)row * d + (k - d);
      float a4[4], b4[4], x[8];
      unpack(ld16(sr), a4);
      unpack(ld16(sr + 4), b4);
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
// A lane holds, for every (fm, fn) tile and i = 0..3, the element at
// row = rbase + 16 fm + i, col = cwave + 16 fn + (lane % 16).

template <class D>
struct EpiElem {
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          static_cast<const D*>(this)->op(rbase + 16 * fm + i, cwave + 16 * fn + (lane & 15),
                                          acc[fm][fn][i]);
  }
};

template <typename T>
struct EpiQKV : EpiElem<EpiQKV<T>> {  // q -> fp32 buffer; k, v -> ring slot
  float* q;
  T* ring_k;
  T* ring_v;
  int M, d, H, hd, W, slot;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    if (col < d) {
      q[(int64_t)row * d + col] = v;
      return;
    }
    int c = col - d;
    T* dst = ring_k;
    if (c >= d) {
      c -= d;
      dst = ring_v;
    }
    const int hh = c / hd, dd = c - hh * hd;
    dst[(((int64_t)row * H + hh) * W + slot) * hd + dd] = to_elem<T>(v);
  }
};

struct EpiStoreF32 : EpiElem<EpiStoreF32> {
  float* out;
  int64_t ld;
  int M;
  __device__ void op(int row, int col, float v) const {
    if (row < M) out[(int64_t)row * ld + col] = v;
  }
};

struct EpiResidual : EpiElem<EpiResidual> {  // dst = h + v; optional copy to out
  const float* h;
  float* dst;
  float* out;
  int64_t out_ld;
  int M, d;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    const int64_t i = (int64_t)row * d + col;
    const float r = h[i] + v;
    dst[i] = r;
    if (out) out[(int64_t)row * out_ld + col] = r;
  }
};

template <typename T>
struct EpiGate : EpiElem<EpiGate<T>> {  // g = sigmoid(v + b); h = g e + (1 - g) alpha s
  float* h;
  const T* e;
  int64_t lde;
  const float* s;
  const float* b;
  float alpha;
  int M, d;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    const float g = sigmoidf_(v + b[col]);
    const float ev = to_f32<T>(e[(int64_t)row * lde + col]);
    const float u = alpha * s[(int64_t)row * d + col];
    h[(int64_t)row * d + col] = g * ev + (1.f - g) * u;
  }
};

template <typename T>
struct EpiSiluMul {  // needs FN even: tile 2j is W1, tile 2j+1 the same columns of W3
  T* act;
  int M, F;
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
    static_assert(FN % 2 == 0, "SiLU-gated epilogue pairs W1 and W3 tiles");
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int p = 0; p < FN / 2; ++p) {
        const int col = (cwave + 32 * p) / 2 + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + 16 * fm + i;
          if (row >= M) continue;
          const float z1 = acc[fm][2 * p][i], z3 = acc[fm][2 * p + 1][i];
          act[(int64_t)row * F + col] = to_elem<T>(z1 * sigmoidf_(z1) * z3);
        }
      }
  }
};

template <typename T>
struct EpiMemproj : EpiElem<EpiMemproj<T>> {  // row = (b, tau), col = (g, k|v, head, dim)
  T* mk;
  T* mv;
  int64_t cap, t0;
  int M, n, B, d, H, hd;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    const int b = row / n, tau = row - b * n;
    const int g = col / (2 * d);
    int c = col - g * 2 * d;
    T* dst = mk;
    if (c >= d) {
      c -= d;
      dst = mv;
    }
    const int hh = c / hd, dd = c - hh * hd;
    dst[((((int64_t)g * B + b) * H + hh) * cap + t0 + tau) * hd + dd] = to_elem<T>(v);
  }
};

// ---- the kernel -----------------------------------------------------------------------------

template <typename T, int WM, int WN, int FM, int FN, class AL, class EP>
__global__ __launch_bounds__(kThreads) void k_gemm(int N, int K, const T* __restrict__ Wt,
                                                   AL al, EP ep) {
  static_assert(WM * WN == kThreads / kWave, "four waves per workgroup");
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  __shared__ float lds[BM];
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  al.prepare(tm * BM, BM, lds);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int wm = wave / WN, wn = wave - wm * WN;
  const int rw = tm * BM + wm * 16 * FM;
  const int cw = tn * BN + wn * 16 * FN;
  const int kl = (lane >> 4) * 8;
  const T* bp[FN];
#pragma unroll
  for (int f = 0; f < FN; ++f) bp[f] = Wt + (int64_t)(cw + 16 * f + (lane & 15)) * K + kl;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < K; k0 += 32) {
    Frag<T> a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = al.load(rw + 16 * i + (lane & 15), k0 + kl);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j].load(bp[j] + k0);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_16x16x32(acc[i][j], a[i], b[j]);
  }
  ep.template tile<FM, FN>(acc, rw + (lane >> 4) * 4, cw, lane);
}

// Tile shapes: (WM, WN, FM, FN).
struct Shape {
  int wm, wn, fm, fn;
  int bm() const { return 16 * fm * wm; }
  int bn() const { return 16 * fn * wn; }
};
constexpr Shape kSmallM{1, 4, 1, 2};  // 16 x 128: batches of up to 16 rows
constexpr Shape kMidM{2, 2, 1, 2};    // 32 x 64
constexpr Shape kBig{2, 2, 2, 2};     // 64 x 64: memory projection

template <typename T, int WM, int WN, int FM, int FN, class AL, class EP>
static hipError_t run_gemm(int M, int N, int K, const void* Wt, const AL& al, const EP& ep,
                           hipStream_t st) {
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  const int64_t blocks = (int64_t)((M + BM - 1) / BM) * (N / BN);
  if (N % BN != 0 || K % 32 != 0 || blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_gemm<T, WM, WN, FM, FN, AL, EP>), dim3((unsigned)blocks), dim3(kThreads),
                     0, st, N, K, static_cast<const T*>(Wt), al, ep);
  return hipGetLastError();
}

// Picks the 16-row shape for small batches when it tiles N, else the 32-row one.
template <typename T, class AL, class EP>
static hipError_t run_step_gemm(int M, int N, int K, const void* Wt, const AL& al, const EP& ep,
                                hipStream_t st) {
  if (M <= 16 && N % kSmallM.bn() == 0)
    return run_gemm<T, kSmallM.wm, kSmallM.wn, kSmallM.fm, kSmallM.fn>(M, N, K, Wt, al, ep, st);
  return run_gemm<T, kMidM.wm, kMidM.wn, kMidM.fm, kMidM.fn>(M, N, K, Wt, al, ep, st);
}

template <typename T>
static inline T* elem(void* base, int64_t off) {
  return static_cast<T*>(base) + off;
}
template <typename T>
static inline const T* elem(const void* base, int64_t off) {
  return static_cast<const T*>(base) + off;
}

// ---- per-use entry points ---------------------------------------------------------------------

template <typename T>
static hipError_t gate_t(const Dims& D, int B, const Packed& P, const StateBufs& S,
                         const void* e_t, int64_t e_ld, hipStream_t st) {
  AGate<T> al{static_cast<const T*>(e_t), e_ld, S.s, D.alpha, B, D.d};
  EpiGate<T> ep;
  ep.h = S.h; ep.e = static_cast<const T*>(e_t); ep.lde = e_ld; ep.s = S.s; ep.b = P.b_gate;
  ep.alpha = D.alpha; ep.M = B; ep.d = D.d;
  return run_step_gemm<T>(B, D.d, 2 * D.d, P.w_gate_t, al, ep, st);
}

template <typename T>
static hipError_t qkv_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                        int slot, hipStream_t st) {
  ANorm<T> al{S.h, P.gamma + (int64_t)l * 3 * D.d, D.eps, B, D.d, 0, nullptr};
  EpiQKV<T> ep;
  const int64_t ring_layer = (int64_t)B * D.H * D.W * D.hd;
  ep.q = S.q; ep.ring_k = elem<T>(S.ring_k, l * ring_layer); ep.ring_v = elem<T>(S.ring_v, l * ring_layer);
  ep.M = B; ep.d = D.d; ep.H = D.H; ep.hd = D.hd; ep.W = D.W; ep.slot = slot;
  return run_step_gemm<T>(B, 3 * D.d, D.d, elem<T>(P.wqkv_t, (int64_t)l * 3 * D.d * D.d), al, ep, st);
}

template <typename T>
static hipError_t cq_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                       hipStream_t st) {
  ANorm<T> al{S.h, P.gamma + (int64_t)l * 3 * D.d + D.d, D.eps, B, D.d, 0, nullptr};
  EpiStoreF32 ep;
  ep.out = S.qc; ep.ld = D.d; ep.M = B;
  return run_step_gemm<T>(B, D.d, D.d, elem<T>(P.wcq_t, (int64_t)l * D.d * D.d), al, ep, st);
}

template <typename T>
static hipError_t w13_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                        hipStream_t st) {
  ANorm<T> al{S.h, P.gamma + (int64_t)l * 3 * D.d + 2 * D.d, D.eps, B, D.d, 0, nullptr};
  EpiSiluMul<T> ep{static_cast<T*>(S.act), B, D.F};
  return run_step_gemm<T>(B, 2 * D.F, D.d, elem<T>(P.w13_t, (int64_t)l * 2 * D.F * D.d), al, ep, st);
}

template <typename T>
static hipError_t residual_t(const Dims& D, int B, int l, int which, const Packed& P,
                             const StateBufs& S, bool dst_s, float* out, int64_t out_ld,
                             hipStream_t st) {
  const void* A = which == 2 ? S.act : S.o;
  const int K = which == 2 ? D.F : D.d;
  const void* Wt = which == 0 ? elem<T>(P.wo_t, (int64_t)l * D.d * D.d)
                 : which == 1 ? elem<T>(P.wco_t, (int64_t)l * D.d * D.d)
                              : elem<T>(P.w2_t, (int64_t)l * D.d * D.F);
  ARows<T> al{static_cast<const T*>(A), K, B};
  EpiResidual ep;
  ep.h = S.h; ep.dst = dst_s ? S.s : S.h; ep.out = out; ep.out_ld = out_ld; ep.M = B; ep.d = D.d;
  return run_step_gemm<T>(B, D.d, K, Wt, al, ep, st);
}

template <typename T>
static hipError_t memproj_t(const Dims& D, int B, const Packed& P, const MemBufs& M,
                            const void* e, int64_t e_seq, int64_t t0, int64_t n, hipStream_t st) {
  const int64_t rows = (int64_t)B * n;
  if (rows > INT32_MAX / 2) return hipErrorInvalidValue;
  ATokens<T> al{static_cast<const T*>(e), e_seq, (int)rows, (int)n, D.d};
  EpiMemproj<T> ep;
  ep.mk = static_cast<T*>(M.k); ep.mv = static_cast<T*>(M.v); ep.cap = M.capacity; ep.t0 = t0;
  ep.M = (int)rows; ep.n = (int)n; ep.B = B; ep.d = D.d; ep.H = D.H; ep.hd = D.hd;
  return run_gemm<T, kBig.wm, kBig.wn, kBig.fm, kBig.fn>((int)rows, D.G * 2 * D.d, D.d, P.wm_t,
                                                        al, ep, st);
}

hipError_t gemm_gate(const Dims& D, int B, const Packed& P, const StateBufs& S, const void* e_t,
                     int64_t e_ld, hipStream_t st) {
  return D.dtype == RLT_BF16 ? gate_t<bf16>(D, B, P, S, e_t, e_ld, st)
                             : gate_t<float>(D, B, P, S, e_t, e_ld, st);
}
hipError_t gemm_qkv(const Dims& D, int B, int l, const Packed& P, const StateBufs& S, int slot,
                    hipStream_t st) {
  return D.dtype == RLT_BF16 ? qkv_t<bf16>(D, B, l, P, S, slot, st)
                             : qkv_t<float>(D, B, l, P, S, slot, st);
}
hipError_t gemm_cq(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                   hipStream_t st) {
  return D.dtype == RLT_BF16 ? cq_t<bf16>(D, B, l, P, S, st) : cq_t<float>(D, B, l, P, S, st);
}
hipError_t gemm_w13(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                    hipStream_t st) {
  return D.dtype == RLT_BF16 ? w13_t<bf16>(D, B, l, P, S, st) : w13_t<float>(D, B, l, P, S, st);
}
hipError_t gemm_residual(const Dims& D, int B, int l, int which, const Packed& P,
                         const StateBufs& S, bool dst_s, float* out, int64_t out_ld,
                         hipStream_t st) {
  return D.dtype == RLT_BF16 ? residual_t<bf16>(D, B, l, which, P, S, dst_s, out, out_ld, st)
                             : residual_t<float>(D, B, l, which, P, S, dst_s, out, out_ld, st);
}
hipError_t launch_memproj(const Dims& D, int B, const Packed& P, const MemBufs& M,
                          const void* e, int64_t e_seq, int64_t t0, int64_t n, hipStream_t st) {
  return D.dtype == RLT_BF16 ? memproj_t<bf16>(D, B, P, M, e, e_seq, t0, n, st)
                             : memproj_t<float>(D, B, P, M, e, e_seq, t0, n, st);
}

}  // namespace rlt
