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
#include "proj.h"

namespace rlt {

template <typename T>
struct ANormed {  // A = hg = h * gamma (dtype, fragment order); rows scaled by 1/rms(h) later
  static constexpr bool kNorm = true;
  static constexpr int kPer = sizeof(T) == 2 ? 1 : 2, kShared = 0;
  const T* hg;
  const float* ssq;  // [M][nchunk] partial sums of h^2 over 32-column chunks
  int nchunk;
  float eps;
  int M, K;
  __device__ void issue(int rt, int, int step, int lane, u32x4* r) const {
    const T* p = hg + ((((int64_t)rt * (K / 32) + step) << 6) + lane) * 8;
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

// A = [hb | o] (K = 2d): h and the self-attention output, both [M][d] in fragment order. Tiles
// of the first d outputs (the residual h1 = h + o W_o) start at k = d and read only o.
template <typename T>
struct AFused {
  static constexpr bool kNorm = false;
  static constexpr int kPer = sizeof(T) == 2 ? 1 : 2, kShared = 0;
  const T* hb;
  const T* o;
  int dsteps;  // d / 32
  int M, d;
  __device__ int kstart(int c0) const { return c0 < d ? dsteps : 0; }
  __device__ void issue(int rt, int, int step, int lane, u32x4* r) const {
    const bool first = step < dsteps;
    const T* p = (first ? hb : o) +
                 ((((int64_t)rt * dsteps + (first ? step : step - dsteps)) << 6) + lane) * 8;
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

template <typename T, bool ROWS>
struct EpiQKV : EpiTile<EpiQKV<T, ROWS>> {  // q -> fp32 buffer; k, v -> the row's ring slot
  float* q;
  T* ring_k;
  T* ring_v;
  const int64_t* pos;
  const uint8_t* active;  // NULL: every row
  int M, d, H, hd, W, slot;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    if (col < d) {
      q[(int64_t)row * d + col] = v;
      return;
    }
    int sl = slot;
    if constexpr (ROWS) {
      if (active && !active[row]) return;
      sl = (int)pos[row] % W;  // positions stay below the memory capacity (2^20)
    }
    int c = col - d;
    T* dst = ring_k;
    if (c >= d) {
      c -= d;
      dst = ring_v;
    }
    const int hh = c / hd, dd = c - hh * hd;
    dst[(((int64_t)row * H + hh) * W + sl) * hd + dd] = to_elem<T>(v);
  }
};

template <typename T, class D>
struct EpiH {
  T* hg;
  const float* gamma;
  float* ssq;
  int nchunk;
  T* hb = nullptr;        // also h itself in the working dtype (fragment order), when set
  bool ssq_only = false;  // chunk sums of h^2 without hg (the scale of an unnormalised query)
  template <int NT, int BM, int BN, int E>
  __device__ void prefetch(Pre<E>& pre, int r0, int c0) const {
    const D& self = static_cast<const D&>(*this);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = threadIdx.x + j * NT;
      if (i >= BM * BN) break;
      const int r = i / BN, c = i - r * BN;
      const int row = min(r0 + r, self.M - 1), col = c0 + c;
      self.load_inputs(row, col, pre.a[j], pre.b[j]);
      pre.c[j] = hg ? gamma[col] : 0.f;
    }
  }
  template <int NT, int BM, int BN, int E>
  __device__ void store(float* tile, int ld, int r0, int c0, const Pre<E>& pre) const {
    const D& self = static_cast<const D&>(*this);
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const int i = threadIdx.x + j * NT;
      if (i >= BM * BN) break;
      const int r = i / BN, c = i - r * BN;
      const int row = r0 + r, col = c0 + c;
      float sq = 0.f;
      if (row < self.M) {
        const float v = self.value(row, col, tile[r * ld + c], pre.a[j], pre.b[j]);
        if (hg) hg[frag_off(row, col, nchunk)] = to_elem<T>(v * pre.c[j]);
        if (hb) hb[frag_off(row, col, nchunk)] = to_elem<T>(v);
        sq = v * v;
      }
      tile[r * ld + c] = sq;
    }
    self.finish(r0, c0, BM);
    if (!hg && !ssq_only) return;
    __syncthreads();
    constexpr int nch = BN / 32;
    for (int j = threadIdx.x; j < BM * nch; j += NT) {
      const int r = j / nch, ch = j - r * nch;
      if (r0 + r >= self.M) continue;
      const float* t = tile + r * ld + ch * 32;
      float v = 0.f;
      for (int c = 0; c < 32; ++c) v += t[c];
      ssq[(int64_t)(r0 + r) * nchunk + c0 / 32 + ch] = v;
    }
  }
};

// dst = h + v; optional copy to out. FINAL: the last launch of a step (dst = s): rows outside
// `active` keep s (and copy it to out), and the positions of the other rows advance.
template <typename T, bool FINAL>
struct EpiResidual : EpiH<T, EpiResidual<T, FINAL>> {
  const float* h;
  float* dst;
  float* out;
  int64_t out_ld;
  const uint8_t* active;  // FINAL only; NULL: every row
  int64_t* pos;           // FINAL only
  int M, d;
  __device__ bool kept(int row) const {
    if constexpr (FINAL) return active && !active[row];
    return false;
  }
  __device__ void load_inputs(int row, int col, float& a, float& b) const {
    a = h[(int64_t)row * d + col];
    b = kept(row) ? dst[(int64_t)row * d + col] : 0.f;
  }
  __device__ float value(int row, int col, float v, float hv, float old) const {
    if (kept(row)) {
      if (out) out[(int64_t)row * out_ld + col] = old;
      return old;
    }
    const float r = hv + v;
    dst[(int64_t)row * d + col] = r;
    if (out) out[(int64_t)row * out_ld + col] = r;
    return r;
  }
  // once per row: the column-0 tile advances the position
  __device__ void finish(int r0, int c0, int BM) const {
    if constexpr (FINAL) {
      if (c0 != 0) return;
      const int row = r0 + (int)threadIdx.x;
      if ((int)threadIdx.x < BM && row < M && !kept(row)) pos[row] += 1;
    }
  }
};

template <typename T>
struct EpiGate : EpiH<T, EpiGate<T>> {  // g = sigmoid(v + b); h = g e + (1 - g) alpha s
  float* h;
  const T* e;
  int64_t lde;
  const float* s;
  const float* b;
  float alpha;
  int M, d;
  __device__ void load_inputs(int row, int col, float& ev, float& sv) const {
    ev = to_f32<T>(e[(int64_t)row * lde + col]);
    sv = s[(int64_t)row * d + col];
  }
  __device__ void finish(int, int, int) const {}
  __device__ float value(int row, int col, float v, float ev, float sv) const {
    const float g = sigmoidf_(v + b[col]);
    const float r = g * ev + (1.f - g) * (alpha * sv);
    h[(int64_t)row * d + col] = r;
    return r;
  }
};

// Outputs 0..d-1: the residual h1 = h + v (EpiResidual, with the chunk sums of h1^2);
// outputs d..2d-1: the unnormalised cross query, stored as fp32 rows of qc. Tiles never straddle
// d (BN divides d), so each workgroup takes one branch.
template <typename T>
struct EpiFusedOQ {
  EpiResidual<T, false> res;
  float* qc;
  int M, d;
  template <int NT, int BM, int BN, int E>
  __device__ void prefetch(Pre<E>& pre, int r0, int c0) const {
    if (c0 < d) res.template prefetch<NT, BM, BN>(pre, r0, c0);
  }
  template <int NT, int BM, int BN, int E>
  __device__ void store(float* tile, int ld, int r0, int c0, const Pre<E>& pre) const {
    if (c0 < d) {
      res.template store<NT, BM, BN>(tile, ld, r0, c0, pre);
      return;
    }
    for (int i = threadIdx.x; i < BM * BN; i += NT) {
      const int r = i / BN, c = i - r * BN;
      if (r0 + r < M) qc[(int64_t)(r0 + r) * d + (c0 - d) + c] = tile[r * ld + c];
    }
  }
};

// C[i][j] = (W_o diag(g1) W_cq)[i][j] into the fused matrix: output row d + j, k = d + i.
template <typename T>
struct EpiPackProduct {
  T* dst;
  int d;
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = rbase + 16 * fm + e, j = cwave + 16 * fn + (lane & 15);
          if (i < d) dst[frag_off(d + j, d + i, 2 * d / 32)] = to_elem<T>(acc[fm][fn][e]);
        }
  }
};

template <typename T>
struct EpiSiluMul {  // packed columns come in blocks of 32: 16 of W1, then the same 16 of W3;
                     // act is written in fragment order (the down projection's operand)
  T* act;
  int M, F;
  float* u = nullptr;  // optional fp32 [M][2F] copy of x W1 | x W3 (kept for the backward pass)
  template <int NT, int BM, int BN, int E>
  __device__ void prefetch(Pre<E>&, int, int) const {}
  template <int NT, int BM, int BN, int E>
  __device__ void store(float* tile, int ld, int r0, int c0, const Pre<E>&) const {
    constexpr int half = BN / 2;
    for (int i = threadIdx.x; i < BM * half; i += NT) {
      const int r = i / half, j = i - r * half;
      const int row = r0 + r;
      if (row >= M) continue;
      const int cp = (j / 16) * 32 + (j % 16);
      const float z1 = tile[r * ld + cp], z3 = tile[r * ld + cp + 16];
      act[frag_off(row, c0 / 2 + j, F / 32)] = to_elem<T>(z1 * sigmoidf_(z1) * z3);
      if (u) {
        u[(int64_t)row * 2 * F + c0 / 2 + j] = z1;
        u[(int64_t)row * 2 * F + F + c0 / 2 + j] = z3;
      }
    }
  }
};

template <typename T>
struct EpiMemproj {  // row = (b, tau), col = (g, k|v, head, dim); register-tile interface
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
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) op(rbase + 16 * fm + i, cwave + 16 * fn + (lane & 15), acc[fm][fn][i]);
  }
};

// ---- per-use entry points ---------------------------------------------------------------------

// Operand hg and chunk sums of the next RMSNorm, with gains `gamma` (NULL: none follows).
template <typename T, class E>
static void next_norm(E& ep, const Dims& D, const StateBufs& S, const float* gamma) {
  ep.hg = gamma ? static_cast<T*>(S.hg) : nullptr;
  ep.gamma = gamma;
  ep.ssq = S.ssq;
  ep.nchunk = D.d / 32;
}

template <typename T>
static ANormed<T> normed(const Dims& D, int B, const StateBufs& S) {
  return ANormed<T>{static_cast<const T*>(S.hg), S.ssq, D.d / 32, D.eps, B, D.d};
}

template <typename T>
static hipError_t gate_t(const Dims& D, int B, const Packed& P, const StateBufs& S,
                         const void* e_t, int64_t e_ld, const Exec& st) {
  AGate<T> al{static_cast<const T*>(e_t), e_ld, S.s, D.alpha, B, D.d};
  EpiGate<T> ep;
  ep.h = S.h; ep.e = static_cast<const T*>(e_t); ep.lde = e_ld; ep.s = S.s; ep.b = P.b_gate;
  ep.alpha = D.alpha; ep.M = B; ep.d = D.d;
  next_norm<T>(ep, D, S, P.gamma);  // layer 0, before self-attention
  ep.hb = static_cast<T*>(S.hb);     // and layer 0's fused output + cross-query projection
  return run_step_gemm<T>(B, D.d, 2 * D.d, P.w_gate_t, al, ep, st);
}

template <typename T, bool ROWS>
static hipError_t qkv_rows_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                             const Exec& st) {
  EpiQKV<T, ROWS> ep;
  const int64_t ring_layer = (int64_t)S.Bt * D.H * D.W * D.hd;
  ep.q = S.q; ep.ring_k = elem<T>(S.ring_k, l * ring_layer); ep.ring_v = elem<T>(S.ring_v, l * ring_layer);
  ep.pos = S.pos; ep.active = S.active;
  ep.M = B; ep.d = D.d; ep.H = D.H; ep.hd = D.hd; ep.W = D.W;
  ep.slot = S.t_uniform >= 0 ? (int)(S.t_uniform % D.W) : -1;
  return run_step_gemm<T>(B, 3 * D.d, D.d, elem<T>(P.wqkv_t, (int64_t)l * 3 * D.d * D.d),
                          normed<T>(D, B, S), ep, st);
}

// every row at the same position and all of them active: one ring slot for the launch
template <typename T>
static hipError_t qkv_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                        const Exec& st) {
  if (S.t_uniform >= 0 && !S.active) return qkv_rows_t<T, false>(D, B, l, P, S, st);
  return qkv_rows_t<T, true>(D, B, l, P, S, st);
}

template <typename T>
static hipError_t cq_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                       const Exec& st) {
  EpiStoreF32 ep;
  ep.out = S.qc; ep.ld = D.d; ep.M = B;
  return run_step_gemm<T>(B, D.d, D.d, elem<T>(P.wcq_t, (int64_t)l * D.d * D.d),
                          normed<T>(D, B, S), ep, st);
}

template <typename T>
static hipError_t w13_t(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                        const Exec& st, float* u_save) {
  EpiSiluMul<T> ep{static_cast<T*>(S.act), B, D.F, u_save};
  return run_step_gemm<T>(B, 2 * D.F, D.d, elem<T>(P.w13_t, (int64_t)l * 2 * D.F * D.d),
                          normed<T>(D, B, S), ep, st);
}

// h (+)= A W for the output projections; the result feeds the next RMSNorm: after the
// self-attention output the cross-attention norm of layer l, after the cross-attention output
// the FFN norm, after the FFN the next layer's first norm (none after the last layer).
template <typename T, bool FINAL>
static hipError_t residual_kind_t(const Dims& D, int B, int l, int which, const Packed& P,
                                  const StateBufs& S, float* out, int64_t out_ld,
                                  const Exec& st) {
  const void* A = which == 2 ? S.act : S.o;
  const int K = which == 2 ? D.F : D.d;
  const void* Wt = which == 0 ? elem<T>(P.wo_t, (int64_t)l * D.d * D.d)
                 : which == 1 ? elem<T>(P.wco_t, (int64_t)l * D.d * D.d)
                              : elem<T>(P.w2_t, (int64_t)l * D.d * D.F);
  AFrag<T> al{static_cast<const T*>(A), K / 32, B};
  EpiResidual<T, FINAL> ep;
  ep.h = S.h; ep.dst = FINAL ? S.s : S.h; ep.out = out; ep.out_ld = out_ld; ep.M = B; ep.d = D.d;
  ep.active = FINAL ? S.active : nullptr;
  ep.pos = FINAL ? S.pos : nullptr;
  const float* g = which < 2 ? P.gamma + ((int64_t)l * 3 + which + 1) * D.d
                 : l + 1 < D.L ? P.gamma + (int64_t)(l + 1) * 3 * D.d : nullptr;
  next_norm<T>(ep, D, S, FINAL ? nullptr : g);
  if (which == 2 && !FINAL) ep.hb = static_cast<T*>(S.hb);  // next layer's fused projection
  return run_step_gemm<T>(B, D.d, K, Wt, al, ep, st);
}

template <typename T>
static hipError_t self_out_cq_t(const Dims& D, int B, int l, const Packed& P,
                                const StateBufs& S, const Exec& st) {
  AFused<T> al{static_cast<const T*>(S.hb), static_cast<const T*>(S.o), D.d / 32, B, D.d};
  EpiFusedOQ<T> ep;
  ep.res.h = S.h; ep.res.dst = S.h; ep.res.out = nullptr; ep.res.out_ld = 0; ep.res.M = B;
  ep.res.d = D.d; ep.res.active = nullptr; ep.res.pos = nullptr;
  next_norm<T>(ep.res, D, S, nullptr);
  ep.res.ssq_only = true;  // the memory attention scales the query by 1/rms(h1)
  ep.qc = S.qc; ep.M = B; ep.d = D.d;
  return run_step_gemm<T>(B, 2 * D.d, 2 * D.d, elem<T>(P.wocq_t, (int64_t)l * 4 * D.d * D.d), al,
                          ep, st);
}

// Fused-matrix construction (once per model): (diag(g1) W_cq)^T and W_o^T into their blocks.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_fuse_blocks(const T* __restrict__ wo,
                                                          const T* __restrict__ wcq,
                                                          const float* __restrict__ g1, int d,
                                                          T* __restrict__ dst,
                                                          T* __restrict__ tmp) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)d * d) return;
  const int k = (int)(i / d), j = (int)(i - (int64_t)k * d);  // input k, output j
  const int ks2 = 2 * d / 32;
  const T v = to_elem<T>(g1[k] * to_f32<T>(wcq[i]));
  dst[frag_off(d + j, k, ks2)] = v;
  tmp[frag_off(j, k, d / 32)] = v;
  dst[frag_off(j, d + k, ks2)] = wo[i];
}

template <typename T>
static hipError_t pack_fused_t(const Dims& D, const Packed& P, const void* wo, const void* wcq,
                               const float* gamma, void* tmp, hipStream_t st) {
  const int d = D.d;
  const int64_t dd = (int64_t)d * d;
  hipError_t e = hipMemsetAsync(P.wocq_t, 0, (size_t)D.L * 4 * dd * sizeof(T), st);
  for (int l = 0; l < D.L && e == hipSuccess; ++l) {
    const T* wo_l = static_cast<const T*>(wo) + l * dd;
    T* dst = elem<T>(P.wocq_t, (int64_t)l * 4 * dd);
    e = launch(k_fuse_blocks<T>, dim3((unsigned)((dd + kThreads - 1) / kThreads)), dim3(kThreads),
               Exec(st), wo_l, static_cast<const T*>(wcq) + l * dd,
               gamma + ((int64_t)l * 3 + 1) * d, d, dst, static_cast<T*>(tmp));
    if (e != hipSuccess) break;
    // W_o diag(g1) W_cq: rows of W_o (row-major) times the scaled W_cq^T just packed in tmp
    ATokens<T> al{wo_l, 0, d, d, d};
    EpiPackProduct<T> ep{dst, d};
    e = run_gemm<T, kBig.wm, kBig.wn, kBig.fm, kBig.fn>(d, d, d, tmp, al, ep, Exec(st));
  }
  return e;
}

// h (+)= A W for the output projections; the result feeds the next RMSNorm: after the
// self-attention output the cross-attention norm of layer l, after the cross-attention output
// the FFN norm, after the FFN the next layer's first norm (none after the last layer).
template <typename T>
static hipError_t residual_t(const Dims& D, int B, int l, int which, const Packed& P,
                             const StateBufs& S, bool dst_s, float* out, int64_t out_ld,
                             const Exec& st) {
  if (dst_s) return residual_kind_t<T, true>(D, B, l, which, P, S, out, out_ld, st);
  return residual_kind_t<T, false>(D, B, l, which, P, S, out, out_ld, st);
}

template <typename T>
static hipError_t memproj_t(const Dims& D, int B, const Packed& P, const MemBufs& M,
                            const void* e, int64_t e_seq, int64_t t0, int64_t n, const Exec& st) {
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
                     int64_t e_ld, const Exec& st) {
  return D.dtype == RLT_BF16 ? gate_t<bf16>(D, B, P, S, e_t, e_ld, st)
                             : gate_t<float>(D, B, P, S, e_t, e_ld, st);
}
hipError_t gemm_qkv(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                    const Exec& st) {
  return D.dtype == RLT_BF16 ? qkv_t<bf16>(D, B, l, P, S, st) : qkv_t<float>(D, B, l, P, S, st);
}
hipError_t gemm_cq(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                   const Exec& st) {
  return D.dtype == RLT_BF16 ? cq_t<bf16>(D, B, l, P, S, st) : cq_t<float>(D, B, l, P, S, st);
}
hipError_t gemm_w13(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                    const Exec& st, float* u_save) {
  return D.dtype == RLT_BF16 ? w13_t<bf16>(D, B, l, P, S, st, u_save)
                             : w13_t<float>(D, B, l, P, S, st, u_save);
}
hipError_t gemm_residual(const Dims& D, int B, int l, int which, const Packed& P,
                         const StateBufs& S, bool dst_s, float* out, int64_t out_ld,
                         const Exec& st) {
  return D.dtype == RLT_BF16 ? residual_t<bf16>(D, B, l, which, P, S, dst_s, out, out_ld, st)
                             : residual_t<float>(D, B, l, which, P, S, dst_s, out, out_ld, st);
}
// ---- readout: logits = RMSNorm(s; out_gamma) W_out ----------------------------------------------
// The norm is split as in the decoder step: one thread per (row, 32-column chunk) writes
// hg = s * gamma (dtype, fragment order) and the chunk's sum of s^2; the projection's loader
// scales each output row by 1/rms. Rows B .. B16-1 of hg are zero.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_readout_prep(const float* __restrict__ s,
                                                           const float* __restrict__ gamma,
                                                           int B, int B16, int d,
                                                           T* __restrict__ hg,
                                                           float* __restrict__ ssq) {
  const int nch = d / 32;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= (int64_t)B16 * nch) return;
  const int row = (int)(i / nch), ch = (int)(i - (int64_t)row * nch);
  float sum = 0.f;
  for (int c = ch * 32; c < ch * 32 + 32; ++c) {
    const float v = row < B ? s[(int64_t)row * d + c] : 0.f;
    hg[frag_off(row, c, nch)] = to_elem<T>(v * gamma[c]);
    sum += v * v;
  }
  if (row < B) ssq[(int64_t)row * nch + ch] = sum;
}

template <typename T>
static hipError_t readout_t(const Dims& D, int B, const HeadBufs& Hd, const float* s, void* hg,
                            float* ssq, float* logits, hipStream_t st) {
  const int B16 = (B + 15) / 16 * 16, nch = D.d / 32;
  const int64_t threads = (int64_t)B16 * nch;
  hipError_t e = launch(k_readout_prep<T>, dim3((unsigned)((threads + kThreads - 1) / kThreads)),
                        dim3(kThreads), Exec(st), s, (const float*)Hd.out_gamma, B, B16, D.d,
                        static_cast<T*>(hg), ssq);
  if (e != hipSuccess) return e;
  EpiStoreF32 ep;
  ep.out = logits; ep.ld = Hd.vocab; ep.M = B;
  return run_step_gemm<T>(B, Hd.vocab, D.d, Hd.w_out_t,
                          ANormed<T>{static_cast<const T*>(hg), ssq, nch, D.eps, B, D.d}, ep,
                          Exec(st));
}

hipError_t launch_readout_logits(const Dims& D, int B, const HeadBufs& Hd, const float* s,
                                 void* hg, float* ssq, float* logits, hipStream_t st) {
  // bf16 vocabularies that tile by 256 columns go through the large-row GEMM (many columns, so
  // MFMA-shaped rather than weight-streaming); the rest through the split-K projection
  if (D.dtype == RLT_BF16 && Hd.vocab % 256 == 0)
    return launch_readout_rows(D, B, Hd, s, hg, logits, st);
  return D.dtype == RLT_BF16 ? readout_t<bf16>(D, B, Hd, s, hg, ssq, logits, st)
                             : readout_t<float>(D, B, Hd, s, hg, ssq, logits, st);
}

hipError_t gemm_self_out_cq(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                            const Exec& st) {
  return D.dtype == RLT_BF16 ? self_out_cq_t<bf16>(D, B, l, P, S, st)
                             : self_out_cq_t<float>(D, B, l, P, S, st);
}

hipError_t launch_pack_fused_ocq(const Dims& D, const Packed& P, const void* wo, const void* wcq,
                                 const float* gamma, void* tmp, hipStream_t st) {
  return D.dtype == RLT_BF16 ? pack_fused_t<bf16>(D, P, wo, wcq, gamma, tmp, st)
                             : pack_fused_t<float>(D, P, wo, wcq, gamma, tmp, st);
}

hipError_t launch_memproj(const Dims& D, int B, const Packed& P, const MemBufs& M,
                          const void* e, int64_t e_seq, int64_t t0, int64_t n, const Exec& st) {
  // many bf16 tokens: the 256 x 256 GEMM, once it has a workgroup for every compute unit
  if (D.dtype == RLT_BF16 && (D.G * 2 * D.d) % 256 == 0 &&
      ((int64_t)B * n + 255) / 256 * (D.G * 2 * D.d / 256) >= 256)
    return launch_memproj_rows(D, B, P, M, e, e_seq, t0, n, st);
  return D.dtype == RLT_BF16 ? memproj_t<bf16>(D, B, P, M, e, e_seq, t0, n, st)
                             : memproj_t<float>(D, B, P, M, e, e_seq, t0, n, st);
}

}  // namespace rlt
