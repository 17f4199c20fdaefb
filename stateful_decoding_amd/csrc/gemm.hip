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
#include <algorithm>
#include <type_traits>

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
template <typename T, class D>
struct EpiH {
  T* hg;
  const float* gamma;
  float* ssq;
  int nchunk;
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
        sq = v * v;
      }
      tile[r * ld + c] = sq;
    }
    self.finish(r0, c0, BM);
    if (!hg) return;
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

template <typename T>
struct EpiSiluMul {  // packed columns come in blocks of 32: 16 of W1, then the same 16 of W3;
                     // act is written in fragment order (the down projection's operand)
  T* act;
  int M, F;
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

template <class AL> struct is_gate : std::false_type {};
template <typename T> struct is_gate<AGate<T>> : std::true_type {};

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

  // k-steps (of 32) of this wave
  const int ksteps = K / 32;
  const int per_w = (ksteps + NW - 1) / NW;
  const int kb = min(ksteps, wave * per_w), ke = min(ksteps, (wave + 1) * per_w);

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

// Tile shape of the memory projection: (WM, WN, FM, FN).
struct Shape {
  int wm, wn, fm, fn;
};
constexpr Shape kBig{2, 2, 2, 2};  // 64 x 64

template <typename T, int WM, int WN, int FM, int FN, class AL, class EP>
static hipError_t run_gemm(int M, int N, int K, const void* Wt, const AL& al, const EP& ep,
                           const Exec& st) {
  constexpr int BM = 16 * FM * WM, BN = 16 * FN * WN;
  const int64_t blocks = (int64_t)((M + BM - 1) / BM) * (N / BN);
  if (N % BN != 0 || K % 32 != 0 || blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
  return launch(k_gemm_tokens<T, WM, WN, FM, FN, AL, EP>, dim3((unsigned)blocks), dim3(kThreads),
                st, N, K, static_cast<const T*>(Wt), al, ep);
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
  if (tiles < 128 && ksteps >= 32) nw = kMaxNW;
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
                        const Exec& st) {
  EpiSiluMul<T> ep{static_cast<T*>(S.act), B, D.F};
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
  return run_step_gemm<T>(B, D.d, K, Wt, al, ep, st);
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
                    const Exec& st) {
  return D.dtype == RLT_BF16 ? w13_t<bf16>(D, B, l, P, S, st) : w13_t<float>(D, B, l, P, S, st);
}
hipError_t gemm_residual(const Dims& D, int B, int l, int which, const Packed& P,
                         const StateBufs& S, bool dst_s, float* out, int64_t out_ld,
                         const Exec& st) {
  return D.dtype == RLT_BF16 ? residual_t<bf16>(D, B, l, which, P, S, dst_s, out, out_ld, st)
                             : residual_t<float>(D, B, l, which, P, S, dst_s, out, out_ld, st);
}
hipError_t launch_memproj(const Dims& D, int B, const Packed& P, const MemBufs& M,
                          const void* e, int64_t e_seq, int64_t t0, int64_t n, const Exec& st) {
  return D.dtype == RLT_BF16 ? memproj_t<bf16>(D, B, P, M, e, e_seq, t0, n, st)
                             : memproj_t<float>(D, B, P, M, e, e_seq, t0, n, st);
}

}  // namespace rlt
