// Token-parallel decoder pass for feedback scale alpha = 0, on gfx950 MFMA.
//
// With alpha = 0 the gated merge no longer reads s_{t-1}: h_t = sigmoid(e_t W_g[:d] + b_g) * e_t.
// Tokens of a sequence are then coupled only through causal attention - the per-layer window
// of the W-1 previous tokens and the memory prefix 1..t - so every decoder layer can process all
// n tokens of all B sequences at once, the way the feedback-off control of the independent
// evaluation was trained ("RLT Runs 96 Blocks Per Token With Recurrent State, No Resets",
// "Three design principles and their caveats": a parallel pass is not equivalent to the
// recurrence in general; the evaluation narrative of "16 per-token recurrence, no quality gain":
// the feedback-off variant trained at 66.0K against 8.4K tokens/s). The result equals n
// recurrent steps up to rounding, and the state is left exactly as those steps leave it.
//
// Per layer: RMSNorm rows -> QKV GEMM (scatter q, k, v per head) -> window flash attention ->
// O GEMM (+ residual) -> RMSNorm -> cross-Q GEMM -> memory flash attention -> cross-O GEMM (+)
// -> RMSNorm -> up GEMM (SiLU product) -> down GEMM (+). All GEMM rows are (sequence, token)
// pairs, so they are large MFMA contractions rather than weight-streaming ones. bf16 only.
#include <math.h>

#include <type_traits>

#include "common.h"
#include "internal.h"

namespace rlt {

// ---- GEMM over all rows: C[R][N] = A[R][K] W[K][N], register tiles ------------------------------
// Workgroup = 4 waves in a 2 x 2 grid, each wave FM x FN fragments of 16 x 16, so a block covers
// (32 FM) x (32 FN). A and W are read in MFMA fragment order; the next k-step's fragments are
// loaded while the current one is multiplied.

struct PA {  // A = bf16 [R16][K] in fragment order
  const bf16* a;
  int ksteps, R;
  __device__ u32x4 load(int row, int step, int lane) const {
    const int rt = min(row, R - 1) >> 4;
    return ld16(a + ((((int64_t)rt * ksteps + step) << 6) + lane) * 8);
  }
};

struct PTokens {  // A row (b, i) = e[b * e_seq + i] (row-major bf16, d per row), n tokens
  const bf16* e;
  int64_t e_seq;
  int n, d, R;
  __device__ u32x4 load(int row, int step, int lane) const {
    row = min(row, R - 1);
    const int b = row / n, i = row - b * n;
    return ld16(e + ((int64_t)b * e_seq + i) * d + step * 32 + (lane >> 4) * 8);
  }
};

template <int FM, int FN, class AL, class EP>
__global__ __launch_bounds__(kThreads) void k_gemm_rows(int N, int ksteps, int wks,
                                                      const bf16* __restrict__ Wt, AL al, EP ep) {
  constexpr int BM = 32 * FM, BN = 32 * FN;
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int rw = tm * BM + (wave / 2) * 16 * FM;
  const int cw = tn * BN + (wave % 2) * 16 * FN;
  const bf16* bp[FN];
#pragma unroll
  for (int j = 0; j < FN; ++j) bp[j] = Wt + ((((int64_t)(cw / 16 + j) * wks) << 6) + lane) * 8;
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ra[FM], rb[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) ra[i] = al.load(rw + 16 * i + (lane & 15), 0, lane);
#pragma unroll
  for (int j = 0; j < FN; ++j) rb[j] = ld16(bp[j]);
  for (int s = 0; s < ksteps; ++s) {
    Frag<bf16> a[FM], b[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i].from_raw(&ra[i]);
#pragma unroll
    for (int j = 0; j < FN; ++j) b[j].from_raw(&rb[j]);
    if (s + 1 < ksteps) {
#pragma unroll
      for (int i = 0; i < FM; ++i) ra[i] = al.load(rw + 16 * i + (lane & 15), s + 1, lane);
#pragma unroll
      for (int j = 0; j < FN; ++j) rb[j] = ld16(bp[j] + (s + 1) * 512);
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_16x16x32(acc[i][j], a[i], b[j]);
  }
  ep.template tile<FM, FN>(acc, rw + (lane >> 4) * 4, cw, lane);
}

// The same product staged through LDS for operands in fragment order: a 128 x 128 block of 4
// waves (64 x 64 each) fetches every k-step's 8 A and 8 B fragments once (16 KB, one 16-byte
// load per thread and operand pair), into one of two LDS buffers while the other is multiplied;
// waves then read their 4 + 4 fragments from LDS. One barrier per k-step.
template <class EP>
__global__ __launch_bounds__(kThreads) void k_gemm_lds(int N, int ksteps, const bf16* __restrict__ A,
                                                     int R, const bf16* __restrict__ Wt, EP ep) {
  constexpr int FM = 4, FN = 4, BM = 128, BN = 128;
  __shared__ __attribute__((aligned(16))) u32x4 as[2][8][kWave];
  __shared__ __attribute__((aligned(16))) u32x4 bs[2][8][kWave];
  const int tiles_n = N / BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x - tm * tiles_n;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / 2, wn = wave % 2;
  // this thread stages fragments f and f + 4 of A and of B (f = tid / 64, its lane = tid % 64)
  const int f = tid / kWave;
  const int last_rt = (R - 1) >> 4;
  const bf16* ap[2];
  const bf16* bp[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int rt = min(tm * 8 + f + 4 * u, last_rt);
    ap[u] = A + ((((int64_t)rt * ksteps) << 6) + lane) * 8;
    bp[u] = Wt + ((((int64_t)(tn * 8 + f + 4 * u) * ksteps) << 6) + lane) * 8;
  }
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 ra[2], rb[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    ra[u] = ld16(ap[u]);
    rb[u] = ld16(bp[u]);
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    as[0][f + 4 * u][lane] = ra[u];
    bs[0][f + 4 * u][lane] = rb[u];
  }
  __syncthreads();
  for (int s = 0; s < ksteps; ++s) {
    const int cur = s & 1;
    if (s + 1 < ksteps) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        ra[u] = ld16(ap[u] + (s + 1) * 512);
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
        as[cur ^ 1][f + 4 * u][lane] = ra[u];
        bs[cur ^ 1][f + 4 * u][lane] = rb[u];
      }
    }
    __syncthreads();
  }
  ep.template tile<FM, FN>(acc, tm * BM + wm * 64 + (lane >> 4) * 4, tn * BN + wn * 64, lane);
}

// Epilogues. Lane l of a wave holds acc[fm][fn][i] = C[rbase + 16 fm + i][cwave + 16 fn + l % 16]
// (rbase already includes 4 (l / 16)). Rows >= R are padding and are never stored.
template <class D>
struct PerElement {
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + 16 * fm + i;
          if (row < static_cast<const D*>(this)->R)
            static_cast<const D*>(this)->op(row, cwave + 16 * fn + (lane & 15), acc[fm][fn][i]);
        }
  }
};

// h = sigmoid(v + b) * e  (the gated merge with alpha = 0)
struct PGate : PerElement<PGate> {
  float* h;
  const bf16* e;
  int64_t e_seq;
  const float* b;
  int n, d, R;
  __device__ void op(int row, int col, float v) const {
    const int bs = row / n, i = row - bs * n;
    const float ev = (float)e[((int64_t)bs * e_seq + i) * d + col];
    h[(int64_t)row * d + col] = sigmoidf_(v + b[col]) * ev;
  }
};

// Query / key / value of every token into per-head blocks [B][H][n][hd]; with N = d (the
// cross-attention query) only q is written.
struct PHeads : PerElement<PHeads> {
  bf16* q;
  bf16* k;
  bf16* v;
  int n, d, H, hd, R;
  __device__ void op(int row, int col, float x) const {
    const int b = row / n, i = row - b * n;
    bf16* dst = q;
    if (col >= d) {
      col -= d;
      dst = k;
      if (col >= d) {
        col -= d;
        dst = v;
      }
    }
    const int hh = col / hd, dd = col - hh * hd;
    dst[(((int64_t)b * H + hh) * n + i) * hd + dd] = (bf16)x;
  }
};

// h += v (fp32, in place); at the last layer also s rows to out (row (b, i) at
// out + b * out_seq + i * d).
struct PResidual : PerElement<PResidual> {
  float* h;
  float* out;
  int64_t out_seq;
  int n, d, R;
  __device__ void op(int row, int col, float v) const {
    float* p = h + (int64_t)row * d + col;
    const float r = *p + v;
    *p = r;
    if (out) {
      const int b = row / n, i = row - b * n;
      out[(int64_t)b * out_seq + (int64_t)i * d + col] = r;
    }
  }
};

// act = SiLU(x W1) * (x W3) in fragment order. The packed up-projection interleaves 16 columns
// of W1 and the same 16 of W3 per 32 columns, and a wave's FN (even) fragments start on a
// multiple of 32, so fragments 2j and 2j + 1 of a lane hold the two factors of one output.
struct PSilu {
  bf16* act;
  int F, R;
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
    static_assert(FN % 2 == 0, "pairs of W1 / W3 fragments");
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int j = 0; j < FN / 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + 16 * fm + i;
          if (row >= R) continue;
          const float z1 = acc[fm][2 * j][i], z3 = acc[fm][2 * j + 1][i];
          const int col = (cwave + 32 * j) / 2 + (lane & 15);
          act[frag_off(row, col, F / 32)] = (bf16)(z1 * sigmoidf_(z1) * z3);
        }
  }
};

// ---- RMSNorm of every row into the next GEMM's operand -------------------------------------------
// One wave per row: a = bf16(h * gamma / sqrt(mean(h^2) + eps)) in fragment order.
__global__ __launch_bounds__(kThreads) void k_norm_rows(const float* __restrict__ h,
                                                        const float* __restrict__ gamma, int d,
                                                        float eps, int R, bf16* __restrict__ a) {
  const int row = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= R) return;
  const float* x = h + (int64_t)row * d;
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += kWave * 4) {
    const u32x4 r = ld16(x + c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float v = __uint_as_float(r[i]);
      ss += v * v;
    }
  }
  ss = wave_sum(ss);
  const float rinv = rsqrtf(ss / (float)d + eps);
  for (int c = lane * 8; c < d; c += kWave * 8) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)(x[c + i] * gamma[c + i] * rinv);
    st16(a + frag_off(row, c, d / 32), __builtin_bit_cast(u32x4, o));
  }
}

// ---- causal flash attention, all queries of a (sequence, head) block at once ----------------------
// A workgroup takes 64 consecutive queries of one (sequence, head); wave w owns queries
// q0 + 16 w .. + 15. Key blocks of 64 are staged in LDS (K as rows, V transposed) and each wave
// computes S^T = K Q^T with MFMA, so a lane holds the scores of one query (lane % 16) against
// keys 4 (lane / 16) + i of each 16-key tile. The softmax is online (running max and sum per
// query, in fp32). For O^T = V^T P^T the MFMA's k index is taken in the order the lane already
// holds P (per 32 keys: keys 4 g + [0, 4) of the first 16-key tile, then of the second,
// g = lane / 16), and V^T is read from LDS in that same order, so P never moves between lanes.
// Masks: the key j of query t is used when j <= t, and for the window also j > t - W.
template <int HD>
__global__ __launch_bounds__(kThreads) void k_flash(const bf16* __restrict__ Q,
                                                    const bf16* __restrict__ K,
                                                    const bf16* __restrict__ V,
                                                    int64_t kv_bh_stride, int n, int H, int W,
                                                    int qblocks, float scale, bf16* __restrict__ o) {
  constexpr int KB = 64, QB = 64, KS = HD / 32, VT = HD / 16, NT = KB / 16, PK = KB / 32;
  __shared__ __attribute__((aligned(16))) bf16 ks[KB][HD + 8];
  __shared__ __attribute__((aligned(16))) bf16 vt[HD][KB + 8];
  // heavy blocks (late queries) first
  const int qb = qblocks - 1 - (int)(blockIdx.x % qblocks);
  const int bh = blockIdx.x / qblocks;
  const int b = bh / H, hh = bh - b * H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane >> 4;
  const int q0 = qb * QB, qw = q0 + wave * 16;
  const int tq = qw + (lane & 15);  // this lane's query (token index)
  const bf16* Qb = Q + ((int64_t)bh * n) * HD;
  const bf16* Kb = K + (int64_t)bh * kv_bh_stride;
  const bf16* Vb = V + (int64_t)bh * kv_bh_stride;

  Frag<bf16> qf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) qf[s].load(Qb + (int64_t)min(tq, n - 1) * HD + 32 * s + 8 * g);

  f32x4 acc[VT];
#pragma unroll
  for (int c = 0; c < VT; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.f;

  const int kend = min(n, q0 + QB);                      // keys this block can use
  const int kbeg = W > 0 ? max(0, q0 - W + 1) / KB * KB : 0;
  // staging: thread -> CH chunks of (key, 8 dims), consecutive threads on consecutive keys, so
  // a wave's transposed V writes fill whole LDS rows without bank conflicts; the next block's
  // chunks are loaded into registers while the current block is multiplied
  constexpr int CH = KB * HD / 8 / kThreads;
  static_assert(CH >= 1 && KB * HD / 8 == CH * kThreads, "staging split");
  u32x4 kr[CH], vr[CH];
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = tid + u * kThreads;
      const int key = k0 + c % KB, dd = (c / KB) * 8;
      kr[u] = vr[u] = u32x4{0, 0, 0, 0};
      if (key < kend) {
        kr[u] = ld16(Kb + (int64_t)key * HD + dd);
        vr[u] = ld16(Vb + (int64_t)key * HD + dd);
      }
    }
  };
  // scores go through exp2: fold log2(e) into the scale
  const float c2 = scale * 1.4426950408889634f;
  if (kbeg < kend) fetch(kbeg);
  for (int k0 = kbeg; k0 < kend; k0 += KB) {
    __syncthreads();  // the previous block's LDS reads are done
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = tid + u * kThreads;
      const int kk = c % KB, dd = (c / KB) * 8;
      *reinterpret_cast<u32x4*>(&ks[kk][dd]) = kr[u];
      const bf16x8 v8 = __builtin_bit_cast(bf16x8, vr[u]);
#pragma unroll
      for (int i = 0; i < 8; ++i) vt[dd + i][kk] = v8[i];
    }
    __syncthreads();
    if (k0 + KB < kend) fetch(k0 + KB);
    // S^T for the NT 16-key tiles
    f32x4 st[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      st[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&ks[16 * j + (lane & 15)][32 * s + 8 * g]));
        st[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s].v, st[j], 0, 0, 0);
      }
    }
    // scale (and mask, unless every key of the block is valid for every query of the wave:
    // all keys exist, none is later than the wave's first query, none falls out of the window
    // of its last)
    const bool interior = k0 + KB <= kend && k0 + KB - 1 <= qw && (W <= 0 || k0 > qw + 15 - W);
    float p[4 * NT];
    float mx = -INFINITY;
    if (interior) {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[4 * j + i] = st[j][i] * c2;
          mx = fmaxf(mx, p[4 * j + i]);
        }
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = k0 + 16 * j + 4 * g + i;
          const bool ok = key <= tq && key < kend && (W <= 0 || key > tq - W);
          p[4 * j + i] = ok ? st[j][i] * c2 : -INFINITY;
          mx = fmaxf(mx, p[4 * j + i]);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    // a query with no key yet keeps m = -inf, l = 0 and adds zero weights (every wave runs the
    // same MFMAs, so no lane leaves the loop early); exp2(-inf) = 0
    const float mn = fmaxf(m, mx);
    const float ms = mn == -INFINITY ? 0.f : mn;
    const float alpha = __builtin_amdgcn_exp2f(m - ms);
    float ps = 0.f;
    bf16x8 pb[PK];
#pragma unroll
    for (int e = 0; e < 4 * NT; ++e) {
      const float x = __builtin_amdgcn_exp2f(p[e] - ms);
      ps += x;
      pb[e / 8][e % 8] = (bf16)x;
    }
    ps += __shfl_xor(ps, 16, kWave);
    ps += __shfl_xor(ps, 32, kWave);
    l = l * alpha + ps;
    m = mn;
#pragma unroll
    for (int c = 0; c < VT; ++c) {
      acc[c] *= alpha;
#pragma unroll
      for (int h = 0; h < PK; ++h) {
        // V^T row 16 c + lane % 16, the 8 keys of this lane's P order in k-step h: tile 2h
        // keys 4g..4g+3, then tile 2h+1 keys 4g..4g+3
        const bf16* vp = &vt[16 * c + (lane & 15)][32 * h];
        const uint2 lo = *reinterpret_cast<const uint2*>(vp + 4 * g);
        const uint2 hi = *reinterpret_cast<const uint2*>(vp + 16 + 4 * g);
        const u32x4 raw = {lo.x, lo.y, hi.x, hi.y};
        acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, raw), pb[h],
                                                         acc[c], 0, 0, 0);
      }
    }
  }
  if (tq >= n) return;
  const float inv = 1.f / l;
  const int row = b * n + tq, d = H * HD;
#pragma unroll
  for (int c = 0; c < VT; ++c) {
    // lane holds O^T[dim 16 c + 4 g + i][query tq]
    const int dim = hh * HD + 16 * c + 4 * g;
    uint2 w;
    bf16 v4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = (bf16)(acc[c][i] * inv);
    w.x = (uint32_t)__builtin_bit_cast(uint16_t, v4[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, v4[1]) << 16);
    w.y = (uint32_t)__builtin_bit_cast(uint16_t, v4[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, v4[3]) << 16);
    *reinterpret_cast<uint2*>(o + frag_off(row, dim, d / 32)) = w;
  }
}

// ---- hand-off to the recurrent path --------------------------------------------------------------
// Ring slots of layer l receive the keys / values of tokens max(0, n - (W - 1)) .. n - 1 (token
// tau in slot tau % W), as n recurrent steps leave them.
__global__ __launch_bounds__(kThreads) void k_fill_ring(const bf16* __restrict__ k,
                                                        const bf16* __restrict__ v, int n, int H,
                                                        int hd, int W, int keep,
                                                        bf16* __restrict__ ring_k,
                                                        bf16* __restrict__ ring_v,
                                                        int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;  // total = B * H * keep * hd
  const int dd = (int)(i % hd);
  int64_t r = i / hd;
  const int e = (int)(r % keep);
  const int64_t bh = r / keep;
  const int tau = n - keep + e;
  const int64_t src = (bh * n + tau) * hd + dd;
  const int64_t dst = (bh * W + tau % W) * hd + dd;
  ring_k[dst] = k[src];
  ring_v[dst] = v[src];
}

__global__ __launch_bounds__(kThreads) void k_copy_last(const float* __restrict__ h, int n, int d,
                                                        int64_t total, float* __restrict__ s) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;  // total = B * d
  const int64_t b = i / d;
  s[i] = h[(b * n + (n - 1)) * d + i % d];
}

// ---- host side ------------------------------------------------------------------------------------

ParLayout par_layout(const Dims& D, int B, int64_t n) {
  ParLayout p;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = (o + bytes + 255) / 256 * 256;
    return at;
  };
  const size_t R = (size_t)B * n, R16 = (R + 63) / 64 * 64, d = D.d;
  p.h = take(R * d * 4);
  p.a = take(R16 * d * 2);
  p.q = take(R * d * 2);
  p.k = take(R * d * 2);
  p.v = take(R * d * 2);
  p.o = take(R16 * d * 2);
  p.act = take(R16 * D.F * 2);
  p.total = o;
  return p;
}

// Every launch of the pass goes through Exec x, timed by the state's profiler as its kind.
struct ParCtx {
  hipStream_t st;
  Profiler* prof;
  hipError_t arm(int kind, double bytes, double flops, Exec& x) const {
    x = Exec(st);
    return prof ? prof->arm(kind, bytes, flops, x) : hipSuccess;
  }
};

template <int FM, int FN, class AL, class EP>
static hipError_t gemm_rows_t(const ParCtx& c, int R, int N, int K, int wks, const void* Wt,
                              const AL& al, const EP& ep, double out_bytes) {
  constexpr int BM = 32 * FM, BN = 32 * FN;
  if (N % BN != 0 || K % 32 != 0) return hipErrorInvalidValue;
  const int64_t blocks = (int64_t)((R + BM - 1) / BM) * (N / BN);
  if (blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
  Exec x(c.st);
  hipError_t e = c.arm(RLT_K_PAR_GEMM, 2.0 * ((double)R * K + (double)K * N) + out_bytes,
                       2.0 * R * N * K, x);
  if (e != hipSuccess) return e;
  return launch(k_gemm_rows<FM, FN, AL, EP>, dim3((unsigned)blocks), dim3(kThreads), x, N, K / 32,
                wks, static_cast<const bf16*>(Wt), al, ep);
}

// Largest register tile the shape allows: 64 x 64 per wave (128 x 128 per block) when N is a
// multiple of 128, else 32 x 32 per wave. Fragment-ordered operands with such N go through LDS.
template <class AL, class EP>
static hipError_t gemm_rows(const ParCtx& c, int R, int N, int K, int wks, const void* Wt,
                            const AL& al, const EP& ep, double out_bytes) {
  if constexpr (std::is_same<AL, PA>::value) {
    if (N % 128 == 0 && wks == K / 32) {
      const int64_t blocks = (int64_t)((R + 127) / 128) * (N / 128);
      if (K % 32 != 0 || blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
      Exec x(c.st);
      hipError_t e = c.arm(RLT_K_PAR_GEMM, 2.0 * ((double)R * K + (double)K * N) + out_bytes,
                           2.0 * R * N * K, x);
      if (e != hipSuccess) return e;
      return launch(k_gemm_lds<EP>, dim3((unsigned)blocks), dim3(kThreads), x, N, K / 32, al.a,
                    R, static_cast<const bf16*>(Wt), ep);
    }
  }
  if (N % 128 == 0) return gemm_rows_t<4, 4>(c, R, N, K, wks, Wt, al, ep, out_bytes);
  return gemm_rows_t<2, 2>(c, R, N, K, wks, Wt, al, ep, out_bytes);
}

// W > 0: window attention (keys t-W+1..t of this layer); W = 0: memory prefix 0..t.
template <int HD>
static hipError_t flash_t(const ParCtx& c, const bf16* q, const bf16* k, const bf16* v,
                          int64_t kv_bh_stride, int B, int n, int H, int W, bf16* o) {
  const int qblocks = (n + 63) / 64;
  const int64_t blocks = (int64_t)B * H * qblocks;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  // keys per query summed over t = 0..n-1: min(t + 1, W) or t + 1
  double keys = 0;
  if (W > 0) {
    const double full = n > W ? (double)(n - W) : 0.0, ramp = n < W ? n : W;
    keys = full * W + ramp * (ramp + 1) / 2;
  } else {
    keys = (double)n * (n + 1) / 2;
  }
  const double bhd = (double)B * H * HD;
  Exec x(c.st);
  hipError_t e = c.arm(W > 0 ? RLT_K_PAR_SELF : RLT_K_PAR_CROSS, bhd * n * 2 * 4.0,
                       4.0 * bhd * keys, x);
  if (e != hipSuccess) return e;
  return launch(k_flash<HD>, dim3((unsigned)blocks), dim3(kThreads), x, q, k, v, kv_bh_stride, n,
                H, W, qblocks, 1.f / sqrtf((float)HD), o);
}

static hipError_t flash(const ParCtx& c, int hd, const bf16* q, const bf16* k, const bf16* v,
                        int64_t kv_bh_stride, int B, int n, int H, int W, bf16* o) {
  switch (hd) {
    case 32: return flash_t<32>(c, q, k, v, kv_bh_stride, B, n, H, W, o);
    case 64: return flash_t<64>(c, q, k, v, kv_bh_stride, B, n, H, W, o);
    case 128: return flash_t<128>(c, q, k, v, kv_bh_stride, B, n, H, W, o);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t norm_rows(const ParCtx& c, const Dims& D, const float* h, const float* gamma,
                            int R, bf16* a) {
  const int per = kThreads / kWave;
  Exec x(c.st);
  hipError_t e = c.arm(RLT_K_PAR_OTHER, (double)R * D.d * 6, 4.0 * R * D.d, x);
  if (e != hipSuccess) return e;
  return launch(k_norm_rows, dim3((unsigned)((R + per - 1) / per)), dim3(kThreads), x, h, gamma,
                D.d, D.eps, R, a);
}

hipError_t launch_parallel(const Dims& D, int B, const Packed& P, const StateBufs& S,
                           const MemBufs& M, const void* e, int64_t e_seq, int64_t n_,
                           float* out, int64_t out_seq, void* ws, hipStream_t st,
                           Profiler* prof) {
  if (D.dtype != RLT_BF16 || n_ < 1 || (int64_t)B * n_ > INT32_MAX / 2) return hipErrorInvalidValue;
  const ParCtx c{st, prof};
  const int n = (int)n_, R = B * n, d = D.d, F = D.F, H = D.H, hd = D.hd;
  const double Rd = (double)R * d;
  const ParLayout Lp = par_layout(D, B, n);
  char* w = static_cast<char*>(ws);
  float* h = reinterpret_cast<float*>(w + Lp.h);
  bf16* a = reinterpret_cast<bf16*>(w + Lp.a);
  bf16* q = reinterpret_cast<bf16*>(w + Lp.q);
  bf16* kk = reinterpret_cast<bf16*>(w + Lp.k);
  bf16* vv = reinterpret_cast<bf16*>(w + Lp.v);
  bf16* o = reinterpret_cast<bf16*>(w + Lp.o);
  bf16* act = reinterpret_cast<bf16*>(w + Lp.act);
  const bf16* eb = static_cast<const bf16*>(e);
  hipError_t err;
  // gated merge, alpha = 0: only the e_t half of W_g contributes
  {
    PTokens al{eb, e_seq, n, d, R};
    PGate ep;
    ep.h = h; ep.e = eb; ep.e_seq = e_seq; ep.b = P.b_gate; ep.n = n; ep.d = d; ep.R = R;
    if ((err = gemm_rows(c, R, d, d, 2 * d / 32, P.w_gate_t, al, ep, Rd * 6)) != hipSuccess)
      return err;
  }
  const int keep = n < D.W - 1 ? n : D.W - 1;
  for (int l = 0; l < D.L; ++l) {
    const bool last = l == D.L - 1;
    const float* gam = P.gamma + (int64_t)l * 3 * d;
    const int64_t wdd = (int64_t)l * d * d;
    // self-attention sublayer
    if ((err = norm_rows(c, D, h, gam, R, a)) != hipSuccess) return err;
    {
      PHeads ep{{}, q, kk, vv, n, d, H, hd, R};
      const bf16* Wq = static_cast<const bf16*>(P.wqkv_t) + (int64_t)l * 3 * d * d;
      if ((err = gemm_rows(c, R, 3 * d, d, d / 32, Wq, PA{a, d / 32, R}, ep, Rd * 6)) !=
          hipSuccess)
        return err;
    }
    if (keep > 0) {
      const int64_t total = (int64_t)B * H * keep * hd;
      const int64_t ring_layer = (int64_t)S.Bt * H * D.W * hd;
      Exec x(st);
      if ((err = c.arm(RLT_K_PAR_OTHER, (double)total * 8, 0, x)) != hipSuccess) return err;
      err = launch(k_fill_ring, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads),
                   x, (const bf16*)kk, (const bf16*)vv, n, H, hd, D.W, keep,
                   static_cast<bf16*>(S.ring_k) + l * ring_layer,
                   static_cast<bf16*>(S.ring_v) + l * ring_layer, total);
      if (err != hipSuccess) return err;
    }
    if ((err = flash(c, hd, q, kk, vv, (int64_t)n * hd, B, n, H, D.W, o)) != hipSuccess) return err;
    {
      PResidual ep{{}, h, nullptr, 0, n, d, R};
      const bf16* Wo = static_cast<const bf16*>(P.wo_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wo, PA{o, d / 32, R}, ep, Rd * 8)) !=
          hipSuccess)
        return err;
    }
    // cross-attention sublayer: memory entries 1..t of this layer's group
    if ((err = norm_rows(c, D, h, gam + d, R, a)) != hipSuccess) return err;
    {
      PHeads ep{{}, q, nullptr, nullptr, n, d, H, hd, R};
      const bf16* Wc = static_cast<const bf16*>(P.wcq_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wc, PA{a, d / 32, R}, ep, Rd * 2)) !=
          hipSuccess)
        return err;
    }
    {
      const int gsel = D.G == 1 ? 0 : l;
      const int64_t grp = (int64_t)gsel * M.Bt * H * M.capacity * hd;
      if ((err = flash(c, hd, q, static_cast<const bf16*>(M.k) + grp,
                       static_cast<const bf16*>(M.v) + grp, M.capacity * hd, B, n, H, 0, o)) !=
          hipSuccess)
        return err;
    }
    {
      PResidual ep{{}, h, nullptr, 0, n, d, R};
      const bf16* Wco = static_cast<const bf16*>(P.wco_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wco, PA{o, d / 32, R}, ep, Rd * 8)) !=
          hipSuccess)
        return err;
    }
    // FFN sublayer
    if ((err = norm_rows(c, D, h, gam + 2 * d, R, a)) != hipSuccess) return err;
    {
      PSilu ep{act, F, R};
      const bf16* W13 = static_cast<const bf16*>(P.w13_t) + (int64_t)l * 2 * F * d;
      if ((err = gemm_rows(c, R, 2 * F, d, d / 32, W13, PA{a, d / 32, R}, ep,
                                 (double)R * F * 2)) != hipSuccess)
        return err;
    }
    {
      PResidual ep{{}, h, last ? out : nullptr, out_seq, n, d, R};
      const bf16* W2 = static_cast<const bf16*>(P.w2_t) + (int64_t)l * d * F;
      if ((err = gemm_rows(c, R, d, F, F / 32, W2, PA{act, F / 32, R}, ep,
                                 Rd * (last && out ? 12 : 8))) != hipSuccess)
        return err;
    }
  }
  const int64_t total = (int64_t)B * d;
  Exec x(st);
  if ((err = c.arm(RLT_K_PAR_OTHER, (double)total * 8, 0, x)) != hipSuccess) return err;
  err = launch(k_copy_last, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads),
               x, (const float*)h, n, d, total, S.s);
  if (err != hipSuccess) return err;
  return launch_set_positions(S.pos, B, n, st);
}

}  // namespace rlt
