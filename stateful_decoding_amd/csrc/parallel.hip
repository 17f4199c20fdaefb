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

// max over the four lanes l, l ^ 16, l ^ 32, l ^ 48 with the gfx950 row swaps (VALU, no LDS):
// each swap leaves the lane's own value and its partner's in the two results, in either order
__device__ __forceinline__ float max_xor16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

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

// The large-row product for N a multiple of 256: a 256 x 256 block of 8 waves (2 x 4, each
// 128 x 64 = 8 x 4 fragments). Each k-step's 16 A and 16 B fragments (32 KB) are copied from
// global memory straight into LDS (global_load_lds, 16 bytes per lane: a fragment is 1 KB in
// lane order in both places), four k-steps deep, so up to three stages are in flight while one
// is multiplied; one barrier per k-step. The weights are the MFMA's first operand, so a lane's
// accumulator holds 4 consecutive output columns of one row and the epilogues store 8 or 16
// contiguous bytes. Workgroups are numbered XCD-major: the i-th workgroup dispatched to an XCD
// takes the i-th tile of that XCD's contiguous share, so the tiles of one row block (sharing
// their A fragments) meet in the same L2.
constexpr int kBigThreads = 512;
constexpr int kBigStages = 4;

// ATok: A is not fragment-ordered but token rows, row (b, i) at A + (b * a_seq + i) * K (a_n
// tokens per sequence): each lane then copies the 16 bytes of its own row, which lands in LDS
// in the same fragment order.
struct ATok {
  int64_t a_seq;
  int a_n;
};

template <class EP, bool TOK = false>
__global__ __launch_bounds__(kBigThreads) void k_gemm_big(int N, int ksteps,
                                                         const bf16* __restrict__ A, int R,
                                                         const bf16* __restrict__ Wt, int wks,
                                                         EP ep, ATok tok) {
  constexpr int FM = 8, FN = 4, PER = 4;  // fragments each wave copies per k-step
  __shared__ __attribute__((aligned(16))) u32x4 sm[kBigStages][32][kWave];
  const int tiles_n = N / 256, nb = (int)gridDim.x;
  int tile = (int)blockIdx.x;
  if ((nb & 7) == 0) tile = (tile & 7) * (nb >> 3) + (tile >> 3);
  const int tm = tile / tiles_n, tn = tile - tm * tiles_n;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;
  const int wm = wave / 4, wn = wave % 4;
  const int last_rt = (R - 1) >> 4;
  // fragment slot f = wave + 8 u of a stage: slots 0..15 are A row tiles, 16..31 W column tiles
  const bf16* gp[PER];
  int gstep[PER];  // elements from one k-step to the next
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int f = wave + 8 * u;
    gstep[u] = 512;
    if (f >= 16) {
      gp[u] = Wt + ((((int64_t)(tn * 16 + f - 16) * wks) << 6) + lane) * 8;
    } else if (TOK) {
      const int r = min(tm * 256 + f * 16 + (lane & 15), R - 1);
      const int b = r / tok.a_n, i = r - b * tok.a_n;
      gp[u] = A + ((int64_t)b * tok.a_seq + i) * (ksteps * 32) + (lane >> 4) * 8;
      gstep[u] = 32;
    } else {
      gp[u] = A + ((((int64_t)min(tm * 16 + f, last_rt) * ksteps) << 6) + lane) * 8;
    }
  }
  auto issue = [&](int s) {
    const int buf = s % kBigStages;
#pragma unroll
    for (int u = 0; u < PER; ++u)
      __builtin_amdgcn_global_load_lds(
          (const void*)(gp[u] + (int64_t)s * gstep[u]),
          (__attribute__((address_space(3))) void*)&sm[buf][wave + 8 * u][0], 16, 0, 0);
  };
  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < kBigStages - 1 && s < ksteps; ++s) issue(s);
  for (int s = 0; s < ksteps; ++s) {
    // this wave's copies of stage s are complete once at most the later stages' remain in
    // flight (s_waitcnt vmcnt(n); lgkmcnt(0) too); the barrier then makes every wave's copies
    // visible and guarantees that stage s - 1's buffer, reused below, is no longer read
    const int later = min(kBigStages - 2, ksteps - 1 - s);
    asm volatile("" ::: "memory");
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(0x0070 | (2 * PER));
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(0x0070 | PER);
    else
      __builtin_amdgcn_s_waitcnt(0x0070);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (s + kBigStages - 1 < ksteps) issue(s + kBigStages - 1);
    const int cur = s % kBigStages;
    Frag<bf16> w[FN];
#pragma unroll
    for (int j = 0; j < FN; ++j) w[j].from_raw(&sm[cur][16 + wn * 4 + j][lane]);
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      Frag<bf16> a;
      a.from_raw(&sm[cur][wm * 8 + i][lane]);
#pragma unroll
      for (int j = 0; j < FN; ++j) mfma_16x16x32(acc[i][j], w[j], a);
    }
  }
  ep.template tile_t<FM, FN>(acc, tm * 256 + wm * 128 + (lane & 15),
                             tn * 256 + wn * 64 + 4 * (lane >> 4), lane);
}

// Epilogues. Lane l of a wave holds acc[fm][fn][i] = C[rbase + 16 fm + i][cwave + 16 fn + l % 16]
// (rbase already includes 4 (l / 16)) after k_gemm_rows / k_gemm_lds, and
// acc[fm][fn][i] = C[row0 + 16 fm][col0 + 16 fn + i] (row0 = rows of l % 16, col0 includes
// 4 (l / 16)) after k_gemm_big (tile_t). Rows >= R are padding and are never stored.
// RMSNorm folded around a product: when ssq is set, the operand was bf16(h * gamma) and output
// row r is scaled by 1/rms(h_r) = rsqrt(sum of the row's nslot partial sums of squares / d +
// eps) (a per-row scalar commutes with the product); otherwise the scale is 1.
struct RowScale {
  const float* rinv = nullptr;  // [R] 1/rms of each row (k_row_rinv), or none
  __device__ float scale(int row) const { return rinv ? rinv[row] : 1.f; }
};

// rinv[row] = rsqrt(sum of the row's nslot partial sums of squares / d + eps)
__global__ __launch_bounds__(kThreads) void k_row_rinv(const float* __restrict__ ssq, int nslot,
                                                       float inv_d, float eps, int R,
                                                       float* __restrict__ rinv) {
  const int row = blockIdx.x * kThreads + threadIdx.x;
  if (row >= R) return;
  const float* p = ssq + (int64_t)row * nslot;
  float t = 0.f;
  for (int j = 0; j < nslot; ++j) t += p[j];
  rinv[row] = rsqrtf(t * inv_d + eps);
}

template <class D>
struct PerElement {
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
    const D& ep = *static_cast<const D*>(this);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = rbase + 16 * fm + i;
        if (row >= ep.R) continue;
        const float sc = ep.scale(row);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          ep.op(row, cwave + 16 * fn + (lane & 15), acc[fm][fn][i] * sc);
      }
  }
  template <int FM, int FN>
  __device__ void tile_t(const f32x4 (&acc)[FM][FN], int row0, int col0, int lane) const {
    const D& ep = *static_cast<const D*>(this);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int row = row0 + 16 * fm;
      if (row < ep.R) {
        const float sc = ep.scale(row);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) ep.op4(row, col0 + 16 * fn, acc[fm][fn] * sc);
      }
    }
  }
};

__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v) {
  bf16 b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) b[i] = (bf16)v[i];
  return uint2{(uint32_t)__builtin_bit_cast(uint16_t, b[0]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, b[1]) << 16),
               (uint32_t)__builtin_bit_cast(uint16_t, b[2]) |
                   ((uint32_t)__builtin_bit_cast(uint16_t, b[3]) << 16)};
}

// h = sigmoid(v + b) * e  (the gated merge with alpha = 0)
struct PGate : PerElement<PGate>, RowScale {
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
  __device__ uint2 e4(int row, int col) const {
    if (row >= R) return uint2{0u, 0u};
    const int bs = row / n, i = row - bs * n;
    return *reinterpret_cast<const uint2*>(e + ((int64_t)bs * e_seq + i) * d + col);
  }
  __device__ void store4(int row, int col, f32x4 v, uint2 eraw, f32x4 bias) const {
    const float ev[4] = {__uint_as_float(eraw.x << 16), __uint_as_float(eraw.x & 0xffff0000u),
                         __uint_as_float(eraw.y << 16), __uint_as_float(eraw.y & 0xffff0000u)};
    f32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = sigmoidf_(v[k] + bias[k]) * ev[k];
    *reinterpret_cast<f32x4*>(h + (int64_t)row * d + col) = r;
  }
  __device__ void op4(int row, int col, f32x4 v) const {
    store4(row, col, v, e4(row, col), *reinterpret_cast<const f32x4*>(b + col));
  }
  // after k_gemm_big: every e_t value of the wave's tile is read before the first store (a
  // wait for a load also waits for the stores issued before it)
  template <int FM, int FN>
  __device__ void tile_t(const f32x4 (&acc)[FM][FN], int row0, int col0, int) const {
    f32x4 bias[FN];
    uint2 ev[FM][FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) bias[fn] = *reinterpret_cast<const f32x4*>(b + col0 + 16 * fn);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) ev[fm][fn] = e4(row0 + 16 * fm, col0 + 16 * fn);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int row = row0 + 16 * fm;
      if (row >= R) continue;
      const float sc = scale(row);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        store4(row, col0 + 16 * fn, acc[fm][fn] * sc, ev[fm][fn], bias[fn]);
    }
  }
};

// Query / key / value of every token into per-head blocks [B][H][n][hd]; with N = d (the
// cross-attention query) only q is written.
struct PHeads : PerElement<PHeads>, RowScale {
  bf16* q;
  bf16* k;
  bf16* v;
  int n, d, H, hd, R;
  float qscale = 1.f;  // queries are stored times qscale (k_flash takes them in log2 units)
  __device__ void op(int row, int col, float x) const {
    const int b = row / n, i = row - b * n;
    bf16* dst = q;
    if (col < d) x *= qscale;
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
  // four consecutive columns never straddle q / k / v or a head (d and hd are multiples of 4)
  __device__ void op4(int row, int col, f32x4 x) const {
    const int b = row / n, i = row - b * n;
    bf16* dst = q;
    if (col < d) x *= qscale;
    if (col >= d) {
      col -= d;
      dst = k;
      if (col >= d) {
        col -= d;
        dst = v;
      }
    }
    const int hh = col / hd, dd = col - hh * hd;
    *reinterpret_cast<uint2*>(dst + (((int64_t)b * H + hh) * n + i) * hd + dd) = pack_bf16x4(x);
  }
  // after k_gemm_big: the (sequence, token) split of each of the wave's FM rows and the
  // (q / k / v, head, dim) split of each of its FN column groups are formed once, not per
  // element (hd is a power of two)
  template <int FM, int FN>
  __device__ void tile_t(const f32x4 (&acc)[FM][FN], int row0, int col0, int) const {
    const int hs = __builtin_ctz((unsigned)hd);
    const int64_t head_sz = (int64_t)n << hs;  // elements of one (sequence, head) block
    int sel[FN];  // 0 q, 1 k, 2 v
    int64_t coff[FN];
    float cs[FN];
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      int col = col0 + 16 * fn;
      sel[fn] = 0;
      cs[fn] = qscale;
      if (col >= d) {
        col -= d;
        sel[fn] = 1;
        cs[fn] = 1.f;
        if (col >= d) {
          col -= d;
          sel[fn] = 2;
        }
      }
      coff[fn] = (int64_t)(col >> hs) * head_sz + (col & (hd - 1));
    }
    int b = row0 / n, i = row0 - b * n;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      if (fm > 0) {  // the next fragment row is 16 rows further
        i += 16;
        if (i >= n) {
          b += i / n;
          i -= (i / n) * n;
        }
      }
      const int row = row0 + 16 * fm;
      if (row >= R) continue;
      const float sc = scale(row);
      const int64_t roff = (int64_t)b * H * head_sz + ((int64_t)i << hs);
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        bf16* dst = sel[fn] == 0 ? q : sel[fn] == 1 ? k : v;
        *reinterpret_cast<uint2*>(dst + roff + coff[fn]) = pack_bf16x4(acc[fm][fn] * (sc * cs[fn]));
      }
    }
  }
};

// h += v (fp32, in place); at the last layer also s rows to out (row (b, i) at
// out + b * out_seq + i * d).
// With hg set (after k_gemm_big only), the epilogue also writes the next RMSNorm's operand
// hg = bf16(h * gnext) in fragment order and, per row, the sum of h^2 over each wave's 64
// columns into ssq[row][col / 64] (d / 64 slots, every one written, so nothing is cleared).
struct PResidual : PerElement<PResidual>, RowScale {
  float* h;
  float* out;
  int64_t out_seq;
  int n, d, R;
  bf16* hg = nullptr;
  const float* gnext = nullptr;
  float* ssq_out = nullptr;
  // The old h of row group q + 1 (two fragment rows) is read before row group q is written: a
  // wait for a load also waits for every store issued before it (one counter for both), so
  // reading each fragment of h right after the previous one's stores would cost a memory round
  // trip per fragment; this way the epilogue costs about one.
  template <int FM, int FN>
  __device__ void tile_t(const f32x4 (&acc)[FM][FN], int row0, int col0, int lane) const {
    static_assert(FM % 2 == 0, "row groups of two fragment rows");
    constexpr int GR = 2, NG = FM / GR;
    f32x4 g[FN];
    if (hg) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
        g[fn] = *reinterpret_cast<const f32x4*>(gnext + col0 + 16 * fn);
    }
    const int slot = (col0 - 4 * (lane >> 4)) / 64;
    f32x4 cur[GR][FN], nxt[GR][FN];
    auto load = [&](int q, f32x4(&v)[GR][FN]) {
#pragma unroll
      for (int i = 0; i < GR; ++i) {
        const int row = row0 + 16 * (q * GR + i);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
          v[i][fn] = row < R ? *reinterpret_cast<const f32x4*>(h + (int64_t)row * d + col0 + 16 * fn)
                             : f32x4{0.f, 0.f, 0.f, 0.f};
      }
    };
    load(0, cur);
#pragma unroll
    for (int q = 0; q < NG; ++q) {
      if (q + 1 < NG) load(q + 1, nxt);
#pragma unroll
      for (int i = 0; i < GR; ++i) {
        const int fm = q * GR + i, row = row0 + 16 * fm;
        float ss = 0.f;
        if (row < R) {
          const float sc = scale(row);
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) {
            const int col = col0 + 16 * fn;
            const f32x4 r = cur[i][fn] + acc[fm][fn] * sc;
            *reinterpret_cast<f32x4*>(h + (int64_t)row * d + col) = r;
            if (out) {
              const int b = row / n, t = row - b * n;
              *reinterpret_cast<f32x4*>(out + (int64_t)b * out_seq + (int64_t)t * d + col) = r;
            }
            if (hg) {
              *reinterpret_cast<uint2*>(hg + frag_off(row, col, d / 32)) = pack_bf16x4(r * g[fn]);
#pragma unroll
              for (int e = 0; e < 4; ++e) ss += r[e] * r[e];
            }
          }
        }
        if (hg) {
          // the four lanes holding this row (lane % 16 equal) cover the wave's 64 columns
          ss += __shfl_xor(ss, 16, kWave);
          ss += __shfl_xor(ss, 32, kWave);
          if (row < R && lane < 16) ssq_out[(int64_t)row * (d / 64) + slot] = ss;
        }
      }
      if (q + 1 < NG) {
#pragma unroll
        for (int i = 0; i < GR; ++i)
#pragma unroll
          for (int fn = 0; fn < FN; ++fn) cur[i][fn] = nxt[i][fn];
      }
    }
  }
  __device__ void op(int row, int col, float v) const {
    float* p = h + (int64_t)row * d + col;
    const float r = *p + v;
    *p = r;
    if (out) {
      const int b = row / n, i = row - b * n;
      out[(int64_t)b * out_seq + (int64_t)i * d + col] = r;
    }
  }
  __device__ void op4(int row, int col, f32x4 v) const {
    f32x4* p = reinterpret_cast<f32x4*>(h + (int64_t)row * d + col);
    const f32x4 r = *p + v;
    *p = r;
    if (out) {
      const int b = row / n, i = row - b * n;
      *reinterpret_cast<f32x4*>(out + (int64_t)b * out_seq + (int64_t)i * d + col) = r;
    }
  }
};

// out[row][col] = v (fp32, row stride ld): the readout's logits
struct PStoreF32 : PerElement<PStoreF32>, RowScale {
  float* out;
  int ld, R;
  __device__ void op(int row, int col, float v) const { out[(int64_t)row * ld + col] = v; }
  __device__ void op4(int row, int col, f32x4 v) const {
    *reinterpret_cast<f32x4*>(out + (int64_t)row * ld + col) = v;
  }
};

// Memory keys and values: row (b, i) = token t0 + i of sequence b, column (g, k|v, head, dim);
// four consecutive columns never straddle a head.
struct PMemproj : PerElement<PMemproj>, RowScale {
  bf16* mk;
  bf16* mv;
  int64_t cap, t0;
  int n, B, d, H, hd, R;
  __device__ void op4(int row, int col, f32x4 x) const {
    const int b = row / n, i = row - b * n;
    const int g = col / (2 * d);
    int c = col - g * 2 * d;
    bf16* dst = mk;
    if (c >= d) {
      c -= d;
      dst = mv;
    }
    const int hh = c / hd, dd = c - hh * hd;
    *reinterpret_cast<uint2*>(dst + ((((int64_t)g * B + b) * H + hh) * cap + t0 + i) * hd + dd) =
        pack_bf16x4(x);
  }
};

// act = SiLU(x W1) * (x W3) in fragment order. The packed up-projection interleaves 16 columns
// of W1 and the same 16 of W3 per 32 columns, and a wave's FN (even) fragments start on a
// multiple of 32, so fragments 2j and 2j + 1 of a lane hold the two factors of one output.
struct PSilu : RowScale {
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
          const float sc = scale(row);
          const float z1 = acc[fm][2 * j][i] * sc, z3 = acc[fm][2 * j + 1][i] * sc;
          const int col = (cwave + 32 * j) / 2 + (lane & 15);
          act[frag_off(row, col, F / 32)] = (bf16)(z1 * sigmoidf_(z1) * z3);
        }
  }
  // after k_gemm_big: fragments 2j / 2j + 1 hold the same 4 consecutive output columns of the
  // W1 and W3 halves, which are 4 consecutive k of one row in the fragment-ordered act
  template <int FM, int FN>
  __device__ void tile_t(const f32x4 (&acc)[FM][FN], int row0, int col0, int lane) const {
    static_assert(FN % 2 == 0, "pairs of W1 / W3 fragments");
    const int cbase = col0 - 4 * (lane >> 4);  // the wave's first packed column (multiple of 32)
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int row = row0 + 16 * fm;
      if (row >= R) continue;
      const float sc = scale(row);
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        f32x4 y;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z1 = acc[fm][2 * j][i] * sc, z3 = acc[fm][2 * j + 1][i] * sc;
          y[i] = z1 * sigmoidf_(z1) * z3;
        }
        const int col = (cbase + 32 * j) / 2 + 4 * (lane >> 4);
        *reinterpret_cast<uint2*>(act + frag_off(row, col, F / 32)) = pack_bf16x4(y);
      }
    }
  }
};

// ---- RMSNorm of every row into the next GEMM's operand -------------------------------------------
// One wave per row: a = bf16(h * gamma / sqrt(mean(h^2) + eps)) in fragment order (FRAG) or
// row-major. Each lane owns 8-column chunks lane, lane + 64, ...; rows of up to 64 x 8 x kNC
// columns are held in registers between the sum of squares and the scaling (one read of h),
// wider ones are read again.
constexpr int kNormChunks = 4;  // d <= 2048 from registers

template <bool FRAG>
__global__ __launch_bounds__(kThreads) void k_norm_rows(const float* __restrict__ h,
                                                        const float* __restrict__ gamma, int d,
                                                        float eps, int R, bf16* __restrict__ a) {
  const int row = blockIdx.x * (kThreads / kWave) + threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  if (row >= R) return;
  const float* x = h + (int64_t)row * d;
  auto store = [&](int c, const float (&v)[8], float rinv) {
    const u32x4 g0 = ld16(gamma + c), g1 = ld16(gamma + c + 4);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = (bf16)(v[i] * __uint_as_float(g0[i]) * rinv);
      o[4 + i] = (bf16)(v[4 + i] * __uint_as_float(g1[i]) * rinv);
    }
    bf16* dst = FRAG ? a + frag_off(row, c, d / 32) : a + (int64_t)row * d + c;
    st16(dst, __builtin_bit_cast(u32x4, o));
  };
  auto load8 = [&](int c, float (&v)[8]) {
    const u32x4 r0 = ld16(x + c), r1 = ld16(x + c + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(r0[i]);
      v[4 + i] = __uint_as_float(r1[i]);
    }
  };
  float ss = 0.f;
  if (d <= kWave * 8 * kNormChunks) {
    float v[kNormChunks][8];
#pragma unroll
    for (int q = 0; q < kNormChunks; ++q) {
      const int c = (lane + kWave * q) * 8;
      if (c < d) {
        load8(c, v[q]);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss += v[q][i] * v[q][i];
      }
    }
    const float rinv = rsqrtf(wave_sum(ss) / (float)d + eps);
#pragma unroll
    for (int q = 0; q < kNormChunks; ++q) {
      const int c = (lane + kWave * q) * 8;
      if (c < d) store(c, v[q], rinv);
    }
  } else {
    for (int c = lane * 8; c < d; c += kWave * 8) {
      float v[8];
      load8(c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) ss += v[i] * v[i];
    }
    const float rinv = rsqrtf(wave_sum(ss) / (float)d + eps);
    for (int c = lane * 8; c < d; c += kWave * 8) {
      float v[8];
      load8(c, v);
      store(c, v, rinv);
    }
  }
}

// ---- causal flash attention, all queries of a (sequence, head) block at once ----------------------
// Transposed values keep each group of 32 keys in the order the P V product takes them: position
// 8 g + 4 u + i holds key 16 u + 4 g + i (g, i < 4; u < 2), so the 8 keys a lane multiplies in one
// k-step (4 g + [0, 4) of the first 16-key tile, then of the second) are adjacent.
__device__ __forceinline__ int vt_key(int p) {
  return (p & ~31) | (((p >> 2) & 1) << 4) | (((p >> 3) & 3) << 2) | (p & 3);
}
__device__ __forceinline__ int vt_pos(int k) {
  return (k & ~31) | (((k >> 2) & 3) << 3) | (((k >> 4) & 1) << 2) | (k & 3);
}

// A workgroup takes QB = 64 QT consecutive queries of one (sequence, head); wave w owns the QT
// 16-query tiles starting at q0 + 16 QT w. Key blocks of 64 are staged in LDS: K in the MFMA's
// fragment order (each 1 KB piece one operand fragment with lane l's 16 bytes at 16 l, so every K
// fragment read is a linear 16-byte read per lane, which the LDS serves at full rate; a row-padded
// tile read 16 rows x 16 bytes at a time runs at half of it), V transposed in padded rows. Each
// wave computes S^T = K Q^T with MFMA, every K fragment read from LDS
// serving its QT query tiles, so a lane holds the scores of one query (lane % 16 of a tile)
// against keys 4 (lane / 16) + i of each 16-key tile. The queries come multiplied by the softmax
// scale and log2(e), so scores are in log2 units. The softmax is online in fp32, against a
// per-query reference maximum that moves only when a block's scores exceed it by more than 8,
// and the score product starts from minus that reference, so its results are the exponents
// exp2 takes; the weight sums are taken by the matrix cores (ones x P^T). For
// O^T = V^T P^T the MFMA's k index is taken in the order the lane already holds P (per 32 keys:
// keys 4 g + [0, 4) of the first 16-key tile, then of the second, g = lane / 16), and V^T is
// read from LDS in that same order, so P never moves between lanes.
// Masks: the key j of query t is used when j <= t, and for the window also j > t - W.
// VTG: the values come transposed from global memory (Vt = [B H][HD][vt_len], keys permuted
// within groups of 32 as vt_key gives, zero from key n up to vt_len, a multiple of 64), so staging
// them into LDS is a plain 16-byte copy; otherwise V is [B H][keys][HD] and is transposed (and
// permuted) on its way into LDS with 2-byte stores.
template <int HD, int QT, bool VTG>
__global__ __launch_bounds__(kThreads, 2) void k_flash(const bf16* __restrict__ Q,
                                                    const bf16* __restrict__ K,
                                                    const bf16* __restrict__ V,
                                                    int64_t kv_bh_stride, int n, int H, int W,
                                                    int qblocks, const bf16* __restrict__ Vt,
                                                    int vt_len, bf16* __restrict__ o) {
  constexpr int KB = 64, QB = 64 * QT, KS = HD / 32, VT = HD / 16, NT = KB / 16, PK = KB / 32;
  constexpr int FK = NT * KS;  // K fragments, (16-key tile j, 32-dim step s) at j KS + s
  // two LDS buffers: block k + 1 is staged while block k is multiplied, one barrier per block.
  // K fragment (j, s), lane l: key 16 j + l % 16, dims 32 s + 8 (l / 16). V^T stays in padded
  // rows [HD][KB + 8] (V^T in fragment order measured slower: 35.6-36.2 against 27.8-28.1 ms of
  // memory attention per pass), read 16 bytes at a time at the lane's permuted key positions.
  __shared__ __attribute__((aligned(16))) u32x4 ks[2][FK][kWave];
  __shared__ __attribute__((aligned(16))) bf16 vt[2][HD][KB + 8];
  // Workgroups are numbered XCD-major (the i-th one dispatched to an XCD takes the i-th of that
  // XCD's contiguous share), so the query blocks of one (sequence, head) run on one XCD and read
  // its keys and values through that XCD's L2; within a (sequence, head), heavy blocks (late
  // queries) first.
  int blk = (int)blockIdx.x;
  const int nblocks = (int)gridDim.x;
  if ((nblocks & 7) == 0) blk = (blk & 7) * (nblocks >> 3) + (blk >> 3);
  const int qb = qblocks - 1 - blk % qblocks;
  const int bh = blk / qblocks;
  const int b = bh / H, hh = bh - b * H;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane >> 4;
  const int q0 = qb * QB, qw = q0 + wave * 16 * QT;  // the wave's first query
  const bf16* Qb = Q + ((int64_t)bh * n) * HD;
  const bf16* Kb = K + (int64_t)bh * kv_bh_stride;
  const bf16* Vb = V + (int64_t)bh * kv_bh_stride;
  const bf16* VTb = VTG ? Vt + (int64_t)bh * HD * vt_len : nullptr;

  int tq[QT];  // this lane's query (token index) in each tile
  Frag<bf16> qf[QT][KS];
  f32x4 acc[QT][VT];
  float mref[QT];
  f32x4 lsum[QT];  // every entry: this lane's query's weight sum
  f32x4 cinit[QT];  // every entry: -mb, the score product's initial value (mb below)
  float thr[QT];    // a block whose maximum exceeds this moves the reference (-inf until set)
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    tq[t] = qw + 16 * t + (lane & 15);
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[t][s].load(Qb + (int64_t)min(tq[t], n - 1) * HD + 32 * s + 8 * g);
#pragma unroll
    for (int c = 0; c < VT; ++c) acc[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    mref[t] = -INFINITY;
    lsum[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    cinit[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    thr[t] = -INFINITY;
  }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;

  const int kend = min(n, q0 + QB);                      // keys this block can use
  const int kbeg = W > 0 ? max(0, q0 - W + 1) / KB * KB : 0;
  // staging: thread -> CH 16-byte slots c = tid + 256 u; for K, slot c is lane c % 64 of fragment
  // c / 64 (linear LDS stores); the transposed values come as (dim c / 8, positions 8 (c % 8) ..),
  // plain values as (key c % 64, dims 8 (c / 64) ..), transposed on the way into LDS. The next
  // block's slots are loaded into registers while the current block is multiplied.
  constexpr int CH = KB * HD / 8 / kThreads;
  static_assert(CH >= 1 && KB * HD / 8 == CH * kThreads && FK * kWave == CH * kThreads, "staging");
  u32x4 kr[CH], vr[CH];
  // each thread's key row within a block, column offset and value offset (elements), added to
  // block-uniform bases, so a block's loads cost one clamp and one multiply-add per K chunk
  int krow[CH], kcol[CH], voff[CH];
#pragma unroll
  for (int u = 0; u < CH; ++u) {
    const int c = tid + u * kThreads, f = c / kWave, l = c % kWave;
    const int j = f / KS, sd = f - j * KS;
    krow[u] = 16 * j + (l & 15);
    kcol[u] = 32 * sd + 8 * (l >> 4);
    if constexpr (VTG)  // dim c / 8, positions 8 (c % 8) .. + 7 of the block
      voff[u] = (c / (KB / 8)) * vt_len + 8 * (c % (KB / 8));
    else  // key c % 64, dims 8 (c / 64) .. + 7
      voff[u] = (c % KB) * HD + (c / KB) * 8;
  }
  auto fetch = [&](int k0) {
    // keys past kend are clamped to the last usable one: their scores are masked to -inf and
    // their weights are 0, so only finiteness matters; transposed-value positions stay below
    // vt_len (zero past n)
    const bf16* kblk = Kb + (int64_t)k0 * HD;
    const int lim = kend - 1 - k0;
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      kr[u] = ld16(kblk + (uint32_t)(min(krow[u], lim) * HD + kcol[u]));
      if constexpr (VTG)
        vr[u] = ld16(VTb + k0 + (uint32_t)voff[u]);
      else
        vr[u] = ld16(Vb + (int64_t)min(k0 + (tid + u * kThreads) % KB, kend - 1) * HD +
                     ((tid + u * kThreads) / KB) * 8);
    }
  };
  if (kbeg < kend) fetch(kbeg);
  for (int k0 = kbeg, buf = 0; k0 < kend; k0 += KB, buf ^= 1) {
    // buffer `buf` was last read two blocks ago, before the previous block's barrier
#pragma unroll
    for (int u = 0; u < CH; ++u) {
      const int c = tid + u * kThreads;
      ks[buf][c / kWave][c % kWave] = kr[u];
      if constexpr (VTG) {
        *reinterpret_cast<u32x4*>(&vt[buf][c / (KB / 8)][8 * (c % (KB / 8))]) = vr[u];
      } else {
        const int kk = c % KB, dd = (c / KB) * 8;
        const bf16x8 v8 = __builtin_bit_cast(bf16x8, vr[u]);
        const int kp = vt_pos(kk);
#pragma unroll
        for (int i = 0; i < 8; ++i) vt[buf][dd + i][kp] = v8[i];
      }
    }
    __syncthreads();
    if (k0 + KB < kend) fetch(k0 + KB);
    // S^T for the NT 16-key tiles of every query tile, started at -mb: the queries carry the
    // softmax scale times log2(e), so st = log2-unit score - mb, the exponent of the weight
    f32x4 st[QT][NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = __builtin_bit_cast(bf16x8, ks[buf][j * KS + s][lane]);
#pragma unroll
        for (int t = 0; t < QT; ++t)
          st[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t][s].v,
                                                             s == 0 ? cinit[t] : st[t][j], 0, 0, 0);
      }
    }
    // V^T fragments of this block, read now so that the LDS latency overlaps the softmax:
    // row 16 c + lane % 16 of V^T, the 8 keys of this lane's P order in k-step h (tile 2h keys
    // 4g..4g+3, then tile 2h+1 keys 4g..4g+3), adjacent in the permuted key order
    bf16x8 vf[VT][PK];
#pragma unroll
    for (int c = 0; c < VT; ++c)
#pragma unroll
      for (int h = 0; h < PK; ++h)
        vf[c][h] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(&vt[buf][16 * c + (lane & 15)][32 * h + 8 * g]));
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      const int qt0 = qw + 16 * t;  // first query of the tile
      // mask, unless every key of the block is valid for every query of the tile: all keys
      // exist, none is later than the tile's first query, none falls out of the window of its
      // last
      const bool interior =
          k0 + KB <= kend && k0 + KB - 1 <= qt0 && (W <= 0 || k0 > qt0 + 15 - W);
      if (!interior) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int key = k0 + 16 * j + 4 * g + i;
            const bool ok = key <= tq[t] && key < kend && (W <= 0 || key > tq[t] - W);
            st[t][j][i] = ok ? st[t][j][i] : -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][j][i]);
      // The weights are exp2(score - mref) (log2 units) against a reference mref that only moves
      // when some query's block maximum exceeds it by more than 8, so a weight is at most 2^8 and
      // the accumulators are rescaled only on those blocks; the result is the same softmax (the
      // reference cancels between numerator and denominator). mb = mref, or 0 while a query has
      // no key yet (mref = -inf: its weights are exp2(-inf) = 0, and its first usable block moves
      // the reference). st holds score - mb; a block that moves a reference shifts st by the
      // change. The four lanes of a query (lane % 16 equal) share its reference: the test uses
      // each lane's own keys, and a block that moves some reference first takes each query's
      // maximum over its four lanes. Every wave runs the same MFMAs, so no lane leaves the loop
      // early.
      if (__ballot(mx > thr[t]) != 0) {
        mx = max_xor16_32(mx);
        const float mb = mref[t] == -INFINITY ? 0.f : mref[t];
        const float mr = fmaxf(mref[t], mx + mb);
        const float alpha = mr == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(mref[t] - mr);
#pragma unroll
        for (int c = 0; c < VT; ++c) acc[t][c] *= alpha;
        lsum[t] *= alpha;
        mref[t] = mr;
        const float mb_new = mr == -INFINITY ? 0.f : mr, shift = mb - mb_new;
#pragma unroll
        for (int j = 0; j < NT; ++j) st[t][j] += shift;
        cinit[t] = f32x4{-mb_new, -mb_new, -mb_new, -mb_new};
        thr[t] = mr == -INFINITY ? -INFINITY : 8.f;
      }
      bf16x8 pb[PK];
#pragma unroll
      for (int e = 0; e < 4 * NT; ++e)
        pb[e / 8][e % 8] = (bf16)__builtin_amdgcn_exp2f(st[t][e / 4][e % 4]);
      // the row sums of the weights as they are multiplied (bf16), by the matrix cores: every
      // row of ones x P^T is the per-query sum
#pragma unroll
      for (int h = 0; h < PK; ++h)
        lsum[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[h], lsum[t], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < VT; ++c)
#pragma unroll
        for (int h = 0; h < PK; ++h)
          acc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[c][h], pb[h], acc[t][c], 0, 0, 0);
    }
  }
  const int d = H * HD;
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    if (tq[t] >= n) continue;
    const float inv = 1.f / lsum[t][0];
    const int row = b * n + tq[t];
#pragma unroll
    for (int c = 0; c < VT; ++c) {
      // lane holds O^T[dim 16 c + 4 g + i][query tq]
      const int dim = hh * HD + 16 * c + 4 * g;
      uint2 w;
      bf16 v4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v4[i] = (bf16)(acc[t][c][i] * inv);
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, v4[0]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, v4[1]) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, v4[2]) |
            ((uint32_t)__builtin_bit_cast(uint16_t, v4[3]) << 16);
      *reinterpret_cast<uint2*>(o + frag_off(row, dim, d / 32)) = w;
    }
  }
}

// ---- values transposed for the prefix attention ----------------------------------------------------
// vt[bh][dd][p] = v[bh][vt_key(p)][dd] for keys < n, 0 for n <= key < vt_len (vt_len a multiple of
// 64; keys permuted within groups of 32 as the P V product takes them). One workgroup per (bh,
// 64-key tile): 64 x HD elements through LDS, 16-byte loads and stores.
template <int HD>
__global__ __launch_bounds__(kThreads) void k_transpose_v(const bf16* __restrict__ v,
                                                          int64_t bh_stride, int n, int vt_len,
                                                          bf16* __restrict__ vt) {
  __shared__ __attribute__((aligned(16))) bf16 t[64][HD + 8];
  const int tiles = vt_len / 64;
  const int64_t bh = blockIdx.x / tiles;
  const int j0 = (int)(blockIdx.x % tiles) * 64;
  const bf16* src = v + bh * bh_stride;
  for (int c = threadIdx.x; c < 64 * HD / 8; c += kThreads) {
    const int j = c / (HD / 8), dd = 8 * (c % (HD / 8));
    const u32x4 r = j0 + j < n ? ld16(src + (int64_t)(j0 + j) * HD + dd) : u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&t[j][dd]) = r;
  }
  __syncthreads();
  bf16* dst = vt + bh * HD * vt_len + j0;
  for (int c = threadIdx.x; c < HD * 8; c += kThreads) {
    const int dd = c / 8, j = 8 * (c % 8);
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = t[vt_key(j + i)][dd];
    st16(dst + (int64_t)dd * vt_len + j, __builtin_bit_cast(u32x4, o));
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

// ---- the causal encoder: embedding gather and the output norm -----------------------------------
// x_0 = E[token] for every row (b, i) of the R = B n rows, widened to fp32; ids outside
// [0, V) embed as zero rows.
__global__ __launch_bounds__(kThreads) void k_embed(const int32_t* __restrict__ tok,
                                                    const bf16* __restrict__ E, int d, int V,
                                                    int64_t total, float* __restrict__ h) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / d;
  const int c = (int)(i - row * d);
  const int t = tok[row];
  h[i] = t >= 0 && t < V ? (float)E[(int64_t)t * d + c] : 0.f;
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
  p.vt = take((size_t)B * d * ((n + 63) / 64 * 64 + 64) * 2);  // values transposed, one group
  p.ssq = take(R * (d / 64 + 1) * 4);  // per-row partial sums of squares (64 columns each), 1/rms
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
                            const AL& al, const EP& ep, double out_bytes,
                            bool force_big = false) {
  constexpr bool kFrag = std::is_same<AL, PA>::value, kTok = std::is_same<AL, PTokens>::value;
  if constexpr (kFrag || kTok) {
    // the 256 x 256 kernel when it has at least one workgroup per compute unit (always when
    // force_big: epilogues that write the next norm's operand exist only in its layout);
    // token rows (PTokens) are read by it directly when each row is exactly K wide
    bool rows_ok = true;
    if constexpr (kTok) rows_ok = al.d == K;
    if (N % 256 == 0 && wks >= K / 32 && rows_ok &&
        (force_big || (int64_t)((R + 255) / 256) * (N / 256) >= 256)) {
      const int64_t blocks = (int64_t)((R + 255) / 256) * (N / 256);
      if (K % 32 != 0 || blocks <= 0 || blocks > INT32_MAX) return hipErrorInvalidValue;
      Exec x(c.st);
      hipError_t e = c.arm(RLT_K_PAR_GEMM, 2.0 * ((double)R * K + (double)K * N) + out_bytes,
                           2.0 * R * N * K, x);
      if (e != hipSuccess) return e;
      if constexpr (kTok)
        return launch(k_gemm_big<EP, true>, dim3((unsigned)blocks), dim3(kBigThreads), x, N,
                      K / 32, al.e, R, static_cast<const bf16*>(Wt), wks, ep,
                      ATok{al.e_seq, al.n});
      else
        return launch(k_gemm_big<EP, false>, dim3((unsigned)blocks), dim3(kBigThreads), x, N,
                      K / 32, al.a, R, static_cast<const bf16*>(Wt), wks, ep, ATok{0, 1});
    }
  }
  if constexpr (kFrag) {
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

// k_flash takes its queries times the softmax scale 1/sqrt(hd) and log2(e) (scores in log2
// units); the projections that write them apply this factor before rounding to bf16.
static float flash_qscale(int hd) { return 1.4426950408889634f / sqrtf((float)hd); }

// W > 0: window attention (keys t-W+1..t of this layer); W = 0: memory prefix 0..t. q holds the
// queries times flash_qscale(hd).
template <int HD>
static hipError_t flash_t(const ParCtx& c, const bf16* q, const bf16* k, const bf16* v,
                          int64_t kv_bh_stride, int B, int n, int H, int W, bf16* o,
                          bf16* vt, bool vt_fresh) {
  // 16-query tiles per wave: with the transposed values (memory prefix, W = 0) two at hd = 64,
  // each K / V fragment read from LDS serving both (22.8-22.9 against 25.9-26.0 ms of memory
  // attention per pass at 200 registers and half the resident waves; the VALU work per key
  // block, its staging and addressing, is shared by twice the queries; four take 423 registers,
  // one wave per SIMD: 46.3-46.8 ms); one for the window,
  // whose 128-query blocks would cover 1.5x the keys they use (3.2 against 2.6 ms), and at
  // hd = 128, where two do not fit in 256 registers
  constexpr int QTV = HD == 64 ? 2 : 1;
  const int QT = vt ? QTV : 1;
  const int qblocks = (n + 64 * QT - 1) / (64 * QT);
  const int64_t blocks = (int64_t)B * H * qblocks;
  const int vt_tiles = (n + 63) / 64 + 1;  // with the spare tile
  if (blocks > INT32_MAX || (int64_t)B * H * vt_tiles > INT32_MAX) return hipErrorInvalidValue;
  // keys per query summed over t = 0..n-1: min(t + 1, W) or t + 1
  double keys = 0;
  if (W > 0) {
    const double full = n > W ? (double)(n - W) : 0.0, ramp = n < W ? n : W;
    keys = full * W + ramp * (ramp + 1) / 2;
  } else {
    keys = (double)n * (n + 1) / 2;
  }
  const double bhd = (double)B * H * HD;
  // one spare (zero) tile per row: rows are then not a power-of-two multiple of 128 bytes apart,
  // so the rows a block reads spread over the L2 channels
  const int vt_len = vt_tiles * 64;
  hipError_t e;
  if (vt && !vt_fresh) {  // values transposed first (timed as its own kind)
    Exec xt(c.st);
    if ((e = c.arm(RLT_K_PAR_OTHER, bhd * (n + vt_len) * 2, 0, xt)) != hipSuccess) return e;
    e = launch(k_transpose_v<HD>, dim3((unsigned)((int64_t)B * H * vt_tiles)), dim3(kThreads), xt,
               v, kv_bh_stride, n, vt_len, vt);
    if (e != hipSuccess) return e;
  }
  Exec x(c.st);
  if ((e = c.arm(W > 0 ? RLT_K_PAR_SELF : RLT_K_PAR_CROSS, bhd * n * 2 * 4.0, 4.0 * bhd * keys,
                 x)) != hipSuccess)
    return e;
  if (vt)
    return launch(k_flash<HD, QTV, true>, dim3((unsigned)blocks), dim3(kThreads), x, q, k, v,
                  kv_bh_stride, n, H, W, qblocks, static_cast<const bf16*>(vt), vt_len, o);
  return launch(k_flash<HD, 1, false>, dim3((unsigned)blocks), dim3(kThreads), x, q, k, v,
                kv_bh_stride, n, H, W, qblocks, static_cast<const bf16*>(nullptr), 0, o);
}

// vt (optional): workspace of B H hd ceil(n / 64) 64 elements for the values transposed first;
// vt_fresh: it already holds these values transposed (the same memory group as the last call)
static hipError_t flash(const ParCtx& c, int hd, const bf16* q, const bf16* k, const bf16* v,
                        int64_t kv_bh_stride, int B, int n, int H, int W, bf16* o,
                        bf16* vt = nullptr, bool vt_fresh = false) {
  switch (hd) {
    case 32: return flash_t<32>(c, q, k, v, kv_bh_stride, B, n, H, W, o, vt, vt_fresh);
    case 64: return flash_t<64>(c, q, k, v, kv_bh_stride, B, n, H, W, o, vt, vt_fresh);
    case 128: return flash_t<128>(c, q, k, v, kv_bh_stride, B, n, H, W, o, vt, vt_fresh);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t norm_rows(const ParCtx& c, const Dims& D, const float* h, const float* gamma,
                            int R, bf16* a) {
  const int per = kThreads / kWave;
  Exec x(c.st);
  hipError_t e = c.arm(RLT_K_PAR_OTHER, (double)R * D.d * 6, 4.0 * R * D.d, x);
  if (e != hipSuccess) return e;
  return launch(k_norm_rows<true>, dim3((unsigned)((R + per - 1) / per)), dim3(kThreads), x, h,
                gamma, D.d, D.eps, R, a);
}

// The RMSNorm before a projection is folded around it when the residual projection before it
// can write the operand (d a multiple of 256, so every projection with N = d runs k_gemm_big):
// the producer stores bf16(h * gamma) and per-row sums of squares, the consumer scales its
// output rows by 1/rms. Otherwise a k_norm_rows launch writes the normalised operand.
static bool norm_folds(const Dims& D) { return D.d % 256 == 0; }

// 1/rms of every row from the partial sums the last residual projection left in ssq; returns
// the consumer's RowScale (rinv sits after the R * d / 64 partial sums).
static hipError_t row_scale(const ParCtx& c, const Dims& D, int R, float* ssq, RowScale* rs) {
  float* rinv = ssq + (int64_t)R * (D.d / 64);
  Exec x(c.st);
  hipError_t e = c.arm(RLT_K_PAR_OTHER, (double)R * (D.d / 64 + 1) * 4, 0, x);
  if (e != hipSuccess) return e;
  e = launch(k_row_rinv, dim3((unsigned)((R + kThreads - 1) / kThreads)), dim3(kThreads), x,
             (const float*)ssq, D.d / 64, 1.f / (float)D.d, D.eps, R, rinv);
  rs->rinv = rinv;
  return e;
}

// PResidual for h += x W; when the next RMSNorm (gain gnext) is folded, it also writes that
// norm's operand into a and the row sums of squares into ssq.
static PResidual residual(const Dims& D, float* h, float* out, int64_t out_seq, int n, int R,
                          const float* gnext, bf16* a, float* ssq) {
  PResidual ep;
  ep.h = h;
  ep.out = out;
  ep.out_seq = out_seq;
  ep.n = n;
  ep.d = D.d;
  ep.R = R;
  if (gnext) {
    ep.hg = a;
    ep.gnext = gnext;
    ep.ssq_out = ssq;
  }
  return ep;
}

hipError_t launch_memproj_rows(const Dims& D, int B, const Packed& P, const MemBufs& M,
                               const void* e, int64_t e_seq, int64_t t0, int64_t n,
                               const Exec& st) {
  const int64_t rows = (int64_t)B * n;
  const int N = D.G * 2 * D.d;
  const int64_t blocks = (rows + 255) / 256 * (N / 256);
  if (D.dtype != RLT_BF16 || N % 256 != 0 || rows > INT32_MAX / 2 || blocks > INT32_MAX)
    return hipErrorInvalidValue;
  PMemproj ep;
  ep.mk = static_cast<bf16*>(M.k);
  ep.mv = static_cast<bf16*>(M.v);
  ep.cap = M.capacity;
  ep.t0 = t0;
  ep.n = (int)n;
  ep.B = B;
  ep.d = D.d;
  ep.H = D.H;
  ep.hd = D.hd;
  ep.R = (int)rows;
  return launch(k_gemm_big<PMemproj, true>, dim3((unsigned)blocks), dim3(kBigThreads), st, N,
                D.d / 32, static_cast<const bf16*>(e), (int)rows,
                static_cast<const bf16*>(P.wm_t), D.d / 32, ep, ATok{e_seq, (int)n});
}

hipError_t launch_readout_rows(const Dims& D, int B, const HeadBufs& Hd, const float* s, void* a,
                               float* logits, hipStream_t st) {
  const int V = Hd.vocab, d = D.d;
  if (D.dtype != RLT_BF16 || V % 256 != 0 || B < 1) return hipErrorInvalidValue;
  const ParCtx c{st, nullptr};
  bf16* ab = static_cast<bf16*>(a);
  hipError_t e = norm_rows(c, D, s, Hd.out_gamma, B, ab);
  if (e != hipSuccess) return e;
  PStoreF32 ep;
  ep.out = logits;
  ep.ld = V;
  ep.R = B;
  return gemm_rows(c, B, V, d, d / 32, Hd.w_out_t, PA{ab, d / 32, B}, ep, (double)B * V * 4);
}

hipError_t launch_encode(const Dims& D, int B, int64_t n_, const Packed& P, const HeadBufs& Hd,
                         const int32_t* tokens, void* e_out, void* ws, hipStream_t st) {
  if (D.dtype != RLT_BF16 || n_ < 1 || (int64_t)B * n_ > INT32_MAX / 2) return hipErrorInvalidValue;
  const ParCtx c{st, nullptr};
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
  hipError_t err;
  const int64_t total = (int64_t)R * d;
  err = launch(k_embed, dim3((unsigned)((total + kThreads - 1) / kThreads)), dim3(kThreads),
               Exec(st), tokens, static_cast<const bf16*>(Hd.embed), d, Hd.vocab, total, h);
  if (err != hipSuccess) return err;
  const bool fold = norm_folds(D);
  float* ssq = reinterpret_cast<float*>(w + Lp.ssq);
  for (int l = 0; l < D.L; ++l) {
    const float* gam = Hd.enc_gamma + (int64_t)l * 2 * d;
    const int64_t wdd = (int64_t)l * d * d;
    // causal self-attention over positions 1..t with the decoder block's matrices; its norm
    // is folded from the previous block's down projection except in the first block
    const bool norm_attn = !fold || l == 0;
    if (norm_attn && (err = norm_rows(c, D, h, gam, R, a)) != hipSuccess) return err;
    {
      PHeads ep{{}, {}, q, kk, vv, n, d, H, hd, R};
      ep.qscale = flash_qscale(hd);
      if (!norm_attn && (err = row_scale(c, D, R, ssq, &ep)) != hipSuccess) return err;
      const bf16* Wq = static_cast<const bf16*>(P.wqkv_t) + (int64_t)l * 3 * d * d;
      if ((err = gemm_rows(c, R, 3 * d, d, d / 32, Wq, PA{a, d / 32, R}, ep, Rd * 6)) !=
          hipSuccess)
        return err;
    }
    if ((err = flash(c, hd, q, kk, vv, (int64_t)n * hd, B, n, H, 0, o,
                     reinterpret_cast<bf16*>(w + Lp.vt))) != hipSuccess)
      return err;
    {
      const PResidual ep = residual(D, h, nullptr, 0, n, R, fold ? gam + d : nullptr, a, ssq);
      const bf16* Wo = static_cast<const bf16*>(P.wo_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wo, PA{o, d / 32, R}, ep, Rd * 8, fold)) !=
          hipSuccess)
        return err;
    }
    // SiLU-gated FFN with the decoder block's matrices
    if (!fold && (err = norm_rows(c, D, h, gam + d, R, a)) != hipSuccess) return err;
    {
      PSilu ep{{}, act, F, R};
      if (fold && (err = row_scale(c, D, R, ssq, &ep)) != hipSuccess) return err;
      const bf16* W13 = static_cast<const bf16*>(P.w13_t) + (int64_t)l * 2 * F * d;
      if ((err = gemm_rows(c, R, 2 * F, d, d / 32, W13, PA{a, d / 32, R}, ep,
                           (double)R * F * 2)) != hipSuccess)
        return err;
    }
    {
      const float* gnext = fold && l + 1 < D.L ? gam + 2 * d : nullptr;
      const PResidual ep = residual(D, h, nullptr, 0, n, R, gnext, a, ssq);
      const bf16* W2 = static_cast<const bf16*>(P.w2_t) + (int64_t)l * d * F;
      if ((err = gemm_rows(c, R, d, F, F / 32, W2, PA{act, F / 32, R}, ep, Rd * 8, fold)) !=
          hipSuccess)
        return err;
    }
  }
  const int per = kThreads / kWave;
  // e = the final norm's output, row-major (the layout rlt_memproj and the gate read)
  return launch(k_norm_rows<false>, dim3((unsigned)((R + per - 1) / per)), dim3(kThreads),
                Exec(st), (const float*)h, Hd.enc_gamma_out, d, D.eps, R,
                static_cast<bf16*>(e_out));
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
  const bool fold = norm_folds(D);
  float* ssq = reinterpret_cast<float*>(w + Lp.ssq);
  for (int l = 0; l < D.L; ++l) {
    const bool last = l == D.L - 1;
    const float* gam = P.gamma + (int64_t)l * 3 * d;
    const int64_t wdd = (int64_t)l * d * d;
    // self-attention sublayer; its norm is folded from the previous block's down projection
    // except in the first block
    const bool norm_attn = !fold || l == 0;
    if (norm_attn && (err = norm_rows(c, D, h, gam, R, a)) != hipSuccess) return err;
    {
      PHeads ep{{}, {}, q, kk, vv, n, d, H, hd, R};
      ep.qscale = flash_qscale(hd);
      if (!norm_attn && (err = row_scale(c, D, R, ssq, &ep)) != hipSuccess) return err;
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
      const PResidual ep = residual(D, h, nullptr, 0, n, R, fold ? gam + d : nullptr, a, ssq);
      const bf16* Wo = static_cast<const bf16*>(P.wo_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wo, PA{o, d / 32, R}, ep, Rd * 8, fold)) !=
          hipSuccess)
        return err;
    }
    // cross-attention sublayer: memory entries 1..t of this layer's group
    if (!fold && (err = norm_rows(c, D, h, gam + d, R, a)) != hipSuccess) return err;
    {
      PHeads ep{{}, {}, q, nullptr, nullptr, n, d, H, hd, R};
      ep.qscale = flash_qscale(hd);
      if (fold && (err = row_scale(c, D, R, ssq, &ep)) != hipSuccess) return err;
      const bf16* Wc = static_cast<const bf16*>(P.wcq_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wc, PA{a, d / 32, R}, ep, Rd * 2)) !=
          hipSuccess)
        return err;
    }
    {
      const int gsel = D.G == 1 ? 0 : l;
      const int64_t grp = (int64_t)gsel * M.Bt * H * M.capacity * hd;
      // with one memory group for every layer its values are transposed once
      if ((err = flash(c, hd, q, static_cast<const bf16*>(M.k) + grp,
                       static_cast<const bf16*>(M.v) + grp, M.capacity * hd, B, n, H, 0, o,
                       reinterpret_cast<bf16*>(w + Lp.vt), D.G == 1 && l > 0)) != hipSuccess)
        return err;
    }
    {
      const PResidual ep =
          residual(D, h, nullptr, 0, n, R, fold ? gam + 2 * d : nullptr, a, ssq);
      const bf16* Wco = static_cast<const bf16*>(P.wco_t) + wdd;
      if ((err = gemm_rows(c, R, d, d, d / 32, Wco, PA{o, d / 32, R}, ep, Rd * 8, fold)) !=
          hipSuccess)
        return err;
    }
    // FFN sublayer
    if (!fold && (err = norm_rows(c, D, h, gam + 2 * d, R, a)) != hipSuccess) return err;
    {
      PSilu ep{{}, act, F, R};
      if (fold && (err = row_scale(c, D, R, ssq, &ep)) != hipSuccess) return err;
      const bf16* W13 = static_cast<const bf16*>(P.w13_t) + (int64_t)l * 2 * F * d;
      if ((err = gemm_rows(c, R, 2 * F, d, d / 32, W13, PA{a, d / 32, R}, ep,
                                 (double)R * F * 2)) != hipSuccess)
        return err;
    }
    {
      const float* gnext = fold && !last ? gam + 3 * d : nullptr;  // the next block's first gain
      const PResidual ep = residual(D, h, last ? out : nullptr, out_seq, n, R, gnext, a, ssq);
      const bf16* W2 = static_cast<const bf16*>(P.w2_t) + (int64_t)l * d * F;
      if ((err = gemm_rows(c, R, d, F, F / 32, W2, PA{act, F / 32, R}, ep,
                                 Rd * (last && out ? 12 : 8), fold)) != hipSuccess)
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
