// Backpropagation through time of the decoder on gfx950: a forward pass over the whole sequence
// that keeps what the reverse walk needs, then the reverse walk over the tokens.
//
// "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", section "Training and serving
// implications": pretraining backpropagates through the full sequence, and the gradient of one
// state with respect to the previous one also runs through the self-attention keys and values
// of the window, not only through s_t. The walk below therefore carries two kinds of gradient
// from token t+1 back to token t: dLoss/ds_t through the next gated merge, and, per layer, the
// gradients of every key/value still inside a later token's window (fp32 accumulators in a
// ring of W slots). Memory keys/values collect gradients from every later token; those sums are
// formed after the walk by a token-parallel pass over each memory entry.
//
// Per token and layer the walk runs, newest layer first (dres = gradient of the residual stream):
//   FFN      recompute u = f [W1 W3] (f = RMSNorm(z)), dm = dres W2^T, du from the SiLU product,
//            df = du [W1 W3]^T, dres += RMSNorm'(z) df
//   cross    doc = dres Wco^T, dqc from one online pass over memory 0..t, dc = dqc Wcq^T,
//            dres += RMSNorm'(y) dc
//   self     do = dres Wo^T, dq and the window's key/value gradients from two passes over the
//            window, da = [dq dk dv] [Wq Wk Wv]^T, dres += RMSNorm'(x) da
// and then the gated merge (dLoss/de_t and the gradient carried to s_{t-1}). The per-token
// GEMMs are the decoder step's split-K projections (k_proj) against transposed copies of the
// packed weights. Weight gradients are sums over all (token, sequence) rows of x^T dy; the walk
// stores both operands for Tc tokens at a time and adds them in large MFMA GEMMs per chunk.
#include <math.h>

#include "proj.h"

namespace rlt {

// ---- workspace -------------------------------------------------------------------------------
namespace {
constexpr size_t kAlignWs = 256;
constexpr int kRowSplits = 32;  // row splits of the deterministic column sums
constexpr int kChunkRows = 4096;
size_t up(size_t x) { return (x + kAlignWs - 1) / kAlignWs * kAlignWs; }

// Backward copies of the packed weights, in elements from the start of the bw region:
// every matrix stored input-major (rows = input features of the forward map) in fragment order.
struct BwOff {
  size_t wg, wqkv, wo, wcq, wco, w13, w2, wm, total;
};
BwOff bw_off(const Dims& D) {
  const size_t d = D.d, F = D.F, L = D.L, G = D.G;
  BwOff o;
  o.wg = 0;                        // [2d][d]   rows: e then u features; k: gate outputs
  o.wqkv = o.wg + 2 * d * d;       // [L][d][3d] k: q, k, v outputs
  o.wo = o.wqkv + L * 3 * d * d;   // [L][d][d]
  o.wcq = o.wo + L * d * d;
  o.wco = o.wcq + L * d * d;
  o.w13 = o.wco + L * d * d;       // [L][d][2F] k: W1 outputs, then W3 outputs
  o.w2 = o.w13 + L * 2 * F * d;    // [L][F][d]
  o.wm = o.w2 + L * F * d;         // [G][d][2d] k: memory key outputs, then value outputs
  o.total = o.wm + G * 2 * d * d;
  return o;
}
}  // namespace

TrainLayout train_layout(const Dims& D, int B, int64_t n) {
  TrainLayout t;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t a = o;
    o = up(o + bytes);
    return a;
  };
  const size_t b = B, d = D.d, F = D.F, L = D.L, H = D.H, es = D.es, N = (size_t)n;
  t.Tc = std::max<int64_t>(1, std::min<int64_t>(n, (kChunkRows + B - 1) / B));
  t.Mc = t.Tc * B;
  const size_t Mc = (size_t)t.Mc;
  t.state = take(state_layout(D, B).total);
  t.mem_k = take((size_t)D.G * b * N * d * es);
  t.mem_v = take((size_t)D.G * b * N * d * es);
  t.bw = take(bw_off(D).total * es);
  t.s_hist = take((N + 1) * b * d * 4);
  const size_t act = L * N * b * d;
  t.xs = take(act * 4);
  t.ys = take(act * 4);
  t.zs = take(act * 4);
  t.qs = take(act * 4);
  t.qcs = take(act * 4);
  t.os = take(act * es);
  t.ocs = take(act * es);
  t.docs = take(act * es);
  t.khist = take(act * es);
  t.vhist = take(act * es);
  t.lse = take(L * N * b * H * 4);
  t.dlt = take(L * N * b * H * 4);
  t.dres = take(b * d * 4);
  t.dn = take(b * d * 4);
  t.dattn = take(b * d * 4);
  t.u13 = take(L * N * b * 2 * F * 4);  // the forward's up-projections u1 | u3, [L][n][B][2F]
  t.gsave = take(b * d * 4);
  t.carry = take(b * d * 4);
  t.rinv = take(b * 3 * 4);
  t.dkacc = take(L * D.W * b * d * es);      // window-backward rings: do of the last W tokens
  t.dvacc = take(2 * L * D.W * b * H * 4);  // and their lse, D
  // per-chunk operand rows of the weight gradients, twice: the walk fills one copy while the
  // gradients of the previous chunk read the other
  const size_t c0 = o;
  t.ca = take(L * Mc * d * es);
  t.cc = take(L * Mc * d * es);
  t.cf = take(L * Mc * d * es);
  t.cm = take(L * Mc * F * es);
  t.yqkv = take(L * Mc * 3 * d * es);
  t.yo = take(L * Mc * d * es);
  t.ycq = take(L * Mc * d * es);
  t.yco = take(L * Mc * d * es);
  t.y13 = take(L * Mc * 2 * F * es);
  t.y2 = take(L * Mc * d * es);
  t.pg = take((3 * L + 1) * Mc * d * 4);
  t.xg = take(Mc * 2 * d * es);
  t.yg = take(Mc * d * es);
  t.cspan = o - c0;
  take(t.cspan);
  t.part = take((3 * L + 1) * kRowSplits * d * 4);
  t.dkv = take(b * N * 2 * d * es);
  // weight-gradient operands transposed to [features][rows] (rows padded to 32)
  const size_t Mp = (Mc + 31) / 32 * 32;
  t.o2 = take((b + 15) / 16 * 16 * d * es);  // second attention-output operand (forward)
  // (one matrix per layer: the weight gradients of all layers are formed in one batch)
  t.tx = take(L * Mp * std::max(2 * d, F) * es);
  t.ty = take(L * Mp * std::max(3 * d, 2 * F) * es);
  t.total = o;
  return t;
}

// ---- small kernels ---------------------------------------------------------------------------

// Transposes a packed forward matrix (rows = N outputs, k = K inputs, fragment order) into the
// backward layout (rows = K inputs, k = N outputs). With w13 set the source rows interleave W1
// and W3 in blocks of 16 and the destination k runs over all W1 outputs, then all W3 outputs.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_repack(const T* __restrict__ src, int N, int K,
                                                     T* __restrict__ dst, int w13, int F,
                                                     int64_t mats) {
  const int64_t per = (int64_t)N * K;
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= per * mats) return;
  const int64_t mi = i / per;
  const int64_t r = i - mi * per;
  const int k = (int)(r / N), c = (int)(r - (int64_t)k * N);  // dst row k (input), column c
  int row = c;                                                  // source row (output)
  if (w13) {
    const int which = c / F, f = c - which * F;
    row = 32 * (f / 16) + 16 * which + f % 16;
  }
  dst[mi * per + frag_off(k, c, N / 32)] = src[mi * per + frag_off(row, k, K / 32)];
}

// dst rows [B][d] = s* (the state before the first token).
__global__ __launch_bounds__(kThreads) void k_fill_start(float* __restrict__ dst,
                                                         const float* __restrict__ s_star, int d,
                                                         int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < total) dst[i] = s_star[i % d];
}

// Copies of the forward's working buffers that the reverse walk keeps (the residual streams and
// the queries are written straight into their save slots by the forward's own kernels):
//   stage 0 (after the gated merge): x = h of layer 0
//   stage 1 (after a layer's cross-attention output projection): the self-attention output o
//           and the cross-attention output oc (fragment order -> rows), and this token's
//           key/value ring slot -> the key/value history
struct SaveArgs {
  int stage, B, d, H, hd, W;
  int64_t n, i;
  const float* h;
  float* h_dst;        // [B][d] rows of token i
  const void* o;       // fragment order [B16][d]
  const void* oc;
  void* o_dst;         // row-major [B][d]
  void* oc_dst;
  const void* ring_k;  // this layer's ring block [B][H][W][hd]
  const void* ring_v;
  void* k_dst;         // this layer's history block [B][H][n][hd]
  void* v_dst;
};

template <typename T>
__global__ __launch_bounds__(kThreads) void k_save(SaveArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)a.B * a.d) return;
  if (a.stage == 0) {
    a.h_dst[idx] = a.h[idx];
    return;
  }
  const int b = (int)(idx / a.d), c = (int)(idx - (int64_t)b * a.d);
  const int64_t f = frag_off(b, c, a.d / 32);
  static_cast<T*>(a.o_dst)[idx] = static_cast<const T*>(a.o)[f];
  static_cast<T*>(a.oc_dst)[idx] = static_cast<const T*>(a.oc)[f];
  const int hh = c / a.hd, dd = c - hh * a.hd;
  const int64_t ring = (((int64_t)b * a.H + hh) * a.W + (int)(a.i % a.W)) * a.hd + dd;
  const int64_t hist = (((int64_t)b * a.H + hh) * a.n + a.i) * a.hd + dd;
  static_cast<T*>(a.k_dst)[hist] = static_cast<const T*>(a.ring_k)[ring];
  static_cast<T*>(a.v_dst)[hist] = static_cast<const T*>(a.ring_v)[ring];
}

// s_traj[b][i] = s_hist[i + 1][b]
__global__ __launch_bounds__(kThreads) void k_traj(const float* __restrict__ s_hist,
                                                   float* __restrict__ out, int B, int64_t n,
                                                   int d) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= (int64_t)B * n * d) return;
  const int c = (int)(idx % d);
  const int64_t rest = idx / d;
  const int64_t i = rest % n;
  const int b = (int)(rest / n);
  out[idx] = s_hist[((i + 1) * B + b) * d + c];
}

// The three RMSNorm outputs of one layer of one token, recomputed for the reverse walk from the
// saved residual streams: a = gain0 x r_x, c = gain1 y r_y, f = gain2 z r_z (dtype rows, the
// GEMM operands) and the scales r. x == NULL: nothing to do.
template <typename T>
struct NormRows {
  const float* x;
  const float* y;
  const float* z;
  const float* gamma;  // [3][d]
  T* a;
  T* c;
  T* f;
  float eps;
};

// Row b of NormRows, by one workgroup; rinv[b * 3 + w] receives the scales.
template <typename T>
__device__ void norm_rows3(const NormRows<T>& nr, int b, int d, float* __restrict__ rinv,
                           float* red) {
  const float* src[3] = {nr.x + (int64_t)b * d, nr.y + (int64_t)b * d, nr.z + (int64_t)b * d};
  T* dst[3] = {nr.a + (int64_t)b * d, nr.c + (int64_t)b * d, nr.f + (int64_t)b * d};
#pragma unroll
  for (int w = 0; w < 3; ++w) {
    float ss = 0.f;
    for (int j = threadIdx.x; j < d; j += kThreads) ss += src[w][j] * src[w][j];
    const float r = rsqrtf(block_sum(ss, red) / (float)d + nr.eps);
    for (int j = threadIdx.x; j < d; j += kThreads)
      dst[w][j] = to_elem<T>(nr.gamma[w * d + j] * src[w][j] * r);
    if (threadIdx.x == 0) rinv[b * 3 + w] = r;
  }
}

// Start of token i's walk, one workgroup per row: dres = G[:, i] + carry (carry = dLoss/ds_i
// through token i+1), its dtype copy (the operand of the FFN down-projection's backward), and
// the norm rows of the last layer.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_walk_begin(const float* __restrict__ G,
                                                         const float* __restrict__ carry,
                                                         float* __restrict__ dres,
                                                         T* __restrict__ dres_t, int d,
                                                         int64_t n, int64_t i, NormRows<T> nr,
                                                         float* __restrict__ rinv) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int64_t o = (int64_t)b * d;
  for (int j = threadIdx.x; j < d; j += kThreads) {
    const float v = G[((int64_t)b * n + i) * d + j] + (carry ? carry[o + j] : 0.f);
    dres[o + j] = v;
    dres_t[o + j] = to_elem<T>(v);
  }
  norm_rows3(nr, b, d, rinv, red);
}

// Backward of an RMSNorm y = gain * x * r at one row per workgroup, added to the residual
// gradient: dres += gain * dn * r - x * r^3 * sum(gain * dn * x) / d. Also writes dres in the
// working dtype (the next GEMM operand, when res_t != NULL) and the row's gain-gradient terms
// dn * x * r (fp32, summed over rows later); then, when nr.x != NULL, the norm rows of the
// layer below (which replace this layer's scales in rinv).
template <typename T>
__global__ __launch_bounds__(kThreads) void k_norm_back(const float* __restrict__ dn,
                                                        const float* __restrict__ x,
                                                        const float* __restrict__ gain,
                                                        float* __restrict__ rinv, int which,
                                                        int d, float* __restrict__ dres,
                                                        T* __restrict__ res_t,
                                                        float* __restrict__ pgain, NormRows<T> nr) {
  __shared__ float red[4];
  const int b = blockIdx.x;
  const int64_t o = (int64_t)b * d;
  const float r = rinv[b * 3 + which];
  float s = 0.f;
  for (int j = threadIdx.x; j < d; j += kThreads) s += gain[j] * dn[o + j] * x[o + j];
  const float inner = block_sum(s, red);
  const float k = r * r * r * inner / (float)d;
  for (int j = threadIdx.x; j < d; j += kThreads) {
    const float g = dn[o + j], xv = x[o + j];
    const float v = dres[o + j] + gain[j] * g * r - xv * k;
    dres[o + j] = v;
    if (res_t) res_t[o + j] = to_elem<T>(v);
    pgain[o + j] = g * xv * r;
  }
  if (nr.x) norm_rows3(nr, b, d, rinv, red);
}

// Column sums of nmat row-major [rows][d] fp32 matrices (matrix m at P + m * stride * d),
// deterministic: k_colsum_part sums kRowSplits row ranges, k_colsum_final adds the splits in
// order to the matrix's output.
__global__ __launch_bounds__(kThreads) void k_colsum_part(const float* __restrict__ P, int64_t rows,
                                                          int64_t stride, int d,
                                                          float* __restrict__ part) {
  const int m = blockIdx.z, split = blockIdx.y;
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= d) return;
  const int64_t per = (rows + kRowSplits - 1) / kRowSplits;
  const int64_t r0 = split * per, r1 = std::min<int64_t>(rows, r0 + per);
  const float* p = P + (int64_t)m * stride * d + c;
  float s = 0.f;
  for (int64_t r = r0; r < r1; ++r) s += p[r * d];
  part[((int64_t)m * kRowSplits + split) * d + c] = s;
}

struct ColOut {
  float* gamma;   // matrices 0 .. 3L-1 add into gamma + m * d
  float* extra;   // matrix 3L (if present) adds into extra
  int n_gamma;
};

__global__ __launch_bounds__(kThreads) void k_colsum_final(const float* __restrict__ part, int d,
                                                           ColOut out) {
  const int m = blockIdx.y;
  const int c = blockIdx.x * kThreads + threadIdx.x;
  if (c >= d) return;
  float s = 0.f;
  for (int k = 0; k < kRowSplits; ++k) s += part[((int64_t)m * kRowSplits + k) * d + c];
  float* dst = m < out.n_gamma ? out.gamma + (int64_t)m * d : out.extra;
  dst[c] += s;
}

// ---- per-token GEMM operands and epilogues -----------------------------------------------------

template <typename T>
struct ARows {  // A = row-major [M][ld] dtype rows
  static constexpr bool kNorm = false;
  static constexpr int kPer = sizeof(T) == 2 ? 1 : 2, kShared = 0;
  const T* a;
  int64_t ld;
  int M;
  __device__ void issue(int, int row, int step, int lane, u32x4* r) const {
    const T* p = a + (int64_t)row * ld + step * 32 + (lane >> 4) * 8;
    r[0] = ld16(p);
    if constexpr (kPer == 2) r[1] = ld16(p + 4);
  }
  __device__ void issue_shared(int, u32x4*) const {}
  __device__ Frag<T> make(const u32x4* r, const u32x4*) const {
    Frag<T> f;
    f.from_raw(r);
    return f;
  }
  // token-GEMM interface
  __device__ Frag<T> load(int row, int k, float&) const {
    Frag<T> f;
    if (row < M) f.load(a + (int64_t)row * ld + k);
    else f.zero();
    return f;
  }
};

// From the forward's u1 | u3: dm -> du1 = dm u3 sigma(u1) (1 + u1 (1 - sigma(u1))),
// du3 = dm silu(u1) (dtype rows [M][2F]), and the product m = silu(u1) u3 (dtype rows [M][F],
// the down projection's weight-gradient operand, as the forward rounded it).
template <typename T>
struct EpiSiluBack : EpiTile<EpiSiluBack<T>> {
  const float* u;
  T* du;
  T* m;
  int M, F;
  __device__ void op(int row, int col, float dm) const {
    if (row >= M) return;
    const float u1 = u[(int64_t)row * 2 * F + col], u3 = u[(int64_t)row * 2 * F + F + col];
    const float sg = sigmoidf_(u1);
    du[(int64_t)row * 2 * F + col] = to_elem<T>(dm * u3 * sg * (1.f + u1 * (1.f - sg)));
    du[(int64_t)row * 2 * F + F + col] = to_elem<T>(dm * u1 * sg);
    m[(int64_t)row * F + col] = to_elem<T>(u1 * sg * u3);
  }
};

// Gate recompute: v = [e ; u] W_g, g = sigmoid(v + b); dz = dres (e - u) g (1 - g). Writes dz
// (dtype and fp32 rows), g, and the gate operand [e ; u] (dtype rows [M][2d]).
template <typename T>
struct EpiGateBack : EpiTile<EpiGateBack<T>> {
  const T* e;
  int64_t lde;
  const float* s;  // s_{t-1} rows
  const float* b;
  const float* dres;
  float alpha;
  T* dz;
  float* dz32;
  float* g;
  T* xg;
  int M, d;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    const int64_t o = (int64_t)row * d + col;
    const float gv = sigmoidf_(v + b[col]);
    const float ev = to_f32<T>(e[(int64_t)row * lde + col]), uv = alpha * s[o];
    const float z = dres[o] * (ev - uv) * gv * (1.f - gv);
    dz[o] = to_elem<T>(z);
    dz32[o] = z;
    g[o] = gv;
    xg[(int64_t)row * 2 * d + col] = to_elem<T>(ev);
    xg[(int64_t)row * 2 * d + d + col] = to_elem<T>(uv);
  }
};

// [de_gate | du_gate] = dz W_g^T: de_t = dres g + de_gate, carry = alpha (dres (1 - g) + du_gate)
struct EpiGateOut : EpiTile<EpiGateOut> {
  const float* dres;
  const float* g;
  float* de;  // row b of token t (NULL: not wanted)
  int64_t de_ld;
  float* carry;
  float alpha;
  int M, d;
  __device__ void op(int row, int col, float v) const {
    if (row >= M) return;
    if (col < d) {
      const int64_t o = (int64_t)row * d + col;
      if (de) de[(int64_t)row * de_ld + col] = dres[o] * g[o] + v;
    } else {
      const int64_t o = (int64_t)row * d + (col - d);
      carry[o] = alpha * (dres[o] * (1.f - g[o]) + v);
    }
  }
};

// de += [dKm | dVm] [WmK | WmV]^T (token GEMM, register tiles)
struct EpiAddF32 {
  float* out;
  int64_t ld;
  int M;
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + 16 * fm + i;
          if (row < M) out[(int64_t)row * ld + cwave + 16 * fn + (lane & 15)] += acc[fm][fn][i];
        }
  }
};

// ---- attention backward of one token ----------------------------------------------------------

template <typename T, int HD>
struct AGeo {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int LPR = HD / VEC;
  static constexpr int RPW = kWave / LPR;
};

// Online state of one row slot for the backward of o = softmax(s) v with s_j = scale q.k_j:
// m = running max, l = sum e_j, c = sum e_j dp_j (dp_j = do.v_j), A = sum e_j dp_j k_j,
// Bk = sum e_j k_j, with e_j = exp(s_j - m). Then D = c / l = sum p_j dp_j and
// dq = scale (A - D Bk) / l.
template <int V>
struct BwdState {
  float m, l, c, A[V], Bk[V];
  __device__ void init() {
    m = -INFINITY;
    l = 0.f;
    c = 0.f;
#pragma unroll
    for (int i = 0; i < V; ++i) A[i] = Bk[i] = 0.f;
  }
  __device__ void merge(float mo, float lo, float co, const float* Ao, const float* Bo) {
    const float mn = fmaxf(m, mo);
    const float a = m == -INFINITY ? 0.f : __expf(m - mn);
    const float b = mo == -INFINITY ? 0.f : __expf(mo - mn);
    l = l * a + lo * b;
    c = c * a + co * b;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      A[i] = A[i] * a + Ao[i] * b;
      Bk[i] = Bk[i] * a + Bo[i] * b;
    }
    m = mn;
  }
};

// Cross-attention backward of token t (0-based) for one (sequence, head) per workgroup: keys
// and values are memory entries 0..t of the layer's group. Writes dq (dtype row-major, the
// query-projection backward's operand), lse = m + log l and D (for the memory gradients formed
// after the walk), and a dtype copy of do (same use).
template <typename T, int HD, int NW, int U>
__device__ __forceinline__ void xattn_back_body(
    const float* __restrict__ q, const float* __restrict__ dout, const T* __restrict__ K,
    const T* __restrict__ V, int64_t bh_stride, int ntok, int H, float scale,
    T* __restrict__ dq, float* __restrict__ lse, float* __restrict__ dlt, T* __restrict__ do_t) {
  using G = AGeo<T, HD>;
  constexpr int VEC = G::VEC, RPB = G::RPW * NW;
  __shared__ float s_m[NW], s_l[NW], s_c[NW];
  __shared__ float s_A[NW][HD], s_B[NW][HD];
  const int bh = blockIdx.x, b = bh / H, hh = bh - b * H, d = H * HD;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int sub = lane % G::LPR, slot = lane / G::LPR;
  const T* Kb = K + (int64_t)bh * bh_stride + sub * VEC;
  const T* Vb = V + (int64_t)bh * bh_stride + sub * VEC;
  const int64_t qo = (int64_t)b * d + hh * HD + sub * VEC;
  float qv[VEC], dv[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    qv[i] = q[qo + i] * scale;
    dv[i] = dout[qo + i];
  }
  BwdState<VEC> S;
  S.init();
  const int first = wave * G::RPW + slot;
  for (int base = 0; base < ntok; base += RPB * U) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * RPB + first;
      const bool ok = row < ntok;
      kr[u] = ok ? ld16_stream(Kb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
      vr[u] = ok ? ld16_stream(Vb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
    }
    float sc[U], dp[U];
    float mb = S.m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC], vf[VEC];
      unpack(kr[u], kf);
      unpack(vr[u], vf);
      float s = 0.f, p = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        s += qv[i] * kf[i];
        p += dv[i] * vf[i];
      }
#pragma unroll
      for (int o = G::LPR / 2; o >= 1; o >>= 1) {
        s += __shfl_xor(s, o, kWave);
        p += __shfl_xor(p, o, kWave);
      }
      const bool ok = base + u * RPB + first < ntok;
      sc[u] = ok ? s : -INFINITY;
      dp[u] = p;
      mb = fmaxf(mb, sc[u]);
    }
    if (mb == -INFINITY) continue;
    const float cs = S.m == -INFINITY ? 0.f : __expf(S.m - mb);
    S.l *= cs;
    S.c *= cs;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      S.A[i] *= cs;
      S.Bk[i] *= cs;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = sc[u] == -INFINITY ? 0.f : __expf(sc[u] - mb);
      float kf[VEC];
      unpack(kr[u], kf);
      S.l += e;
      S.c += e * dp[u];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        S.A[i] += e * dp[u] * kf[i];
        S.Bk[i] += e * kf[i];
      }
    }
    S.m = mb;
  }
#pragma unroll
  for (int o = G::LPR; o < kWave; o <<= 1) {
    const float mo = __shfl_xor(S.m, o, kWave), lo = __shfl_xor(S.l, o, kWave),
                co = __shfl_xor(S.c, o, kWave);
    float Ao[VEC], Bo[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      Ao[i] = __shfl_xor(S.A[i], o, kWave);
      Bo[i] = __shfl_xor(S.Bk[i], o, kWave);
    }
    S.merge(mo, lo, co, Ao, Bo);
  }
  if (slot == 0) {
    if (sub == 0) {
      s_m[wave] = S.m;
      s_l[wave] = S.l;
      s_c[wave] = S.c;
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      s_A[wave][sub * VEC + i] = S.A[i];
      s_B[wave][sub * VEC + i] = S.Bk[i];
    }
  }
  __syncthreads();
  if (tid < HD) {
    BwdState<1> R;
    R.m = s_m[0];
    R.l = s_l[0];
    R.c = s_c[0];
    R.A[0] = s_A[0][tid];
    R.Bk[0] = s_B[0][tid];
    for (int w = 1; w < NW; ++w) R.merge(s_m[w], s_l[w], s_c[w], &s_A[w][tid], &s_B[w][tid]);
    const float D = R.c / R.l;
    const int64_t o = (int64_t)b * d + hh * HD + tid;
    dq[o] = to_elem<T>(scale * (R.A[0] - D * R.Bk[0]) / R.l);
    do_t[o] = to_elem<T>(dout[o]);
    if (tid == 0) {
      lse[bh] = R.m + __logf(R.l);
      dlt[bh] = D;
    }
  }
}

template <typename T, int HD, int NW, int U>
__global__ __launch_bounds__(NW * kWave) void k_xattn_back(
    const float* __restrict__ q, const float* __restrict__ dout, const T* __restrict__ K,
    const T* __restrict__ V, int64_t bh_stride, int ntok, int H, float scale,
    T* __restrict__ dq, float* __restrict__ lse, float* __restrict__ dlt, T* __restrict__ do_t,
    unsigned long long* clk) {
  const LaunchClock lc{clk};
  lc.start();
  xattn_back_body<T, HD, NW, U>(q, dout, K, V, bh_stride, ntok, H, scale, dq, lse, dlt, do_t);
  lc.stop();
}

// Self-attention backward of token t for one (sequence, head) per workgroup.
//   dq_t: one online pass over the window keys j = lo..t (lo = max(0, t - W + 1)) of the layer's
//         key/value history, as for the memory prefix; it also yields lse_t and D_t, which go
//         with do_t to rings of W slots (slot t % W) for the tokens walked after this one.
//   dk_t, dv_t: token t's key/value is seen by the later tokens t' = t..min(t + W - 1, n - 1),
//         all walked already: dk_t = scale sum_t' dz_t't q_t', dv_t = sum_t' p_t't do_t' with
//         p_t't = exp(scale q_t'.k_t - lse_t') and dz = p (do_t'.v_t - D_t'), from the saved
//         queries and the rings. Writes [dq | dk | dv] (dtype) to out [M][3d].
template <typename T, int HD, int NW, int U>
__device__ __forceinline__ void swa_back_body(
    const float* __restrict__ qs, const float* __restrict__ dout, const T* __restrict__ K,
    const T* __restrict__ V, int64_t n, int64_t t, int64_t hi_cap, int W, int B, int H,
    float scale, T* __restrict__ ring_do, float* __restrict__ ring_lse,
    float* __restrict__ ring_dlt, T* __restrict__ out) {
  using G = AGeo<T, HD>;
  constexpr int VEC = G::VEC, RPB = G::RPW * NW;
  __shared__ float s_m[NW], s_l[NW], s_c[NW];
  __shared__ float s_A[NW][HD], s_B[NW][HD];
  __shared__ float s_stat[2];
  const int bh = blockIdx.x, b = bh / H, hh = bh - b * H, d = H * HD;
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int sub = lane % G::LPR, slot = lane / G::LPR;
  const int64_t lo = t - W + 1 > 0 ? t - W + 1 : 0;
  const int nk = (int)(t - lo + 1);
  const T* Kb = K + ((int64_t)bh * n + lo) * HD + sub * VEC;
  const T* Vb = V + ((int64_t)bh * n + lo) * HD + sub * VEC;
  const int64_t ho = hh * HD + sub * VEC;  // this lane's dims within a row of d
  const float* q_t = qs + t * B * d + (int64_t)b * d;
  float qv[VEC], dv[VEC];
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    qv[i] = q_t[ho + i] * scale;
    dv[i] = dout[(int64_t)b * d + ho + i];
  }
  // ---- dq_t, lse_t, D_t: online pass over the window keys
  BwdState<VEC> S;
  S.init();
  const int first = wave * G::RPW + slot;
  for (int base = 0; base < nk; base += RPB * U) {
    u32x4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = base + u * RPB + first;
      const bool ok = row < nk;
      kr[u] = ok ? ld16(Kb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
      vr[u] = ok ? ld16(Vb + (int64_t)row * HD) : u32x4{0, 0, 0, 0};
    }
    float sc[U], dp[U];
    float mb = S.m;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[VEC], vf[VEC];
      unpack(kr[u], kf);
      unpack(vr[u], vf);
      float sv = 0.f, pv = 0.f;
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        sv += qv[i] * kf[i];
        pv += dv[i] * vf[i];
      }
#pragma unroll
      for (int o = G::LPR / 2; o >= 1; o >>= 1) {
        sv += __shfl_xor(sv, o, kWave);
        pv += __shfl_xor(pv, o, kWave);
      }
      const bool ok = base + u * RPB + first < nk;
      sc[u] = ok ? sv : -INFINITY;
      dp[u] = pv;
      mb = fmaxf(mb, sc[u]);
    }
    if (mb == -INFINITY) continue;
    const float cs = S.m == -INFINITY ? 0.f : __expf(S.m - mb);
    S.l *= cs;
    S.c *= cs;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      S.A[i] *= cs;
      S.Bk[i] *= cs;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float e = sc[u] == -INFINITY ? 0.f : __expf(sc[u] - mb);
      float kf[VEC];
      unpack(kr[u], kf);
      S.l += e;
      S.c += e * dp[u];
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        S.A[i] += e * dp[u] * kf[i];
        S.Bk[i] += e * kf[i];
      }
    }
    S.m = mb;
  }
#pragma unroll
  for (int o = G::LPR; o < kWave; o <<= 1) {
    const float mo = __shfl_xor(S.m, o, kWave), lo2 = __shfl_xor(S.l, o, kWave),
                co = __shfl_xor(S.c, o, kWave);
    float Ao[VEC], Bo[VEC];
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      Ao[i] = __shfl_xor(S.A[i], o, kWave);
      Bo[i] = __shfl_xor(S.Bk[i], o, kWave);
    }
    S.merge(mo, lo2, co, Ao, Bo);
  }
  if (slot == 0) {
    if (sub == 0) {
      s_m[wave] = S.m;
      s_l[wave] = S.l;
      s_c[wave] = S.c;
    }
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      s_A[wave][sub * VEC + i] = S.A[i];
      s_B[wave][sub * VEC + i] = S.Bk[i];
    }
  }
  __syncthreads();
  const int64_t ro = (int64_t)b * 3 * d + hh * HD;  // this head's columns of out row b
  const int64_t rslot = t % W;
  if (tid < HD) {
    BwdState<1> R;
    R.m = s_m[0];
    R.l = s_l[0];
    R.c = s_c[0];
    R.A[0] = s_A[0][tid];
    R.Bk[0] = s_B[0][tid];
    for (int w = 1; w < NW; ++w) R.merge(s_m[w], s_l[w], s_c[w], &s_A[w][tid], &s_B[w][tid]);
    const float D = R.c / R.l;
    out[ro + tid] = to_elem<T>(scale * (R.A[0] - D * R.Bk[0]) / R.l);
    ring_do[(rslot * B + b) * d + hh * HD + tid] = to_elem<T>(dout[(int64_t)b * d + hh * HD + tid]);
    if (tid == 0) {
      const float lse = R.m + __logf(R.l);
      s_stat[0] = lse;
      s_stat[1] = D;
      ring_lse[rslot * B * H + bh] = lse;
      ring_dlt[rslot * B * H + bh] = D;
    }
  }
  __syncthreads();
  // ---- dk_t, dv_t: token t itself (from registers and LDS), then the later tokens
  float kt[VEC], vt[VEC], gk[VEC], gv[VEC];
  {
    float kf[VEC], vf[VEC];
    unpack(ld16(Kb + (int64_t)(nk - 1) * HD), kf);  // row t of the history
    unpack(ld16(Vb + (int64_t)(nk - 1) * HD), vf);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      kt[i] = kf[i];
      vt[i] = vf[i];
      gk[i] = 0.f;
      gv[i] = 0.f;
    }
  }
  // last token whose window holds t (and, with the window detached at segment starts, that is
  // in t's segment: hi_cap is the segment's last token)
  const int64_t hi = t + W - 1 < hi_cap ? t + W - 1 : hi_cap;
  const int nq = (int)(hi - t + 1);
  for (int r = first; r < nq; r += RPB) {
    const int64_t tp = t + r;
    float qf[VEC], df[VEC], lse, D;
    if (r == 0) {
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        qf[i] = qv[i] / scale;
        df[i] = dv[i];
      }
      lse = s_stat[0];
      D = s_stat[1];
    } else {
      const float* qp = qs + tp * B * d + (int64_t)b * d + ho;
      const int64_t sl = tp % W;
      u32x4 raw = ld16(ring_do + (sl * B + b) * d + ho);
      float tmp[VEC];
      unpack(raw, tmp);
#pragma unroll
      for (int i = 0; i < VEC; ++i) {
        qf[i] = qp[i];
        df[i] = tmp[i];
      }
      lse = ring_lse[sl * B * H + bh];
      D = ring_dlt[sl * B * H + bh];
    }
    float sv = 0.f, pv = 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      sv += qf[i] * kt[i];
      pv += df[i] * vt[i];
    }
#pragma unroll
    for (int o = G::LPR / 2; o >= 1; o >>= 1) {
      sv += __shfl_xor(sv, o, kWave);
      pv += __shfl_xor(pv, o, kWave);
    }
    const float pj = __expf(scale * sv - lse);
    const float dz = pj * (pv - D);
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      gk[i] += scale * dz * qf[i];
      gv[i] += pj * df[i];
    }
  }
  // sum over the slots of the wave, then over the waves
#pragma unroll
  for (int o = G::LPR; o < kWave; o <<= 1)
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      gk[i] += __shfl_xor(gk[i], o, kWave);
      gv[i] += __shfl_xor(gv[i], o, kWave);
    }
  if (slot == 0)
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      s_A[wave][sub * VEC + i] = gk[i];
      s_B[wave][sub * VEC + i] = gv[i];
    }
  __syncthreads();
  if (tid < HD) {
    float k = 0.f, v = 0.f;
    for (int w = 0; w < NW; ++w) {
      k += s_A[w][tid];
      v += s_B[w][tid];
    }
    out[ro + d + tid] = to_elem<T>(k);
    out[ro + 2 * d + tid] = to_elem<T>(v);
  }
}

template <typename T, int HD, int NW, int U>
__global__ __launch_bounds__(NW * kWave) void k_swa_back(
    const float* __restrict__ qs, const float* __restrict__ dout, const T* __restrict__ K,
    const T* __restrict__ V, int64_t n, int64_t t, int64_t hi_cap, int W, int B, int H,
    float scale, T* __restrict__ ring_do, float* __restrict__ ring_lse,
    float* __restrict__ ring_dlt, T* __restrict__ out,
    unsigned long long* clk) {
  const LaunchClock lc{clk};
  lc.start();
  swa_back_body<T, HD, NW, U>(qs, dout, K, V, n, t, hi_cap, W, B, H, scale, ring_do, ring_lse,
                              ring_dlt, out);
  lc.stop();
}

// ---- memory gradients after the walk ------------------------------------------------------------
// For memory entry j of one (sequence, head) and each layer using the group:
//   dV_j = sum_{t >= j} p_tj do_t,  dK_j = scale sum_{t >= j} p_tj (do_t . V_j - D_t) qc_t
// with p_tj = exp(scale qc_t . K_j - lse_t). One workgroup takes 64 entries (4 lanes each, a
// quarter of the head dims per lane) and walks the later tokens in tiles staged in LDS. Writes
// [dK | dV] rows (b * n + j) in dtype.
template <typename T, int HD>
__global__ __launch_bounds__(kThreads) void k_mem_back(
    const T* __restrict__ K, const T* __restrict__ V, const float* __restrict__ qcs,
    const T* __restrict__ docs, const float* __restrict__ lse, const float* __restrict__ dlt,
    int l0, int l1, int B, int64_t n, int H, float scale, T* __restrict__ dkv) {
  constexpr int KB = 64, TQ = 16, Q4 = HD / 4;
  __shared__ float s_q[TQ][HD], s_do[TQ][HD], s_lse[TQ], s_D[TQ];
  const int bh = blockIdx.y, b = bh / H, hh = bh - b * H, d = H * HD;
  const int64_t j0 = (int64_t)blockIdx.x * KB;
  const int tid = threadIdx.x, key = tid / 4, part = tid % 4;
  const int64_t j = j0 + key;
  const bool valid = j < n;
  float kf[Q4], vf[Q4], gk[Q4], gv[Q4];
  const T* kp = K + ((int64_t)bh * n + (valid ? j : 0)) * HD + part * Q4;
  const T* vp = V + ((int64_t)bh * n + (valid ? j : 0)) * HD + part * Q4;
#pragma unroll
  for (int i = 0; i < Q4; ++i) {
    kf[i] = to_f32<T>(kp[i]);
    vf[i] = to_f32<T>(vp[i]);
    gk[i] = 0.f;
    gv[i] = 0.f;
  }
  const int64_t layer = n * B * d;  // elements per layer of qcs / docs
  for (int l = l0; l < l1; ++l) {
    for (int64_t t0 = j0; t0 < n; t0 += TQ) {
      __syncthreads();
      for (int x = tid; x < TQ * HD; x += kThreads) {
        const int r = x / HD, c = x - r * HD;
        const int64_t t = t0 + r;
        const int64_t o = l * layer + (t * B + b) * d + hh * HD + c;
        s_q[r][c] = t < n ? qcs[o] : 0.f;
        s_do[r][c] = t < n ? to_f32<T>(docs[o]) : 0.f;
      }
      if (tid < TQ) {
        const int64_t t = t0 + tid;
        const int64_t o = ((int64_t)l * n + t) * B * H + bh;
        s_lse[tid] = t < n ? lse[o] : INFINITY;
        s_D[tid] = t < n ? dlt[o] : 0.f;
      }
      __syncthreads();
      for (int r = 0; r < TQ; ++r) {
        float s = 0.f, p = 0.f;
#pragma unroll
        for (int i = 0; i < Q4; ++i) {
          s += s_q[r][part * Q4 + i] * kf[i];
          p += s_do[r][part * Q4 + i] * vf[i];
        }
        s += __shfl_xor(s, 1, kWave);
        s += __shfl_xor(s, 2, kWave);
        p += __shfl_xor(p, 1, kWave);
        p += __shfl_xor(p, 2, kWave);
        const int64_t t = t0 + r;
        const float pj = (valid && t >= j && t < n) ? __expf(scale * s - s_lse[r]) : 0.f;
        const float dz = pj * (p - s_D[r]);
#pragma unroll
        for (int i = 0; i < Q4; ++i) {
          gv[i] += pj * s_do[r][part * Q4 + i];
          gk[i] += scale * dz * s_q[r][part * Q4 + i];
        }
      }
    }
  }
  if (!valid) return;
  T* o = dkv + ((int64_t)b * n + j) * 2 * d + hh * HD + part * Q4;
#pragma unroll
  for (int i = 0; i < Q4; ++i) {
    o[i] = to_elem<T>(gk[i]);
    o[d + i] = to_elem<T>(gv[i]);
  }
}

// The same memory gradients on MFMA (bf16 models). One workgroup takes 64 entries of one
// (sequence, head), 16 per wave, and walks the later tokens in tiles of 32 staged in LDS (queries
// converted to bf16, row-major for the score products and transposed for the gradient products).
// Per tile and wave: S = Q K^T and dP = dO V^T (the wave's keys and values stay in registers as
// the B operands), p = exp(scale S - lse), dz = p (dP - D), then dV += p^T dO and dK += dz^T Q.
// The score tiles leave each lane holding one entry's values for tokens 4g..4g+3 and 16+4g..
// 16+4g+3 (g = lane / 16), which is taken as the contraction order of the gradient products, so
// p and dz never move; the staged transposes are read in that order.
template <int HD>
__global__ __launch_bounds__(kThreads) void k_mem_back_mfma(
    const bf16* __restrict__ K, const bf16* __restrict__ V, const float* __restrict__ qcs,
    const bf16* __restrict__ docs, const float* __restrict__ lse, const float* __restrict__ dlt,
    int l0, int l1, int B, int n, int H, float scale, bf16* __restrict__ dkv) {
  constexpr int KB = 64, TQ = 32, KS = HD / 32, CT = HD / 16;
  __shared__ __attribute__((aligned(16))) bf16 q_r[TQ][HD + 8];
  __shared__ __attribute__((aligned(16))) bf16 o_r[TQ][HD + 8];
  __shared__ __attribute__((aligned(16))) bf16 q_t[HD][TQ + 8];
  __shared__ __attribute__((aligned(16))) bf16 o_t[HD][TQ + 8];
  __shared__ float s_lse[TQ], s_D[TQ];
  const int bh = blockIdx.y, b = bh / H, hh = bh - b * H, d = H * HD;
  const int j0 = blockIdx.x * KB;
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave, g = lane >> 4;
  const int jw = j0 + 16 * wave;
  const int jl = jw + (lane & 15);  // this lane's entry as an operand / score column
  const bf16* Kb = K + (int64_t)bh * n * HD;
  const bf16* Vb = V + (int64_t)bh * n * HD;
  Frag<bf16> kf[KS], vf[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    if (jl < n) {
      kf[s].load(Kb + (int64_t)jl * HD + 32 * s + 8 * g);
      vf[s].load(Vb + (int64_t)jl * HD + 32 * s + 8 * g);
    } else {
      kf[s].zero();
      vf[s].zero();
    }
  }
  f32x4 gk[CT], gv[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) gk[c] = gv[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float c2 = scale * 1.4426950408889634f, l2e = 1.4426950408889634f;
  const int64_t layer = (int64_t)n * B * d;
  for (int l = l0; l < l1; ++l) {
    for (int t0 = j0 / TQ * TQ; t0 < n; t0 += TQ) {
      __syncthreads();  // the previous tile's LDS reads are done
      for (int x = tid; x < TQ * HD / 4; x += kThreads) {  // 4 dims per item
        const int r = x / (HD / 4), c = (x % (HD / 4)) * 4;
        const int t = t0 + r;
        float qv[4] = {0.f, 0.f, 0.f, 0.f}, ov[4] = {0.f, 0.f, 0.f, 0.f};
        if (t < n) {
          const int64_t o = l * layer + ((int64_t)t * B + b) * d + hh * HD + c;
          const u32x4 raw = ld16(qcs + o);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            qv[i] = __uint_as_float(raw[i]);
            ov[i] = (float)docs[o + i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16 qb = (bf16)qv[i], ob = (bf16)ov[i];
          q_r[r][c + i] = qb;
          o_r[r][c + i] = ob;
          q_t[c + i][r] = qb;
          o_t[c + i][r] = ob;
        }
      }
      if (tid < TQ) {
        const int t = t0 + tid;
        const int64_t o = ((int64_t)l * n + t) * B * H + bh;
        s_lse[tid] = t < n ? lse[o] * l2e : INFINITY;
        s_D[tid] = t < n ? dlt[o] : 0.f;
      }
      __syncthreads();
      if (t0 + TQ <= jw) continue;  // every token of the tile is earlier than the wave's entries
      // scores and output-gradient products of the two 16-token halves
      f32x4 sc[2], dp[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sc[h] = dp[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 qa = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(&q_r[16 * h + (lane & 15)][32 * s + 8 * g]));
          const bf16x8 oa = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(&o_r[16 * h + (lane & 15)][32 * s + 8 * g]));
          sc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[s].v, sc[h], 0, 0, 0);
          dp[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[s].v, dp[h], 0, 0, 0);
        }
      }
      // lane holds token rows 16 h + 4 g + i of entry column jl
      bf16x8 pb, zb;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tr = 16 * h + 4 * g + i, t = t0 + tr;
          const bool ok = t < n && t >= jl && jl < n;
          const float pj = ok ? __builtin_amdgcn_exp2f(sc[h][i] * c2 - s_lse[tr]) : 0.f;
          pb[4 * h + i] = (bf16)pj;
          zb[4 * h + i] = (bf16)(pj * (dp[h][i] - s_D[tr]));
        }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        // B operands: dims 16 c + lane % 16, tokens in the lanes' contraction order
        const bf16* op = &o_t[16 * c + (lane & 15)][0];
        const bf16* qp = &q_t[16 * c + (lane & 15)][0];
        const uint2 olo = *reinterpret_cast<const uint2*>(op + 4 * g);
        const uint2 ohi = *reinterpret_cast<const uint2*>(op + 16 + 4 * g);
        const uint2 qlo = *reinterpret_cast<const uint2*>(qp + 4 * g);
        const uint2 qhi = *reinterpret_cast<const uint2*>(qp + 16 + 4 * g);
        const u32x4 orw = {olo.x, olo.y, ohi.x, ohi.y};
        const u32x4 qrw = {qlo.x, qlo.y, qhi.x, qhi.y};
        gv[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb, __builtin_bit_cast(bf16x8, orw), gv[c],
                                                        0, 0, 0);
        gk[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(zb, __builtin_bit_cast(bf16x8, qrw), gk[c],
                                                        0, 0, 0);
      }
    }
  }
  // lane holds rows (entries) jw + 4 g + i, column (dim) 16 c + lane % 16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int j = jw + 4 * g + i;
    if (j >= n) continue;
    bf16* o = dkv + ((int64_t)b * n + j) * 2 * d + hh * HD + (lane & 15);
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      o[16 * c] = (bf16)(scale * gk[c][i]);
      o[d + 16 * c] = (bf16)gv[c][i];
    }
  }
}

// ---- weight gradients: C[K][N] += X[M][K]^T Y[M][N] ----------------------------------------------
// Both operands are first transposed to [features][rows] in MFMA fragment order (rows padded with
// zeros to a multiple of 32), which makes the contraction over rows the fragments' k dimension;
// the product is then the register-tiled token GEMM (k_gemm_tokens) with the transposed X as
// operand A and the transposed Y in the place of the packed weights.

// dst[frag_off(c, m, Mp / 32)] = src[m][c] for m < M, zero for M <= m < Mp. One workgroup per
// 32 x 32 tile, staged in LDS; each store is 8 consecutive rows of one column (16 bytes bf16).
// blockIdx.z = z transposes matrix z of a batch: src + z src_z, dst + z dst_z.
template <typename T>
__global__ __launch_bounds__(kThreads) void k_mfrag(const T* __restrict__ src, int64_t ld,
                                                    int64_t M, int64_t Mp, T* __restrict__ dst,
                                                    int64_t src_z, int64_t dst_z) {
  __shared__ T tile[32][33];
  src += blockIdx.z * src_z;
  dst += blockIdx.z * dst_z;
  const int64_t m0 = (int64_t)blockIdx.y * 32;
  const int c0 = blockIdx.x * 32;
  const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;
  for (int r = ty; r < 32; r += 8) {
    const int64_t m = m0 + r;
    tile[r][tx] = m < M ? src[m * ld + c0 + tx] : to_elem<T>(0.f);
  }
  __syncthreads();
  if (threadIdx.x >= 128) return;
  const int c = threadIdx.x / 4, g = threadIdx.x % 4;
  T v[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = tile[g * 8 + e][c];
  T* o = dst + frag_off(c0 + c, (int)(m0 + g * 8), (int)(Mp / 32));
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = v[e];
}

template <typename T>
struct AMfrag {  // A = [rows][K] in fragment order (ksteps = K / 32); token-GEMM interface
  const T* a;
  int ksteps;
  int M;
  int64_t zs = 0;  // elements between the operands of consecutive products of a batch
  __device__ Frag<T> load(int row, int k, float&) const {
    Frag<T> f;
    if (row < M) f.load(a + frag_off(row, k, ksteps));
    else f.zero();
    return f;
  }
};

// Output column c goes to p[c / split] at (row, c % split) of a [rows][split] fp32 matrix,
// added to what is there.
struct WDst {
  float* p[3];
  int split;
};

struct EpiAddSplit {
  WDst dst;
  int M;
  int64_t zs = 0;  // elements between the outputs of consecutive products of a batch
  template <int FM, int FN>
  __device__ void tile(const f32x4 (&acc)[FM][FN], int rbase, int cwave, int lane) const {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = rbase + 16 * fm + i;
          const int c = cwave + 16 * fn + (lane & 15);
          const int which = c / dst.split, cc = c - which * dst.split;
          if (row < M) dst.p[which][(int64_t)row * dst.split + cc] += acc[fm][fn][i];
        }
  }
};

template <typename T>
__device__ __forceinline__ AMfrag<T> batch_at(const AMfrag<T>& a, int z) {
  AMfrag<T> r = a;
  r.a += z * a.zs;
  return r;
}
__device__ __forceinline__ EpiAddSplit batch_at(const EpiAddSplit& e, int z) {
  EpiAddSplit r = e;
  for (int i = 0; i < 3; ++i)
    if (r.dst.p[i]) r.dst.p[i] += z * e.zs;
  return r;
}

// ---- host side ---------------------------------------------------------------------------------

template <typename T>
static inline T* el(void* base, int64_t off) {
  return static_cast<T*>(base) + off;
}
template <typename T>
static inline const T* el(const void* base, int64_t off) {
  return static_cast<const T*>(base) + off;
}
static inline unsigned blocks_for(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

#define RLT_TRY(...)                       \
  do {                                     \
    hipError_t err_ = (__VA_ARGS__);       \
    if (err_ != hipSuccess) return err_;   \
  } while (0)

// C[K][N] += X[M][K]^T Y[M][N] through the transposition scratch tx, ty (>= Mp * K and
// Mp * N elements, Mp = M rounded up to 32).
template <typename T>
static hipError_t wgrad(const T* X, int64_t ldx, const T* Y, int64_t ldy, int64_t M, int K, int N,
                        WDst dst, T* tx, T* ty, const Exec& xt, const Exec& x) {
  if (K % 64 || N % 64 || M <= 0 || M > INT32_MAX / 2) return hipErrorInvalidValue;
  const int64_t Mp = (M + 31) / 32 * 32;
  RLT_TRY(launch(k_mfrag<T>, dim3(K / 32, (unsigned)(Mp / 32)), dim3(kThreads), xt, X, ldx, M, Mp,
                 tx, (int64_t)0, (int64_t)0));
  RLT_TRY(launch(k_mfrag<T>, dim3(N / 32, (unsigned)(Mp / 32)), dim3(kThreads), Exec(xt.st), Y,
                 ldy, M, Mp, ty, (int64_t)0, (int64_t)0));
  return run_gemm<T, kBig.wm, kBig.wn, kBig.fm, kBig.fn>(
      K, N, (int)Mp, ty, AMfrag<T>{tx, (int)(Mp / 32), K}, EpiAddSplit{dst, K}, x);
}

// The same for the L layers of one weight kind at once (bf16, K and N multiples of 128): layer l
// reads X + l xz and Y + l yz and adds into the destinations shifted by l dz; one transpose
// launch per operand and one batched GEMM.
template <typename T>
static hipError_t wgrad_layers(const T* X, int64_t ldx, int64_t xz, const T* Y, int64_t ldy,
                               int64_t yz, int64_t M, int K, int N, int L, WDst dst, int64_t dz,
                               T* tx, T* ty, const Exec& xt, const Exec& x) {
  if constexpr (std::is_same<T, bf16>::value) {
    if (K % 128 || N % 128 || M <= 0 || M > INT32_MAX / 2 || L < 1) return hipErrorInvalidValue;
    const int64_t Mp = (M + 31) / 32 * 32;
    RLT_TRY(launch(k_mfrag<T>, dim3(K / 32, (unsigned)(Mp / 32), L), dim3(kThreads), xt, X, ldx,
                   M, Mp, tx, xz, (int64_t)K * Mp));
    RLT_TRY(launch(k_mfrag<T>, dim3(N / 32, (unsigned)(Mp / 32), L), dim3(kThreads),
                   Exec(xt.st), Y, ldy, M, Mp, ty, yz, (int64_t)N * Mp));
    return run_gemm_batched(K, N, (int)Mp, L, ty, (int64_t)N * Mp,
                            AMfrag<T>{tx, (int)(Mp / 32), K, (int64_t)K * Mp},
                            EpiAddSplit{dst, K, dz}, x);
  } else {
    return hipErrorInvalidValue;
  }
}

template <typename T, int HD>
static hipError_t xattn_back(int BH, const float* q, const float* dout, const T* K, const T* V,
                             int64_t bh_stride, int ntok, int H, T* dq, float* lse, float* dlt,
                             T* do_t, const Exec& x) {
  const float scale = 1.f / sqrtf((float)HD);
  const int nw = BH >= 1024 ? 4 : BH >= 512 ? 8 : 16;
#define RLT_XB(NW)                                                                             \
  return launch(k_xattn_back<T, HD, NW, 4>, dim3(BH), dim3(NW * kWave), x, q, dout, K, V,        \
                bh_stride, ntok, H, scale, dq, lse, dlt, do_t, x.clk)
  if (nw == 4) RLT_XB(4);
  if (nw == 8) RLT_XB(8);
  RLT_XB(16);
#undef RLT_XB
}

template <typename T, int HD>
static hipError_t swa_back(int BH, int B, const float* qs, const float* dout, const T* K,
                           const T* V, int64_t n, int64_t t, int64_t hi_cap, int W, int H,
                           T* ring_do, float* ring_lse, float* ring_dlt, T* out, const Exec& x) {
  const float scale = 1.f / sqrtf((float)HD);
  const int nw = BH >= 1024 ? 4 : BH >= 512 ? 8 : 16;
#define RLT_SB(NW)                                                                              \
  return launch(k_swa_back<T, HD, NW, 4>, dim3(BH), dim3(NW * kWave), x, qs, dout, K, V, n, t,   \
                hi_cap, W, B, H, scale, ring_do, ring_lse, ring_dlt, out, x.clk)
  if (nw == 4) RLT_SB(4);
  if (nw == 8) RLT_SB(8);
  RLT_SB(16);
#undef RLT_SB
}

// Column sums of `nmat` fp32 matrices of `rows` valid rows (matrix m at P + m * stride * d)
// added to out (matrices below out.n_gamma into out.gamma + m * d, the next into out.extra).
static hipError_t colsums(const float* P, int nmat, int64_t rows, int64_t stride, int d,
                          float* part, ColOut out, const Exec& x, const Exec& x2) {
  RLT_TRY(launch(k_colsum_part, dim3(blocks_for(d), kRowSplits, nmat), dim3(kThreads), x, P, rows,
                 stride, d, part));
  return launch(k_colsum_final, dim3(blocks_for(d), nmat), dim3(kThreads), x2,
                (const float*)part, d, out);
}

template <typename T>
struct Walk {  // pointers into the workspace of one call, for the rows [b0, b0 + rows)
  const Dims& D;
  int B;  // all rows: the stride of every row-indexed buffer
  int64_t n;
  const TrainLayout& TL;
  void* ws;
  int b0 = 0, rows = 0;
  size_t cpar = 0;  // byte offset of the chunk-buffer copy in use (0 or TL.cspan)
  template <typename P>
  P* at(size_t off) const {
    return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
  }
  // a chunk buffer (ca .. yg) in the copy in use
  template <typename P>
  P* cat(size_t off) const {
    return at<P>(off + cpar);
  }
  // rows of chunk-local token li in a per-layer chunk buffer of `width` columns
  T* chunk(size_t base, int l, int64_t width, int64_t li) const {
    return cat<T>(base) + ((int64_t)l * TL.Mc + li * B + b0) * width;
  }
  // fp32 gain/bias-gradient rows: matrix m (3 l + which, or 3 L for the gate bias)
  float* pg(int m, int64_t li) const {
    return cat<float>(TL.pg) + ((int64_t)m * TL.Mc + li * B + b0) * D.d;
  }
  // [L][n][B][d] saved rows of layer l, token i
  template <typename P>
  P* saved(size_t base, int l, int64_t i) const {
    return at<P>(base) + (((int64_t)l * n + i) * B + b0) * D.d;
  }
  // per-row scratch of `width` values per row
  template <typename P>
  P* row(size_t base, int64_t width) const {
    return at<P>(base) + (int64_t)b0 * width;
  }
  Walk group(int g0, int nrows) const {
    Walk w = *this;
    w.b0 = g0;
    w.rows = nrows;
    return w;
  }
};

// Exec of one launch: armed with timing events when `prof` times `kind` and the launch is
// sampled; the first arming error is kept and reported at the end.
struct Timer {
  Profiler* prof;
  hipStream_t st;
  hipError_t err = hipSuccess;
  // grid > 0: a self-timing kernel of `grid` workgroups (clock slots when attached)
  Exec at(int kind, double bytes, double flops, bool sampled = true, int64_t grid = 0) {
    Exec x(st);
    if (prof && sampled && err == hipSuccess) err = prof->arm(kind, bytes, flops, x, grid);
    return x;
  }
};

// The reverse walk over token i (chunk-local index li). Algorithmic bytes: weights, operands
// and results once each (es per dtype element, 4 per fp32 one).
template <typename T, int HD>
static hipError_t walk_token(const Walk<T>& w, const Packed& P, const MemBufs& M, const T* e,
                             const float* G, float* de, int64_t i, int64_t li, int64_t segment,
                             uint32_t detach, Timer& tm, bool sampled) {
  const Dims& D = w.D;
  const TrainLayout& TL = w.TL;
  // B: this group's rows (GEMM rows, grids); Bt: all rows (strides); b0: the group's first row
  const int B = w.rows, Bt = w.B, b0 = w.b0, d = D.d, F = D.F, L = D.L, H = D.H, BH = B * D.H;
  const int64_t n = w.n;
  const BwOff bo = bw_off(D);
  const T* bw = w.template at<T>(TL.bw);
  float* dres = w.template row<float>(TL.dres, d);
  float* dn = w.template row<float>(TL.dn, d);
  float* dattn = w.template row<float>(TL.dattn, d);
  float* rinv = w.template row<float>(TL.rinv, 3);
  float* gsave = w.template row<float>(TL.gsave, d);
  float* carry = w.template row<float>(TL.carry, d);
  G += (int64_t)b0 * n * d;
  e += (int64_t)b0 * n * d;
  if (de) de += (int64_t)b0 * n * d;
  const int64_t dd = (int64_t)d * d;
  const double b = B, es = (double)D.es, rows32 = b * d * 4, rowsT = b * d * es;
  // a per-token projection: N x K weights, A rows of K, `out` bytes of results
  // weights are charged in proportion to this group's rows: once per token over all groups
  const double share = (double)B / Bt;
  auto proj = [&](double N, double K, double out) {
    return tm.at(RLT_K_BWD_PROJ, N * K * es * share + b * K * es + out, 2 * b * N * K, sampled);
  };
  auto other = [&](double bytes) { return tm.at(RLT_K_BWD_OTHER, bytes, 0, sampled); };

  // the norm rows of layer l (the three saved residual streams of token i)
  auto rows_of = [&](int l) {
    return NormRows<T>{w.template saved<float>(TL.xs, l, i), w.template saved<float>(TL.ys, l, i),
                       w.template saved<float>(TL.zs, l, i), P.gamma + (int64_t)l * 3 * d,
                       w.chunk(TL.ca, l, d, li), w.chunk(TL.cc, l, d, li),
                       w.chunk(TL.cf, l, d, li), D.eps};
  };
  const double nrb = 3 * rows32 + 3 * rowsT;  // bytes of one set of norm rows
  // the gradient of s_i through token i+1 is dropped when i+1 starts a segment that detaches s
  const bool cut_state = segment > 0 && (detach & RLT_DETACH_STATE) && (i + 1) % segment == 0;
  RLT_TRY(launch(k_walk_begin<T>, dim3(B), dim3(kThreads), other(3 * rows32 + rowsT + nrb), G,
                 cut_state ? (const float*)nullptr : (const float*)carry, dres,
                 w.chunk(TL.y2, L - 1, d, li), d, n, i, rows_of(L - 1), rinv));
  const int64_t hi_cap = segment > 0 && (detach & RLT_DETACH_WINDOW)
                             ? std::min<int64_t>(n - 1, (i / segment + 1) * segment - 1)
                             : n - 1;
  for (int l = L - 1; l >= 0; --l) {
    const float* gam = P.gamma + (int64_t)l * 3 * d;
    const float* xs = w.template saved<float>(TL.xs, l, i);
    const float* ys = w.template saved<float>(TL.ys, l, i);
    const float* zs = w.template saved<float>(TL.zs, l, i);
    // feed-forward: from the forward's u1 | u3, dm -> du -> df -> dres
    const float* u13 = w.template at<float>(TL.u13) + (((int64_t)l * n + i) * Bt + b0) * 2 * F;
    T* y13 = w.chunk(TL.y13, l, 2 * F, li);
    {
      EpiSiluBack<T> ep;
      ep.u = u13; ep.du = y13; ep.m = w.chunk(TL.cm, l, F, li); ep.M = B; ep.F = F;
      RLT_TRY(run_step_gemm<T>(B, F, d, bw + bo.w2 + (int64_t)l * F * d,
                               ARows<T>{w.chunk(TL.y2, l, d, li), d, B}, ep,
                               proj(F, d, b * F * (8 + 3 * es))));
    }
    EpiStoreF32 to_dn;
    to_dn.out = dn; to_dn.ld = d; to_dn.M = B;
    EpiStoreF32 to_dattn;
    to_dattn.out = dattn; to_dattn.ld = d; to_dattn.M = B;
    RLT_TRY(run_step_gemm<T>(B, d, 2 * F, bw + bo.w13 + (int64_t)l * d * 2 * F,
                             ARows<T>{y13, 2 * F, B}, to_dn, proj(d, 2 * F, rows32)));
    T* yco = w.chunk(TL.yco, l, d, li);
    const double nb = 5 * rows32 + rowsT;  // dn, x, dres in, dres out, gain terms; dtype copy
    const NormRows<T> none{};
    RLT_TRY(launch(k_norm_back<T>, dim3(B), dim3(kThreads), other(nb), (const float*)dn, zs,
                   gam + 2 * d, rinv, 2, d, dres, yco, w.pg(3 * l + 2, li), none));
    // cross-attention
    RLT_TRY(run_step_gemm<T>(B, d, d, bw + bo.wco + l * dd, ARows<T>{yco, d, B}, to_dattn,
                             proj(d, d, rows32)));
    const int g = D.G == 1 ? 0 : l;
    const int64_t grp = ((int64_t)g * Bt + b0) * n * d;
    T* ycq = w.chunk(TL.ycq, l, d, li);
    const int64_t stat = ((int64_t)l * n + i) * Bt * H + (int64_t)b0 * H;
    const double ntok = (double)(i + 1);
    RLT_TRY(xattn_back<T, HD>(BH, w.template saved<float>(TL.qcs, l, i), dattn,
                              el<T>(M.k, grp), el<T>(M.v, grp), n * HD, (int)(i + 1), H, ycq,
                              w.template at<float>(TL.lse) + stat,
                              w.template at<float>(TL.dlt) + stat,
                              w.template saved<T>(TL.docs, l, i),
                              tm.at(RLT_K_BWD_CROSS, ntok * b * 2 * d * es + 2 * rows32 +
                                        2 * rowsT + 8 * b * H, 8 * b * d * ntok, sampled, BH)));
    RLT_TRY(run_step_gemm<T>(B, d, d, bw + bo.wcq + l * dd, ARows<T>{ycq, d, B}, to_dn,
                             proj(d, d, rows32)));
    T* yo = w.chunk(TL.yo, l, d, li);
    RLT_TRY(launch(k_norm_back<T>, dim3(B), dim3(kThreads), other(nb), (const float*)dn, ys,
                   gam + d, rinv, 1, d, dres, yo, w.pg(3 * l + 1, li), none));
    // self-attention
    RLT_TRY(run_step_gemm<T>(B, d, d, bw + bo.wo + l * dd, ARows<T>{yo, d, B}, to_dattn,
                             proj(d, d, rows32)));
    T* yqkv = w.chunk(TL.yqkv, l, 3 * d, li);
    const int64_t hist = ((int64_t)l * Bt + b0) * n * d;
    const int64_t rd = (int64_t)l * D.W * Bt * d + (int64_t)b0 * d;
    const int64_t rs = (int64_t)l * D.W * Bt * H + (int64_t)b0 * H;
    const double nk = (double)std::min<int64_t>(i + 1, D.W);
    const double nq = (double)std::min<int64_t>(hi_cap - i + 1, D.W);
    RLT_TRY(swa_back<T, HD>(BH, Bt, w.template at<float>(TL.qs) + (int64_t)l * n * Bt * d + b0 * d,
                            dattn, w.template at<T>(TL.khist) + hist,
                            w.template at<T>(TL.vhist) + hist, n, i, hi_cap, D.W, H,
                            w.template at<T>(TL.dkacc) + rd, w.template at<float>(TL.dvacc) + rs,
                            w.template at<float>(TL.dvacc) + (int64_t)L * D.W * Bt * H + rs, yqkv,
                            tm.at(RLT_K_BWD_SELF, nk * b * 2 * d * es + nq * b * d * (4 + es) +
                                      2 * rows32 + 4 * rowsT, (10 * nk + 8 * nq) * b * d,
                                  sampled, BH)));
    RLT_TRY(run_step_gemm<T>(B, d, 3 * d, bw + bo.wqkv + (int64_t)l * 3 * dd,
                             ARows<T>{yqkv, 3 * d, B}, to_dn, proj(d, 3 * d, rows32)));
    RLT_TRY(launch(k_norm_back<T>, dim3(B), dim3(kThreads), other(nb + (l > 0 ? nrb : 0)),
                   (const float*)dn, xs, gam, rinv, 0, d, dres,
                   l > 0 ? w.chunk(TL.y2, l - 1, d, li) : (T*)nullptr, w.pg(3 * l, li),
                   l > 0 ? rows_of(l - 1) : none));
  }
  // gated merge: recompute g, then dz, then de_t and the carry to s_{t-1}
  const T* et = e + i * d;
  const float* s_prev = w.template at<float>(TL.s_hist) + (i * Bt + b0) * d;
  T* yg = w.template cat<T>(TL.yg) + (li * Bt + b0) * d;
  {
    AGate<T> al{et, n * d, s_prev, D.alpha, B, d};
    EpiGateBack<T> ep;
    ep.e = et; ep.lde = n * d; ep.s = s_prev; ep.b = P.b_gate; ep.dres = dres; ep.alpha = D.alpha;
    ep.dz = yg; ep.dz32 = w.pg(3 * L, li); ep.g = gsave;
    ep.xg = w.template cat<T>(TL.xg) + (li * Bt + b0) * 2 * d; ep.M = B; ep.d = d;
    RLT_TRY(run_step_gemm<T>(B, d, 2 * d, P.w_gate_t, al, ep,
                             proj(d, 2 * d, 3 * rows32 + rowsT + b * 2 * d * es)));
  }
  {
    EpiGateOut ep;
    ep.dres = dres; ep.g = gsave; ep.de = de ? de + i * d : nullptr; ep.de_ld = n * d;
    ep.carry = carry; ep.alpha = D.alpha; ep.M = B; ep.d = d;
    RLT_TRY(run_step_gemm<T>(B, 2 * d, d, bw + bo.wg, ARows<T>{yg, d, B}, ep,
                             proj(2 * d, d, 4 * rows32)));
  }
  return hipSuccess;
}

// Weight and gain gradients of the chunk of tokens [i0, i1).
template <typename T>
static hipError_t chunk_grads(const Walk<T>& w, const GradPtrs& g, int64_t i0, int64_t i1,
                              Timer& tm) {
  const Dims& D = w.D;
  const TrainLayout& TL = w.TL;
  const int B = w.B, d = D.d, F = D.F, L = D.L;
  const int64_t rows = (i1 - i0) * B, dd = (int64_t)d * d, dF = (int64_t)d * F;
  const double es = (double)D.es;
  T* tx = w.template at<T>(TL.tx);
  T* ty = w.template at<T>(TL.ty);
  // operands transposed once (read + write), then the GEMM (reads both, adds into fp32 C)
  auto gw = [&](const T* X, int64_t ldx, const T* Y, int64_t ldy, int K, int N, WDst dst) {
    return wgrad<T>(X, ldx, Y, ldy, rows, K, N, dst, tx, ty,
                    tm.at(RLT_K_BWD_OTHER, 2.0 * rows * (K + N) * es, 0),
                    tm.at(RLT_K_BWD_WGRAD, rows * (K + N) * es + (double)K * N * 8,
                          2.0 * rows * K * N));
  };
  if (std::is_same<T, bf16>::value && d % 128 == 0 && F % 128 == 0) {
    // every layer of one weight kind in one batch: layer strides of the chunk buffers (Mc rows
    // of `width`), of the saved rows ([L][n][B][d]) and of the gradients
    const int64_t Mc = TL.Mc, sz = w.n * B * d;
    auto gl = [&](const T* X, int64_t ldx, int64_t xz, const T* Y, int64_t ldy, int64_t yz,
                  int K, int N, WDst dst, int64_t dz) {
      return wgrad_layers<T>(X, ldx, xz, Y, ldy, yz, rows, K, N, L, dst, dz, tx, ty,
                             tm.at(RLT_K_BWD_OTHER, L * 2.0 * rows * (K + N) * es, 0),
                             tm.at(RLT_K_BWD_WGRAD, L * (rows * (K + N) * es + (double)K * N * 8),
                                   L * 2.0 * rows * K * N));
    };
    RLT_TRY(gl(w.chunk(TL.ca, 0, d, 0), d, Mc * d, w.chunk(TL.yqkv, 0, 3 * d, 0), 3 * d,
               Mc * 3 * d, d, 3 * d, WDst{{g.wq, g.wk, g.wv}, d}, dd));
    RLT_TRY(gl(w.template saved<T>(TL.os, 0, i0), d, sz, w.chunk(TL.yo, 0, d, 0), d, Mc * d, d,
               d, WDst{{g.wo, nullptr, nullptr}, d}, dd));
    RLT_TRY(gl(w.chunk(TL.cc, 0, d, 0), d, Mc * d, w.chunk(TL.ycq, 0, d, 0), d, Mc * d, d, d,
               WDst{{g.wcq, nullptr, nullptr}, d}, dd));
    RLT_TRY(gl(w.template saved<T>(TL.ocs, 0, i0), d, sz, w.chunk(TL.yco, 0, d, 0), d, Mc * d,
               d, d, WDst{{g.wco, nullptr, nullptr}, d}, dd));
    RLT_TRY(gl(w.chunk(TL.cf, 0, d, 0), d, Mc * d, w.chunk(TL.y13, 0, 2 * F, 0), 2 * F,
               Mc * 2 * F, d, 2 * F, WDst{{g.w1, g.w3, nullptr}, F}, dF));
    RLT_TRY(gl(w.chunk(TL.cm, 0, F, 0), F, Mc * F, w.chunk(TL.y2, 0, d, 0), d, Mc * d, F, d,
               WDst{{g.w2, nullptr, nullptr}, d}, dF));
  } else {
    for (int l = 0; l < L; ++l) {
      RLT_TRY(gw(w.chunk(TL.ca, l, d, 0), d, w.chunk(TL.yqkv, l, 3 * d, 0), 3 * d, d, 3 * d,
                 WDst{{g.wq + l * dd, g.wk + l * dd, g.wv + l * dd}, d}));
      RLT_TRY(gw(w.template saved<T>(TL.os, l, i0), d, w.chunk(TL.yo, l, d, 0), d, d, d,
                 WDst{{g.wo + l * dd, nullptr, nullptr}, d}));
      RLT_TRY(gw(w.chunk(TL.cc, l, d, 0), d, w.chunk(TL.ycq, l, d, 0), d, d, d,
                 WDst{{g.wcq + l * dd, nullptr, nullptr}, d}));
      RLT_TRY(gw(w.template saved<T>(TL.ocs, l, i0), d, w.chunk(TL.yco, l, d, 0), d, d, d,
                 WDst{{g.wco + l * dd, nullptr, nullptr}, d}));
      RLT_TRY(gw(w.chunk(TL.cf, l, d, 0), d, w.chunk(TL.y13, l, 2 * F, 0), 2 * F, d, 2 * F,
                 WDst{{g.w1 + l * dF, g.w3 + l * dF, nullptr}, F}));
      RLT_TRY(gw(w.chunk(TL.cm, l, F, 0), F, w.chunk(TL.y2, l, d, 0), d, F, d,
                 WDst{{g.w2 + l * dF, nullptr, nullptr}, d}));
    }
  }
  RLT_TRY(gw(w.template cat<T>(TL.xg), 2 * d, w.template cat<T>(TL.yg), d, 2 * d, d,
             WDst{{g.w_gate, nullptr, nullptr}, d}));
  const double cs = (3.0 * L + 1) * rows * d * 4;
  return colsums(w.pg(0, 0), 3 * L + 1, rows, TL.Mc, d, w.template at<float>(TL.part),
                 ColOut{g.gamma, g.b_gate, 3 * L}, tm.at(RLT_K_BWD_OTHER, cs, cs / 4),
                 tm.at(RLT_K_BWD_OTHER, 0, 0));
}

template <typename T, int HD>
static hipError_t bptt_t(const Dims& D, int B, int64_t n, const Packed& P, const void* e_v,
                         const float* G, float* s_traj, const GradPtrs& g, float* de, void* ws,
                         int64_t segment, uint32_t detach, hipStream_t st, hipStream_t aux,
                         hipEvent_t ev_fork, hipEvent_t ev_join, hipStream_t gs,
                         const hipEvent_t* gev, Profiler* prof) {
  const TrainLayout TL = train_layout(D, B, n);
  const Walk<T> w{D, B, n, TL, ws};
  const int d = D.d, F = D.F, L = D.L, H = D.H;
  const T* e = static_cast<const T*>(e_v);
  const Exec x(st);
  Timer tm{prof, st};
  const int64_t stride = prof ? prof->stride : 1;
  const double b = B, es = (double)D.es, dsz = d, Fd = F;
  // backward copies of the weights
  {
    const BwOff bo = bw_off(D);
    T* bw = w.template at<T>(TL.bw);
    auto repack = [&](const void* src, int N, int K, T* dst, int w13, int64_t mats) {
      const double bytes = 2.0 * N * K * mats * es;
      return launch(k_repack<T>, dim3(blocks_for((int64_t)N * K * mats)), dim3(kThreads),
                    tm.at(RLT_K_BWD_OTHER, bytes, 0), static_cast<const T*>(src), N, K, dst, w13,
                    F, mats);
    };
    RLT_TRY(repack(P.w_gate_t, d, 2 * d, bw + bo.wg, 0, 1));
    RLT_TRY(repack(P.wqkv_t, 3 * d, d, bw + bo.wqkv, 0, L));
    RLT_TRY(repack(P.wo_t, d, d, bw + bo.wo, 0, L));
    RLT_TRY(repack(P.wcq_t, d, d, bw + bo.wcq, 0, L));
    RLT_TRY(repack(P.wco_t, d, d, bw + bo.wco, 0, L));
    RLT_TRY(repack(P.w13_t, 2 * F, d, bw + bo.w13, 1, L));
    RLT_TRY(repack(P.w2_t, d, F, bw + bo.w2, 0, L));
    RLT_TRY(repack(P.wm_t, 2 * d, d, bw + bo.wm, 0, D.G));
  }
  // state, memory, s_0 = s*
  StateBufs S;
  {
    const StateLayout SL = state_layout(D, B);
    char* base = w.template at<char>(TL.state);
    S.Bt = B;
    S.s = reinterpret_cast<float*>(base + SL.s);
    S.ring_k = base + SL.ring_k;
    S.ring_v = base + SL.ring_v;
    S.h = reinterpret_cast<float*>(base + SL.h);
    S.q = reinterpret_cast<float*>(base + SL.q);
    S.qc = reinterpret_cast<float*>(base + SL.qc);
    S.hg = base + SL.hg;
    S.ssq = reinterpret_cast<float*>(base + SL.ssq);
    S.o = base + SL.o;
    S.act = base + SL.act;
    S.hb = base + SL.hb;
    S.pos = reinterpret_cast<int64_t*>(base + SL.pos);
    S.part = reinterpret_cast<float*>(base + SL.part);
    S.active = nullptr;
    S.t_uniform = 0;
    S.t_max = 0;
  }
  MemBufs M{w.template at<void>(TL.mem_k), w.template at<void>(TL.mem_v), n, B};
  float* s_hist = w.template at<float>(TL.s_hist);
  RLT_TRY(launch_reset(D, B, P, S, st));
  {
    const double rows = b * n;
    RLT_TRY(launch_memproj(D, B, P, M, e, n, 0, n,
                           tm.at(RLT_K_MEMPROJ, es * (rows * dsz + D.G * 2 * dsz * dsz +
                                                      rows * D.G * 2 * dsz),
                                 2 * rows * dsz * D.G * 2 * dsz)));
  }
  RLT_TRY(launch(k_fill_start, dim3(blocks_for((int64_t)B * d)), dim3(kThreads), x, s_hist,
                 (const float*)P.s_star, d, (int64_t)B * d));
  // row groups: two halves of the batch on two streams (the caller's and `aux`), as the decoder
  // step runs them, when the batch is large enough; joined around the weight-gradient GEMMs
  const int ng = aux && B >= 2 * kGroupRows ? 2 : 1;
  const int half = ng == 2 ? ((B + 1) / 2 + 15) / 16 * 16 : B;
  const int row0[3] = {0, half, B};
  Timer gtm[2] = {Timer{prof, st}, Timer{prof, aux}};
  auto fork = [&]() -> hipError_t {
    if (ng < 2) return hipSuccess;
    RLT_TRY(hipEventRecord(ev_fork, st));
    return hipStreamWaitEvent(aux, ev_fork, 0);
  };
  auto join = [&]() -> hipError_t {
    if (ng < 2) return hipSuccess;
    RLT_TRY(hipEventRecord(ev_join, aux));
    return hipStreamWaitEvent(st, ev_join, 0);
  };
  // forward, saving x, y, z, q, qc, o, oc and every key/value (bytes counted as in the decoder
  // step)
  const int64_t ring_layer = (int64_t)B * H * D.W * D.hd;
  RLT_TRY(fork());
  StateBufs Sg[2];
  MemBufs Mg[2];
  for (int gi = 0; gi < ng; ++gi) {
    Sg[gi] = state_rows(D, S, row0[gi]);
    Mg[gi] = memory_rows(D, M, row0[gi]);
  }
  for (int64_t i = 0; i < n; ++i) {
    const bool smp = i % stride == 0;
    const double nv = (double)std::min<int64_t>(i + 1, D.W), t = (double)(i + 1);
    for (int gi = 0; gi < ng; ++gi) {
      const int b0 = row0[gi], rb = row0[gi + 1] - b0;
      const Walk<T> wg = w.group(b0, rb);
      Timer& tg = gtm[gi];
      StateBufs& Sx = Sg[gi];
      Sx.t_uniform = i;
      Sx.t_max = i;
      const double bg = rb, a32 = bg * d * 4, ad = bg * d * es;
      const double sh = bg / B;  // this group's share of each weight read
      RLT_TRY(gemm_gate(D, rb, P, Sx, e + ((int64_t)b0 * n + i) * d, n * d,
                        tg.at(RLT_K_GATE, 2 * dsz * dsz * es * sh + ad + 2 * a32,
                              4 * bg * dsz * dsz, smp)));
      const dim3 grid(blocks_for((int64_t)rb * d));
      {
        SaveArgs a{};
        a.stage = 0; a.B = rb; a.d = d;
        a.h = Sx.h;
        a.h_dst = wg.template saved<float>(TL.xs, 0, i);
        RLT_TRY(launch(k_save<T>, grid, dim3(kThreads), tg.at(RLT_K_BWD_OTHER, 2 * a32, 0, smp),
                       a));
      }
      for (int l = 0; l < L; ++l) {
        const bool last = l == L - 1;
        // queries straight into their save slots; the cross-attention output into a second
        // buffer, so both outputs survive to the layer's single copy
        StateBufs Sl = Sx;
        Sl.q = wg.template saved<float>(TL.qs, l, i);
        Sl.qc = wg.template saved<float>(TL.qcs, l, i);
        StateBufs Sc = Sl;
        Sc.o = w.template at<char>(TL.o2) + (size_t)b0 * d * D.es;
        RLT_TRY(gemm_qkv(D, rb, l, P, Sl,
                         tg.at(RLT_K_QKV, 3 * dsz * dsz * es * sh + 2 * a32 + 2 * ad,
                               6 * bg * dsz * dsz, smp)));
        RLT_TRY(attn_self(D, rb, l, Sl,
                          tg.at(RLT_K_SELF_ATTN, nv * bg * 2 * dsz * es + a32 + ad,
                                4 * bg * dsz * nv, smp)));
        RLT_TRY(gemm_residual(D, rb, l, 0, P, Sl, false, wg.template saved<float>(TL.ys, l, i), d,
                              tg.at(RLT_K_SELF_OUT, dsz * dsz * es * sh + ad + 3 * a32,
                                    2 * bg * dsz * dsz, smp)));
        RLT_TRY(gemm_cq(D, rb, l, P, Sl,
                        tg.at(RLT_K_CROSS_Q, dsz * dsz * es * sh + 2 * a32, 2 * bg * dsz * dsz,
                              smp)));
        RLT_TRY(attn_cross(D, rb, l, Sc, Mg[gi],
                           tg.at(RLT_K_CROSS_ATTN, t * bg * 2 * dsz * es + a32 + ad,
                                 4 * bg * dsz * t, smp)));
        RLT_TRY(gemm_residual(D, rb, l, 1, P, Sc, false, wg.template saved<float>(TL.zs, l, i), d,
                              tg.at(RLT_K_CROSS_OUT, dsz * dsz * es * sh + ad + 3 * a32,
                                    2 * bg * dsz * dsz, smp)));
        SaveArgs a{};
        a.stage = 1; a.B = rb; a.d = d; a.H = H; a.hd = D.hd; a.W = D.W; a.n = n; a.i = i;
        a.o = Sl.o;
        a.oc = Sc.o;
        a.o_dst = wg.template saved<T>(TL.os, l, i);
        a.oc_dst = wg.template saved<T>(TL.ocs, l, i);
        a.ring_k = el<T>(Sx.ring_k, l * ring_layer);
        a.ring_v = el<T>(Sx.ring_v, l * ring_layer);
        a.k_dst = w.template at<T>(TL.khist) + ((int64_t)l * B + b0) * n * d;
        a.v_dst = w.template at<T>(TL.vhist) + ((int64_t)l * B + b0) * n * d;
        RLT_TRY(launch(k_save<T>, grid, dim3(kThreads),
                       tg.at(RLT_K_BWD_OTHER, 8 * ad, 0, smp), a));
        RLT_TRY(gemm_w13(D, rb, l, P, Sl,
                         tg.at(RLT_K_FFN_UP, 2 * Fd * dsz * es * sh + a32 + bg * Fd * (es + 8),
                               4 * bg * dsz * Fd, smp),
                         w.template at<float>(TL.u13) + (((int64_t)l * n + i) * B + b0) * 2 * F));
        float* next = last ? s_hist + ((i + 1) * B + b0) * d
                           : wg.template saved<float>(TL.xs, l + 1, i);
        RLT_TRY(gemm_residual(D, rb, l, 2, P, Sl, last, next, d,
                              tg.at(RLT_K_FFN_DOWN, Fd * dsz * es * sh + bg * Fd * es + 3 * a32,
                                    2 * bg * dsz * Fd, smp)));
      }
    }
  }
  RLT_TRY(join());
  if (s_traj)
    RLT_TRY(launch(k_traj, dim3(blocks_for((int64_t)B * n * d)), dim3(kThreads), x,
                   (const float*)s_hist, s_traj, B, n, d));
  // gradients start at zero
  {
    const int64_t dd = (int64_t)d * d, dF = (int64_t)d * F;
    struct Z {
      float* p;
      int64_t n;
    } zs[] = {{g.s_star, d},     {g.w_gate, 2 * dd}, {g.b_gate, d},     {g.gamma, 3LL * L * d},
              {g.wq, L * dd},    {g.wk, L * dd},     {g.wv, L * dd},    {g.wo, L * dd},
              {g.wcq, L * dd},   {g.wco, L * dd},    {g.w1, L * dF},    {g.w3, L * dF},
              {g.w2, L * dF},    {g.wmk, D.G * dd},  {g.wmv, D.G * dd}};
    for (const Z& z : zs) RLT_TRY(hipMemsetAsync(z.p, 0, sizeof(float) * z.n, st));
    if (de) RLT_TRY(hipMemsetAsync(de, 0, sizeof(float) * B * n * d, st));
    RLT_TRY(hipMemsetAsync(w.template at<float>(TL.carry), 0, sizeof(float) * B * d, st));
  }
  // the reverse walk, one chunk of Tc tokens at a time (newest chunk first). With the gradient
  // stream gs, chunk c's weight gradients run there while the walk goes on with chunk c + 1 in
  // the other copy of the chunk buffers; the walk of chunk c + 2 waits until they are done.
  // The gradients still accumulate chunk after chunk in the same order.
  Timer gtg{prof, gs ? gs : st};
  bool done_rec[2] = {false, false};
  int64_t c = 0;
  for (int64_t i1 = n; i1 > 0; ++c) {
    const int64_t i0 = std::max<int64_t>(0, i1 - TL.Tc);
    const int p = (int)(c & 1);
    Walk<T> wc = w;
    wc.cpar = p ? TL.cspan : 0;
    if (done_rec[p]) RLT_TRY(hipStreamWaitEvent(st, gev[2 + p], 0));
    RLT_TRY(fork());
    for (int64_t i = i1 - 1; i >= i0; --i)
      for (int gi = 0; gi < ng; ++gi)
        RLT_TRY(walk_token<T, HD>(wc.group(row0[gi], row0[gi + 1] - row0[gi]), P, M, e, G, de,
                                  i, i - i0, segment, detach, gtm[gi], i % stride == 0));
    RLT_TRY(join());
    if (gs) {
      RLT_TRY(hipEventRecord(gev[p], st));
      RLT_TRY(hipStreamWaitEvent(gs, gev[p], 0));
      RLT_TRY(chunk_grads<T>(wc, g, i0, i1, gtg));
      RLT_TRY(hipEventRecord(gev[2 + p], gs));
      done_rec[p] = true;
    } else {
      RLT_TRY(chunk_grads<T>(wc, g, i0, i1, tm));
    }
    i1 = i0;
  }
  for (int p = 0; p < 2; ++p)
    if (done_rec[p]) RLT_TRY(hipStreamWaitEvent(st, gev[2 + p], 0));
  RLT_TRY(gtg.err);
  // s_0 = s* for every sequence
  RLT_TRY(colsums(w.template at<float>(TL.carry), 1, B, B, d, w.template at<float>(TL.part),
                  ColOut{nullptr, g.s_star, 0}, x, x));
  // memory entries: gradients from every later token, then the memory projection's backward
  const BwOff bo = bw_off(D);
  const float scale = 1.f / sqrtf((float)HD);
  T* dkv = w.template at<T>(TL.dkv);
  const double rows = b * n;
  for (int gi = 0; gi < D.G; ++gi) {
    const int l0 = D.G == 1 ? 0 : gi, l1 = D.G == 1 ? L : gi + 1;
    const int64_t grp = (int64_t)gi * B * n * d;
    const double nl = l1 - l0;
    const Exec xm = tm.at(RLT_K_BWD_MEM,
                          rows * dsz * (4 * es + nl * (4 + es)) + nl * rows * H * 8,
                          nl * 4.0 * b * dsz * (double)n * (double)(n + 1));
    const dim3 mgrid((unsigned)((n + 63) / 64), B * H);
    if constexpr (std::is_same<T, bf16>::value)
      RLT_TRY(launch(k_mem_back_mfma<HD>, mgrid, dim3(kThreads), xm, el<T>(M.k, grp),
                     el<T>(M.v, grp), (const float*)w.template at<float>(TL.qcs),
                     (const T*)w.template at<T>(TL.docs),
                     (const float*)w.template at<float>(TL.lse),
                     (const float*)w.template at<float>(TL.dlt), l0, l1, B, (int)n, H, scale,
                     dkv));
    else
      RLT_TRY(launch(k_mem_back<T, HD>, mgrid, dim3(kThreads), xm, el<T>(M.k, grp),
                     el<T>(M.v, grp), (const float*)w.template at<float>(TL.qcs),
                     (const T*)w.template at<T>(TL.docs),
                     (const float*)w.template at<float>(TL.lse),
                     (const float*)w.template at<float>(TL.dlt), l0, l1, B, n, H, scale, dkv));
    for (int64_t r0 = 0; r0 < (int64_t)B * n; r0 += TL.Mc) {  // in chunks of rows
      const int64_t rc = std::min<int64_t>(TL.Mc, (int64_t)B * n - r0);
      RLT_TRY(wgrad<T>(e + r0 * d, d, dkv + r0 * 2 * d, 2 * d, rc, d, 2 * d,
                       WDst{{g.wmk + (int64_t)gi * d * d, g.wmv + (int64_t)gi * d * d, nullptr},
                            d},
                       w.template at<T>(TL.tx), w.template at<T>(TL.ty),
                       tm.at(RLT_K_BWD_OTHER, 2.0 * rc * 3 * dsz * es, 0),
                       tm.at(RLT_K_BWD_WGRAD, rc * 3 * dsz * es + 2 * dsz * dsz * 8,
                             2.0 * rc * dsz * 2 * dsz)));
    }
    if (de) {
      const T* wm = w.template at<T>(TL.bw) + bo.wm + (int64_t)gi * 2 * d * d;
      RLT_TRY(run_gemm<T, kBig.wm, kBig.wn, kBig.fm, kBig.fn>(
          (int)((int64_t)B * n), d, 2 * d, wm, ARows<T>{dkv, 2 * d, (int)((int64_t)B * n)},
          EpiAddF32{de, d, (int)((int64_t)B * n)},
          tm.at(RLT_K_BWD_PROJ, 2 * dsz * dsz * es + rows * 2 * dsz * es + rows * dsz * 8,
                2 * rows * dsz * 2 * dsz)));
    }
  }
  RLT_TRY(gtm[0].err);
  RLT_TRY(gtm[1].err);
  return tm.err;
}

hipError_t launch_bptt(const Dims& D, int B, int64_t n, const Packed& P, const void* e,
                       const float* G, float* s_traj, const GradPtrs& g, float* de, void* ws,
                       int64_t segment, uint32_t detach, hipStream_t st, hipStream_t aux,
                       hipEvent_t ev_fork, hipEvent_t ev_join, hipStream_t gs,
                       const hipEvent_t* gev, Profiler* prof) {
#define RLT_BPTT(HDV)                                                                         \
  return D.dtype == RLT_BF16                                                                  \
             ? bptt_t<bf16, HDV>(D, B, n, P, e, G, s_traj, g, de, ws, segment, detach, st,   \
                                 aux, ev_fork, ev_join, gs, gev, prof)                        \
             : bptt_t<float, HDV>(D, B, n, P, e, G, s_traj, g, de, ws, segment, detach, st,  \
                                  aux, ev_fork, ev_join, gs, gev, prof)
  switch (D.hd) {
    case 32: RLT_BPTT(32);
    case 64: RLT_BPTT(64);
    case 128: RLT_BPTT(128);
    default: return hipErrorInvalidValue;
  }
#undef RLT_BPTT
}

#undef RLT_TRY

}  // namespace rlt
