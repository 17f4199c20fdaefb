// Sampling of the next token from readout logits on gfx950, with the behaviour log-probability
// of the action under the distribution actually sampled from ("RLT Runs 96 Blocks Per Token With
// Recurrent State, No Resets", "Three design principles and their caveats", model-RL co-design:
// temperature and truncation included).
//
// One workgroup per row. q = softmax(z / temperature); tokens are ordered by descending logit
// (the order of q), ties by ascending id. Top-k keeps the first k of that order, top-p the
// shortest prefix of the top-k tokens whose mass reaches p times the top-k mass; the action is
// the first kept token, in ascending id, at which the running kept mass exceeds u times the
// kept mass. Temperature 0 is greedy (the first maximal logit, probability 1).
//
// Selections run on exact integers, so every decision is a function of the logits alone,
// independent of thread timing: thresholds are found by radix selection (four 8-bit digit
// passes) over an order-preserving 32-bit key of the logit, with integer counts for top-k and
// fixed-point masses (q scaled by 2^40, 64-bit) for top-p and for the inverse CDF. Each token's
// fixed-point mass is computed once and kept in a scratch row, so every pass sees the same
// values.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace rlt {

namespace {

constexpr int kST = 256;                     // threads per row
constexpr double kFix = 1099511627776.0;     // 2^40
typedef unsigned long long u64;

// Larger logit <=> larger key (finite logits).
__device__ __forceinline__ uint32_t order_key(float z) {
  const uint32_t b = __float_as_uint(z);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

struct Shared {
  uint32_t cnt[256];
  u64 mass[256];
  u64 scan[kST];
  float red[kST / kWave];
  u64 tot;
  int sel[2];
};

__device__ __forceinline__ float block_max(float v, Shared& sh) {
  v = wave_max(v);
  if (threadIdx.x % kWave == 0) sh.red[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh.red[0];
  for (int w = 1; w < kST / kWave; ++w) r = fmaxf(r, sh.red[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, Shared& sh) {
  v = wave_sum(v);
  if (threadIdx.x % kWave == 0) sh.red[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh.red[0];
  for (int w = 1; w < kST / kWave; ++w) r += sh.red[w];
  __syncthreads();
  return r;
}

// Exclusive prefix of per-thread values in thread order; sh.tot receives the total.
__device__ __forceinline__ u64 block_excl_scan(u64 v, Shared& sh) {
  sh.scan[threadIdx.x] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    u64 run = 0;
    for (int t = 0; t < kST; ++t) {
      const u64 x = sh.scan[t];
      sh.scan[t] = run;
      run += x;
    }
    sh.tot = run;
  }
  __syncthreads();
  const u64 r = sh.scan[threadIdx.x];
  __syncthreads();
  return r;
}

// Every thread owns the contiguous ids [lo, hi) of the row, so thread order is id order.
struct Chunk {
  int lo, hi;
  __device__ Chunk(int V) {
    const int c = (V + kST - 1) / kST;
    lo = min(V, (int)threadIdx.x * c);
    hi = min(V, lo + c);
  }
};

// The first id, in ascending order, at which the running sum of w(i) over ids with w(i) > 0
// exceeds thr (thr < 0: the first id with w(i) > 0); V if none. All threads get the result.
template <class Wt>
__device__ int first_crossing(int V, Wt w, long long thr, Shared& sh) {
  const Chunk ch(V);
  u64 own = 0;
  for (int i = ch.lo; i < ch.hi; ++i) own += w(i);
  const u64 before = block_excl_scan(own, sh);
  if (threadIdx.x == 0) sh.sel[0] = V;
  __syncthreads();
  const long long b0 = (long long)before, b1 = (long long)(before + own);
  if (own > 0 && b1 > thr && b0 <= (thr < 0 ? 0 : thr)) {
    u64 run = before;
    for (int i = ch.lo; i < ch.hi; ++i) {
      const u64 x = w(i);
      if (x == 0) continue;
      run += x;
      if ((long long)run > thr) {
        atomicMin(&sh.sel[0], i);
        break;
      }
    }
  }
  __syncthreads();
  const int r = sh.sel[0];
  __syncthreads();
  return r;
}

}  // namespace

// fq: scratch [B][V] u64 (fixed-point masses of the tempered distribution).
__global__ __launch_bounds__(kST) void k_sample(const float* __restrict__ logits, int V,
                                                float temperature, int top_k, float top_p,
                                                const float* __restrict__ u,
                                                u64* __restrict__ fqbuf,
                                                int32_t* __restrict__ tok_out,
                                                float* __restrict__ lp_beh,
                                                float* __restrict__ lp_model) {
  __shared__ Shared sh;
  const int tid = threadIdx.x, row = blockIdx.x;
  const float* z = logits + (int64_t)row * V;
  u64* fq = fqbuf + (int64_t)row * V;
  float mx = -INFINITY;
  for (int i = tid; i < V; i += kST) mx = fmaxf(mx, z[i]);
  mx = block_max(mx, sh);
  float s1 = 0.f;
  for (int i = tid; i < V; i += kST) s1 += expf(z[i] - mx);
  const float log_z1 = logf(block_sum(s1, sh));

  int a;
  float lpb;
  if (!(temperature > 0.f)) {
    // greedy: the first maximal logit
    if (tid == 0) sh.sel[1] = V;
    __syncthreads();
    for (int i = tid; i < V; i += kST)
      if (z[i] == mx) {
        atomicMin(&sh.sel[1], i);
        break;
      }
    __syncthreads();
    a = sh.sel[1];
    lpb = 0.f;
  } else {
    const float inv_t = 1.f / temperature, mt = mx * inv_t;
    float st = 0.f;
    for (int i = tid; i < V; i += kST) st += expf(z[i] * inv_t - mt);
    st = block_sum(st, sh);
    const float inv_st = 1.f / st;
    for (int i = tid; i < V; i += kST)
      fq[i] = (u64)((double)(expf(z[i] * inv_t - mt) * inv_st) * kFix + 0.5);
    __syncthreads();  // fq rows are re-read below by other threads of this workgroup

    // top-k: the k-th largest key, and how many of the tokens holding it are kept
    const bool use_k = top_k > 0 && top_k < V;
    uint32_t kth = 0;
    int tie_cut_k = V;
    if (use_k) {
      uint32_t prefix = 0, pmask = 0;
      int remaining = top_k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int j = tid; j < 256; j += kST) sh.cnt[j] = 0;
        __syncthreads();
        {
          // runs of equal digits are counted in registers and added once (most logits share
          // the leading digit, which would serialise the LDS atomics)
          uint32_t cur = 256u, run = 0u;
          for (int i = tid; i < V; i += kST) {
            const uint32_t key = order_key(z[i]);
            if ((key & pmask) != prefix) continue;
            const uint32_t dg = (key >> shift) & 255u;
            if (dg != cur) {
              if (run) atomicAdd(&sh.cnt[cur], run);
              cur = dg;
              run = 0u;
            }
            ++run;
          }
          if (run) atomicAdd(&sh.cnt[cur], run);
        }
        __syncthreads();
        if (tid == 0) {
          int cum = 0, dsel = 0;
          for (int dg = 255; dg >= 0; --dg) {
            if (cum + (int)sh.cnt[dg] >= remaining) {
              dsel = dg;
              break;
            }
            cum += (int)sh.cnt[dg];
          }
          sh.sel[0] = dsel;
          sh.sel[1] = remaining - cum;
        }
        __syncthreads();
        prefix |= (uint32_t)sh.sel[0] << shift;
        pmask |= 255u << shift;
        remaining = sh.sel[1];
        __syncthreads();
      }
      kth = prefix;
      // ties at the k-th key: the first `remaining` of them in ascending id
      tie_cut_k = first_crossing(
          V, [&](int i) -> u64 { return order_key(z[i]) == kth ? 1ull : 0ull; },
          (long long)remaining - 1, sh);
    }
    auto in_topk = [&](int i) -> bool {
      if (!use_k) return true;
      const uint32_t key = order_key(z[i]);
      return key > kth || (key == kth && i <= tie_cut_k);
    };

    // top-p over the top-k tokens
    const bool use_p = top_p < 1.f;
    uint32_t thp = 0;
    int tie_cut_p = V;
    if (use_p) {
      u64 mk = 0;
      for (int i = tid; i < V; i += kST)
        if (in_topk(i)) mk += fq[i];
      (void)block_excl_scan(mk, sh);
      const double target = (double)top_p * (double)sh.tot;
      uint32_t prefix = 0, pmask = 0;
      u64 above = 0;  // mass of the top-k tokens whose key is above the current digit range
      for (int shift = 24; shift >= 0; shift -= 8) {
        for (int j = tid; j < 256; j += kST) {
          sh.cnt[j] = 0;
          sh.mass[j] = 0;
        }
        __syncthreads();
        {
          uint32_t cur = 256u, run = 0u;
          u64 msum = 0;
          for (int i = tid; i < V; i += kST) {
            const uint32_t key = order_key(z[i]);
            if ((key & pmask) != prefix || !in_topk(i)) continue;
            const uint32_t dg = (key >> shift) & 255u;
            if (dg != cur) {
              if (run) {
                atomicAdd(&sh.cnt[cur], run);
                atomicAdd(&sh.mass[cur], msum);
              }
              cur = dg;
              run = 0u;
              msum = 0;
            }
            ++run;
            msum += fq[i];
          }
          if (run) {
            atomicAdd(&sh.cnt[cur], run);
            atomicAdd(&sh.mass[cur], msum);
          }
        }
        __syncthreads();
        if (tid == 0) {
          u64 cum = above;
          int dsel = -1, lowest = 0;
          for (int dg = 255; dg >= 0; --dg) {
            if (sh.cnt[dg] == 0) continue;
            lowest = dg;
            if ((double)(cum + sh.mass[dg]) >= target) {
              dsel = dg;
              break;
            }
            cum += sh.mass[dg];
          }
          if (dsel < 0) {  // rounding left the whole range short of the target: keep all of it
            dsel = lowest;
            cum -= sh.mass[lowest];
          }
          sh.sel[0] = dsel;
          sh.tot = cum;
        }
        __syncthreads();
        prefix |= (uint32_t)sh.sel[0] << shift;
        pmask |= 255u << shift;
        above = sh.tot;
        __syncthreads();
      }
      thp = prefix;
      // tokens holding the threshold key, in ascending id, until the mass reaches the target
      const double need = target - (double)above;
      const long long thr = need <= 0.0 ? -1 : (long long)ceil(need) - 1;
      tie_cut_p = first_crossing(
          V,
          [&](int i) -> u64 { return order_key(z[i]) == thp && in_topk(i) ? fq[i] : 0ull; },
          thr, sh);
      if (tie_cut_p == V) tie_cut_p = V - 1;  // every tie is kept
    }
    auto kept = [&](int i) -> bool {
      if (!in_topk(i)) return false;
      if (!use_p) return true;
      const uint32_t key = order_key(z[i]);
      return key > thp || (key == thp && i <= tie_cut_p);
    };

    // inverse CDF over the kept tokens in ascending id
    u64 mown = 0;
    {
      const Chunk ch(V);
      for (int i = ch.lo; i < ch.hi; ++i)
        if (kept(i)) mown += fq[i];
    }
    (void)block_excl_scan(mown, sh);
    const u64 mass = sh.tot;
    __syncthreads();
    u64 tu = (u64)floor((double)u[row] * (double)mass);
    if (tu >= mass) tu = mass - 1;
    a = first_crossing(
        V, [&](int i) -> u64 { return kept(i) ? fq[i] : 0ull; }, (long long)tu, sh);
    if (a >= V) a = V - 1;  // not reached: the kept mass is positive and tu < mass
    lpb = (z[a] * inv_t - mt - logf(st)) - logf((float)((double)mass / kFix));
  }
  if (tid == 0) {
    tok_out[row] = a;
    lp_beh[row] = lpb;
    lp_model[row] = z[a] - mx - log_z1;
  }
}

hipError_t launch_sample(int B, int V, const float* logits, float temperature, int top_k,
                         float top_p, const float* u, void* fq, int32_t* tokens,
                         float* logp_behaviour, float* logp_model, hipStream_t st) {
  return launch(k_sample, dim3((unsigned)B), dim3(kST), Exec(st), logits, V, temperature, top_k,
                top_p, u, static_cast<u64*>(fq), tokens, logp_behaviour, logp_model);
}

}  // namespace rlt
