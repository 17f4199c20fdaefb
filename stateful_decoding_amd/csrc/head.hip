// Sampling of the next token from readout logits on gfx950, with the behaviour log-probability
// of the action under the distribution actually sampled from ("RLT Runs 96 Blocks Per Token With
// Recurrent State, No Resets", "Three design principles and their caveats", model-RL co-design:
// temperature and truncation included).
//
// One workgroup (16 waves) per row. q = softmax(z / temperature); tokens are ordered by descending logit
// (the order of q), ties by ascending id. Top-k keeps the first k of that order, top-p the
// shortest prefix of the top-k tokens whose mass reaches p times the top-k mass; the action is
// the first kept token, in ascending id, at which the running kept mass exceeds u times the
// kept mass. Temperature 0 is greedy (the first maximal logit, probability 1).
//
// Selections run on exact integers, so every decision is a function of the logits alone,
// independent of thread timing: thresholds are found by radix selection (four 8-bit digit
// passes) over an order-preserving 32-bit key of the logit, with integer counts for top-k and
// fixed-point masses (q scaled by 2^40, 64-bit) for top-p and for the inverse CDF. A token's
// fixed-point mass is recomputed from its logit by one expression wherever it is used, so every
// pass sees the same values. Scans in id order are two-level: per-wave totals in LDS, then one
// wave walks its 64-id strips with a lane prefix.
#include <math.h>

#include "common.h"
#include "internal.h"

namespace rlt {

namespace {

constexpr int kST = 1024;                    // threads per row
constexpr int kNW = kST / kWave;             // waves per row
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
  u64 wtot[kNW];  // per-wave totals
  float red[kNW];
  u64 part[4];    // per-wave totals of the 256-entry digit scans
  u64 tot;
  int sel[2];
};

__device__ __forceinline__ u64 wave_sum_u64(u64 v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// inclusive prefix over the lanes of a wave
template <typename U>
__device__ __forceinline__ U wave_incl_scan(U v) {
  const int lane = threadIdx.x % kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const U y = __shfl_up(v, o, kWave);
    if (lane >= o) v += y;
  }
  return v;
}

__device__ __forceinline__ float block_max(float v, Shared& sh) {
  v = wave_max(v);
  if (threadIdx.x % kWave == 0) sh.red[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh.red[0];
  for (int w = 1; w < kNW; ++w) r = fmaxf(r, sh.red[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float v, Shared& sh) {
  v = wave_sum(v);
  if (threadIdx.x % kWave == 0) sh.red[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = sh.red[0];
  for (int w = 1; w < kNW; ++w) r += sh.red[w];
  __syncthreads();
  return r;
}

__device__ __forceinline__ u64 block_sum_u64(u64 v, Shared& sh) {
  v = wave_sum_u64(v);
  if (threadIdx.x % kWave == 0) sh.wtot[threadIdx.x / kWave] = v;
  __syncthreads();
  u64 r = 0;
  for (int w = 0; w < kNW; ++w) r += sh.wtot[w];
  __syncthreads();
  return r;
}

// Wave w owns the contiguous ids [lo, hi) (a multiple of 64 long, the last one shorter) and its
// lanes walk them 64 at a time, so every load is coalesced and wave order is id order.
struct Range {
  int lo, hi;
  __device__ explicit Range(int V) {
    const int c = (V + kST - 1) / kST * kWave;
    lo = min(V, (int)(threadIdx.x / kWave) * c);
    hi = min(V, lo + c);
  }
};

// The first id, in ascending order, at which the running sum of w(i) over ids with w(i) > 0
// exceeds thr (thr < 0: the first id with w(i) > 0); V if none. All threads get the result.
template <class Wt>
__device__ int first_crossing(int V, Wt w, long long thr, Shared& sh) {
  const Range r(V);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  u64 own = 0;
  for (int i = r.lo + lane; i < r.hi; i += kWave) own += w(i);
  own = wave_sum_u64(own);
  if (lane == 0) sh.wtot[wave] = own;
  if (threadIdx.x == 0) sh.sel[0] = V;
  __syncthreads();
  // the wave holding the crossing: the first with positive mass whose inclusive sum exceeds thr
  int cw = kNW;
  u64 before = 0, run = 0;
  for (int j = 0; j < kNW; ++j) {
    const u64 x = sh.wtot[j];
    if (cw == kNW && x > 0 && (long long)(run + x) > thr) {
      cw = j;
      before = run;
    }
    run += x;
  }
  if (wave == cw) {
    for (int base = r.lo; base < r.hi; base += kWave) {
      const int i = base + lane;
      const u64 x = i < r.hi ? w(i) : 0ull;
      const u64 incl = wave_incl_scan(x);
      const u64 hit = __ballot(x > 0 && (long long)(before + incl) > thr);
      if (hit) {
        if (lane == 0) sh.sel[0] = base + __ffsll((unsigned long long)hit) - 1;
        break;
      }
      before += __shfl(incl, kWave - 1, kWave);
    }
  }
  __syncthreads();
  const int res = sh.sel[0];
  __syncthreads();
  return res;
}

// Radix step of a count selection: with sh.cnt[] holding the counts of the 256 digits, the
// digit (from the top) at which the running count reaches `remaining`, into sh.sel[0], and how
// many of that digit are still needed, into sh.sel[1]. Threads 0..255 take digit 255 - tid.
__device__ void select_count_digit(int remaining, Shared& sh) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  uint32_t c = 0, incl = 0;
  if (tid < 256) {
    c = sh.cnt[255 - tid];
    incl = wave_incl_scan(c);
    if (lane == kWave - 1) sh.part[w] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    for (int j = 0; j < w; ++j) incl += (uint32_t)sh.part[j];
    const uint32_t excl = incl - c;
    if ((int)excl < remaining && remaining <= (int)incl) {
      sh.sel[0] = 255 - tid;
      sh.sel[1] = remaining - (int)excl;
    }
  }
  __syncthreads();
}

// Radix step of a mass selection: with sh.cnt[] / sh.mass[] holding the counts and masses of
// the 256 digits and `above` the mass above this digit range, the first non-empty digit from the
// top at which the running mass reaches `target` (the lowest non-empty digit when rounding
// leaves the whole range short), into sh.sel[0], and the mass above it into sh.tot.
__device__ void select_mass_digit(u64 above, double target, Shared& sh) {
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  uint32_t c = 0;
  u64 m = 0, incl = 0;
  if (tid == 0) {
    sh.sel[0] = -1;
    sh.sel[1] = 256;
  }
  if (tid < 256) {
    c = sh.cnt[255 - tid];
    m = sh.mass[255 - tid];
    incl = wave_incl_scan(m);
    if (lane == kWave - 1) sh.part[w] = incl;
  }
  __syncthreads();
  if (tid < 256) {
    for (int j = 0; j < w; ++j) incl += sh.part[j];
    if (c > 0) {
      // the running mass only grows towards lower digits, so the first digit from the top
      // that reaches the target is the highest one that does
      if ((double)(above + incl) >= target) atomicMax(&sh.sel[0], 255 - tid);
      atomicMin(&sh.sel[1], 255 - tid);
    }
  }
  __syncthreads();
  const int dsel = sh.sel[0] >= 0 ? sh.sel[0] : sh.sel[1];
  if (tid < 256 && 255 - tid == dsel) sh.tot = above + (incl - m);
  __syncthreads();
  if (tid == 0) sh.sel[0] = dsel;
  __syncthreads();
}

}  // namespace

constexpr int kLdsVocab = 32768;  // rows up to this size are staged in LDS (128 KB)
constexpr int kCand = 4096;       // top-k sets up to this size are compacted into LDS

// One workgroup of 1024 threads per row. With kLds the row is copied into LDS once (16-byte
// loads, all in flight together) and every pass reads it there; otherwise every pass reads the
// row coalesced from global memory. The fixed-point mass of a token is recomputed from its
// logit wherever it is needed, by the same expression, so every pass sees the same integers.
template <bool kLds>
__global__ __launch_bounds__(kST) void k_sample(const float* __restrict__ logits, int V,
                                                float temperature, int top_k, float top_p,
                                                const float* __restrict__ u,
                                                int32_t* __restrict__ tok_out,
                                                float* __restrict__ lp_beh,
                                                float* __restrict__ lp_model) {
  __shared__ Shared sh;
  __shared__ __attribute__((aligned(16))) float zrow[kLds ? kLdsVocab : 1];
  __shared__ int cand[kCand];
  const int tid = threadIdx.x, row = blockIdx.x, lane = tid % kWave;
  const float* zg = logits + (int64_t)row * V;
  if (kLds) {  // V <= kLdsVocab and a multiple of 64: V / 4 float4 chunks
    for (int c = tid; c < V / 4; c += kST)
      *reinterpret_cast<u32x4*>(&zrow[4 * c]) = ld16(zg + 4 * c);
    __syncthreads();
  }
  const float* z = kLds ? zrow : zg;
  const Range rg(V);
  float mx = -INFINITY;
  for (int i = rg.lo + lane; i < rg.hi; i += kWave) mx = fmaxf(mx, z[i]);
  mx = block_max(mx, sh);

  int a;
  float lpb, log_z1;
  if (!(temperature > 0.f)) {
    float s1 = 0.f;
    for (int i = rg.lo + lane; i < rg.hi; i += kWave) s1 += expf(z[i] - mx);
    log_z1 = logf(block_sum(s1, sh));
    // greedy: the first maximal logit
    a = first_crossing(V, [&](int i) -> u64 { return z[i] == mx ? 1ull : 0ull; }, -1, sh);
    lpb = 0.f;
  } else {
    const float inv_t = 1.f / temperature, mt = mx * inv_t;
    float s1 = 0.f, st = 0.f;
    for (int i = rg.lo + lane; i < rg.hi; i += kWave) {
      const float zi = z[i];
      s1 += expf(zi - mx);
      st += expf(fmaf(zi, inv_t, -mt));
    }
    log_z1 = logf(block_sum(s1, sh));
    st = block_sum(st, sh);
    const float inv_st = 1.f / st;
    // fixed-point mass of token i under the tempered distribution
    auto fq = [&](int i) -> u64 {
      return (u64)((double)(expf(fmaf(z[i], inv_t, -mt)) * inv_st) * kFix + 0.5);
    };

    // top-k: the k-th largest key, and how many of the tokens holding it are kept
    const bool use_k = top_k > 0 && top_k < V;
    uint32_t kth = 0;
    int tie_cut_k = V;
    if (use_k) {
      uint32_t prefix = 0, pmask = 0;
      int remaining = top_k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) sh.cnt[tid] = 0;
        __syncthreads();
        {
          // runs of equal digits are counted in registers and added once (most logits share
          // the leading digit, which would serialise the LDS atomics)
          uint32_t cur = 256u, run = 0u;
          for (int i = rg.lo + lane; i < rg.hi; i += kWave) {
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
        select_count_digit(remaining, sh);
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

    // Top-p and the inverse CDF run over N positions j in ascending token id(j): the compact
    // list of the top-k tokens when there are at most kCand of them, else all V tokens
    // (member(j): token id(j) is in the top-k).
    auto tail = [&](int N, auto id, auto member) {
      const Range rn(N);
      const bool use_p = top_p < 1.f;
      uint32_t thp = 0;
      int tie_cut_p = V;
      if (use_p) {
        u64 mk = 0;
        for (int j = rn.lo + lane; j < rn.hi; j += kWave)
          if (member(j)) mk += fq(id(j));
        const double target = (double)top_p * (double)block_sum_u64(mk, sh);
        uint32_t prefix = 0, pmask = 0;
        u64 above = 0;  // mass of the top-k tokens whose key is above the current digit range
        for (int shift = 24; shift >= 0; shift -= 8) {
          if (tid < 256) {
            sh.cnt[tid] = 0;
            sh.mass[tid] = 0;
          }
          __syncthreads();
          {
            uint32_t cur = 256u, run = 0u;
            u64 msum = 0;
            for (int j = rn.lo + lane; j < rn.hi; j += kWave) {
              const int i = id(j);
              const uint32_t key = order_key(z[i]);
              if ((key & pmask) != prefix || !member(j)) continue;
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
              msum += fq(i);
            }
            if (run) {
              atomicAdd(&sh.cnt[cur], run);
              atomicAdd(&sh.mass[cur], msum);
            }
          }
          __syncthreads();
          select_mass_digit(above, target, sh);
          prefix |= (uint32_t)sh.sel[0] << shift;
          pmask |= 255u << shift;
          above = sh.tot;
          __syncthreads();
        }
        thp = prefix;
        // tokens holding the threshold key, in ascending id, until the mass reaches the target
        const double need = target - (double)above;
        const long long thr = need <= 0.0 ? -1 : (long long)ceil(need) - 1;
        const int jp = first_crossing(
            N,
            [&](int j) -> u64 {
              const int i = id(j);
              return order_key(z[i]) == thp && member(j) ? fq(i) : 0ull;
            },
            thr, sh);
        tie_cut_p = jp < N ? id(jp) : V - 1;  // none reached: every tie is kept
      }
      auto kept = [&](int j) -> bool {
        if (!member(j)) return false;
        if (!use_p) return true;
        const int i = id(j);
        const uint32_t key = order_key(z[i]);
        return key > thp || (key == thp && i <= tie_cut_p);
      };

      // inverse CDF over the kept tokens in ascending id
      u64 mown = 0;
      for (int j = rn.lo + lane; j < rn.hi; j += kWave)
        if (kept(j)) mown += fq(id(j));
      const u64 mass = block_sum_u64(mown, sh);
      u64 tu = (u64)floor((double)u[row] * (double)mass);
      if (tu >= mass) tu = mass - 1;
      const int ja = first_crossing(
          N, [&](int j) -> u64 { return kept(j) ? fq(id(j)) : 0ull; }, (long long)tu, sh);
      // not reached cannot happen: the kept mass is positive and tu < mass
      a = ja < N ? id(ja) : V - 1;
      lpb = (z[a] * inv_t - mt - logf(st)) - logf((float)((double)mass / kFix));
    };

    if (use_k && top_k <= kCand) {
      // the top-k ids in ascending order: per-wave counts, then each wave writes its members
      // strip by strip at its offset (ballot positions within a strip)
      u64 cnt = 0;
      for (int i = rg.lo + lane; i < rg.hi; i += kWave) cnt += in_topk(i) ? 1ull : 0ull;
      cnt = wave_sum_u64(cnt);
      if (lane == 0) sh.wtot[tid / kWave] = cnt;
      __syncthreads();
      int pos = 0, total = 0;
      for (int w = 0; w < kNW; ++w) {
        if (w < tid / kWave) pos += (int)sh.wtot[w];
        total += (int)sh.wtot[w];
      }
      for (int b0 = rg.lo; b0 < rg.hi; b0 += kWave) {
        const int i = b0 + lane;
        const bool m = i < rg.hi && in_topk(i);
        const u64 bal = __ballot(m);
        const int at = pos + __popcll(bal & ((1ull << lane) - 1ull));
        if (m && at < kCand) cand[at] = i;
        pos += __popcll(bal);
      }
      __syncthreads();
      tail(min(total, kCand), [&](int j) -> int { return cand[j]; },
           [](int) -> bool { return true; });
    } else {
      tail(V, [](int j) -> int { return j; }, [&](int j) -> bool { return in_topk(j); });
    }
  }
  if (tid == 0) {
    tok_out[row] = a;
    lp_beh[row] = lpb;
    lp_model[row] = z[a] - mx - log_z1;
  }
}

hipError_t launch_sample(int B, int V, const float* logits, float temperature, int top_k,
                         float top_p, const float* u, int32_t* tokens, float* logp_behaviour,
                         float* logp_model, hipStream_t st) {
  if (V <= kLdsVocab && V % 4 == 0)
    return launch(k_sample<true>, dim3((unsigned)B), dim3(kST), Exec(st), logits, V, temperature,
                  top_k, top_p, u, tokens, logp_behaviour, logp_model);
  return launch(k_sample<false>, dim3((unsigned)B), dim3(kST), Exec(st), logits, V, temperature,
                top_k, top_p, u, tokens, logp_behaviour, logp_model);
}

}  // namespace rlt
