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

// Calls f(i, z[i]) for this lane's ids of the wave range r, eight 64-id strips at a time with
// their eight loads issued before any is used.
template <class F>
__device__ __forceinline__ void for_lane(const Range& r, const float* z, F f) {
  const int lane = threadIdx.x % kWave;
  for (int b0 = r.lo; b0 < r.hi; b0 += 8 * kWave) {
    float v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = b0 + q * kWave + lane;
      v[q] = i < r.hi ? z[i] : 0.f;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int i = b0 + q * kWave + lane;
      if (i < r.hi) f(i, v[q]);
    }
  }
}

// The first id, in ascending order, at which the running sum of w(i) over ids with w(i) > 0
// exceeds thr (thr < 0: the first id with w(i) > 0); V if none. All threads get the result.
// Within its wave range every lane owns a contiguous run of ids: the lane sums (integers, so
// the order of addition is free; each lane starts at its own offset so that the 64 lanes read
// different LDS banks), one lane scan in the wave that holds the crossing, and a sequential
// walk by the one lane that holds it.
template <class Wt>
__device__ int first_crossing(int V, Wt w, long long thr, Shared& sh) {
  const Range r(V);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int per = (r.hi - r.lo + kWave - 1) / kWave;  // ids per lane (the last lanes fewer)
  const int l0 = min(r.hi, r.lo + lane * per), l1 = min(r.hi, l0 + per), len = l1 - l0;
  u64 own = 0;
  const int start = len > 0 ? lane % len : 0;
  for (int j0 = 0; j0 < len; j0 += 8) {
    u64 x[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      int jj = start + j0 + q;
      jj -= jj >= len ? len : 0;
      x[q] = j0 + q < len ? w(l0 + jj) : 0ull;
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) own += x[q];
  }
  const u64 wsum = wave_sum_u64(own);
  if (lane == 0) sh.wtot[wave] = wsum;
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
    const u64 incl = wave_incl_scan(own);
    const u64 hit = __ballot(own > 0 && (long long)(before + incl) > thr);
    if (hit && lane == __ffsll((unsigned long long)hit) - 1) {
      u64 acc = before + incl - own;
      for (int i = l0; i < l1; ++i) {
        const u64 x = w(i);
        acc += x;
        if (x > 0 && (long long)acc > thr) {
          sh.sel[0] = i;
          break;
        }
      }
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
static_assert(kCand >= kNW * 256, "the candidate list holds the per-wave digit histograms");

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
  for_lane(rg, z, [&](int, float zi) { mx = fmaxf(mx, zi); });
  mx = block_max(mx, sh);

  int a;
  float lpb, log_z1;
  if (!(temperature > 0.f)) {
    float s1 = 0.f;
    for_lane(rg, z, [&](int, float zi) { s1 += __expf(zi - mx); });
    log_z1 = logf(block_sum(s1, sh));
    // greedy: the first maximal logit
    a = first_crossing(V, [&](int i) -> u64 { return z[i] == mx ? 1ull : 0ull; }, -1, sh);
    lpb = 0.f;
  } else {
    const float inv_t = 1.f / temperature, mt = mx * inv_t;
    float s1 = 0.f, st = 0.f;
    // the normalisers use the hardware exponential: st scales every fixed-point mass by the
    // same factor, which cancels in every decision (all of them compare ratios of masses)
    for_lane(rg, z, [&](int, float zi) {
      s1 += __expf(zi - mx);
      st += __expf(fmaf(zi, inv_t, -mt));
    });
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
    int tie_cut_k = V, ties_kept = 0;
    if (use_k) {
      uint32_t prefix = 0, pmask = 0;
      int remaining = top_k;
      for (int shift = 24; shift >= 0; shift -= 8) {
        // per-wave histograms (in the candidate list's LDS, unused until the selection is
        // done), so that waves do not contend for the few digits most logits share; runs of
        // equal digits in a lane are added once
        uint32_t* hist = reinterpret_cast<uint32_t*>(cand) + (tid / kWave) * 256;
        for (int j = tid; j < kNW * 256; j += kST) reinterpret_cast<uint32_t*>(cand)[j] = 0;
        __syncthreads();
        {
          uint32_t cur = 256u, run = 0u;
          for_lane(rg, z, [&](int, float zi) {
            const uint32_t key = order_key(zi);
            if ((key & pmask) != prefix) return;
            const uint32_t dg = (key >> shift) & 255u;
            if (dg != cur) {
              if (run) atomicAdd(&hist[cur], run);
              cur = dg;
              run = 0u;
            }
            ++run;
          });
          if (run) atomicAdd(&hist[cur], run);
        }
        __syncthreads();
        if (tid < 256) {
          uint32_t c = 0;
          for (int w = 0; w < kNW; ++w) c += reinterpret_cast<const uint32_t*>(cand)[w * 256 + tid];
          sh.cnt[tid] = c;
        }
        __syncthreads();
        select_count_digit(remaining, sh);
        prefix |= (uint32_t)sh.sel[0] << shift;
        pmask |= 255u << shift;
        remaining = sh.sel[1];
        __syncthreads();
      }
      kth = prefix;
      ties_kept = remaining;  // the first `remaining` tokens holding the k-th key, by id
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

    // The ids holding a key >= kth (the top-k and every tie at its boundary) in ascending
    // order, when there are at most kCand: per-wave counts, then each wave writes its ids strip
    // by strip at its offset (ballot positions within a strip). The ties kept are then found
    // on that list; more ids, or no top-k, and the same is done over all V tokens.
    int total = kCand + 1;
    if (use_k && top_k <= kCand) {
      u64 cnt = 0;
      for_lane(rg, z, [&](int, float zi) { cnt += order_key(zi) >= kth ? 1ull : 0ull; });
      cnt = wave_sum_u64(cnt);
      if (lane == 0) sh.wtot[tid / kWave] = cnt;
      __syncthreads();
      int pos = 0;
      total = 0;
      for (int w = 0; w < kNW; ++w) {
        if (w < tid / kWave) pos += (int)sh.wtot[w];
        total += (int)sh.wtot[w];
      }
      if (total <= kCand) {
        for (int b0 = rg.lo; b0 < rg.hi; b0 += 8 * kWave) {
          float v[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int i = b0 + q * kWave + lane;
            v[q] = i < rg.hi ? z[i] : 0.f;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int i = b0 + q * kWave + lane;
            const bool m = i < rg.hi && order_key(v[q]) >= kth;
            const u64 bal = __ballot(m);
            if (m) cand[pos + __popcll(bal & ((1ull << lane) - 1ull))] = i;
            pos += __popcll(bal);
          }
        }
      }
      __syncthreads();
    }
    if (total <= kWave) {
      // At most 64 candidates: wave 0 holds one per lane (ascending id = ascending lane) and
      // takes every decision with lane operations. Top-k keeps the ties at kth of rank below
      // ties_kept; top-p keeps a member when the mass of the members before it in the
      // nucleus order (key descending, id ascending) is still below the target, which is the
      // shortest prefix reaching it; the action is the first kept member, by id, whose
      // inclusive kept mass exceeds floor(u * mass).
      if (tid < kWave) {
        const bool valid = lane < total;
        const int i = valid ? cand[lane] : 0;
        const uint32_t key = valid ? order_key(z[i]) : 0u;
        const u64 ties = __ballot(valid && key == kth);
        const int rank = __popcll(ties & ((1ull << lane) - 1ull));
        const bool mem = valid && (key > kth || (key == kth && rank < ties_kept));
        const u64 f = mem ? fq(i) : 0ull;
        bool keep = mem;
        if (top_p < 1.f) {
          const double target = (double)top_p * (double)wave_sum_u64(f);
          u64 before = 0;
          for (int o = 0; o < kWave; ++o) {
            const uint32_t ko = __shfl(key, o, kWave);
            const u64 fo = __shfl(f, o, kWave);
            before += (ko > key || (ko == key && o < lane)) ? fo : 0ull;
          }
          keep = mem && (double)before < target;
        }
        const u64 kf = keep ? f : 0ull;
        const u64 incl = wave_incl_scan(kf);
        const u64 mass = __shfl(incl, kWave - 1, kWave);
        u64 tu = (u64)floor((double)u[row] * (double)mass);
        if (tu >= mass) tu = mass - 1;
        const u64 hit = __ballot(kf > 0 && incl > tu);
        if (lane == 0) {
          // hit != 0: the kept mass is positive and tu < mass
          sh.sel[0] = hit ? cand[__ffsll((unsigned long long)hit) - 1] : V - 1;
          sh.tot = mass;
        }
      }
      __syncthreads();
      a = sh.sel[0];
      lpb = (z[a] * inv_t - mt - logf(st)) - logf((float)((double)sh.tot / kFix));
    } else if (total <= kCand) {
      const int jt = first_crossing(
          total, [&](int j) -> u64 { return order_key(z[cand[j]]) == kth ? 1ull : 0ull; },
          (long long)ties_kept - 1, sh);
      tie_cut_k = cand[jt];  // jt < total: at least ties_kept ties are listed
      tail(total, [&](int j) -> int { return cand[j]; },
           [&](int j) -> bool { return in_topk(cand[j]); });
    } else {
      if (use_k)
        tie_cut_k = first_crossing(
            V, [&](int i) -> u64 { return order_key(z[i]) == kth ? 1ull : 0ull; },
            (long long)ties_kept - 1, sh);
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
