// Internal interface between the C-ABI host code (api.cpp) and the HIP kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "rlt.h"

namespace rlt {

constexpr int kMaxWindow = 1024;
// The memory attention of a small batch (fewer than 128 sequence-head pairs) splits each
// prefix into up to kMaxSplits contiguous parts, one workgroup each, and merges their partial
// softmax states in a second launch.
constexpr int kMaxSplits = 16;
constexpr int64_t kMaxCapacity = (int64_t)1 << 20;  // memory entries per sequence
// Large batches run as row groups of about kGroupRows sequences (multiples of 16), each on its
// own stream, at most kMaxGroups of them: one group's latency-bound projections then overlap
// other groups' bandwidth-bound attention.
#ifndef RLT_GROUP_ROWS
#define RLT_GROUP_ROWS 128
#endif
constexpr int kGroupRows = RLT_GROUP_ROWS;
constexpr int kMaxGroups = 4;

// Where a kernel runs: its stream and, when it is being timed, either a pair of events that the
// launch itself records at the start and at the end of the kernel (hipExtLaunchKernel), or,
// for kernels that stamp themselves (the attention kernels), device slots of two clock values
// per workgroup (its start, its end) that the kernel fills.
struct Exec {
  hipStream_t st;
  hipEvent_t start = nullptr, stop = nullptr;
  unsigned long long* clk = nullptr;
  Exec(hipStream_t s) : st(s) {}  // NOLINT: a plain stream is an untimed Exec
  Exec(hipStream_t s, hipEvent_t a, hipEvent_t b) : st(s), start(a), stop(b) {}
};

template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, const Exec& x,
                         Args... args) {
  if (x.start)
    hipExtLaunchKernelGGL(kernel, grid, block, 0, x.st, x.start, x.stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, 0, x.st, args...);
  return hipGetLastError();
}

// Sizes derived from a validated rlt_config.
struct Dims {
  int d, H, hd, L, F, W, G, dtype;
  float alpha, eps;
  size_t es;  // element size of dtype
};

// Device pointers of the packed weights (all inside the model workspace). Every matrix is
// stored transposed (output-major) in MFMA fragment order (frag_off in common.h).
//   w_gate_t [d][2d]   gate weights
//   wqkv_t   [L][3d][d]
//   wo_t, wcq_t, wco_t [L][d][d]
//   w13_t    [L][2F][d]  rows in blocks of 32: 16 rows of W1^T then the same 16 of W3^T
//   w2_t     [L][d][F]
//   wm_t     [G][2d][d]  W_mK^T rows then W_mV^T rows
//   wocq_t   [L][2d][2d] the self-attention output projection fused with the next
//                        cross-attention query: rows 0..d-1 (outputs h) hold W_o^T in
//                        k = d..2d-1 (k < d is never read); rows d..2d-1 (unnormalised cross
//                        queries) hold (diag(g1) W_cq)^T in k < d and (W_o diag(g1) W_cq)^T in
//                        k >= d, g1 = that layer's cross-attention RMSNorm gain
struct Packed {
  void* w_gate_t;
  float* b_gate;
  float* s_star;
  float* gamma;
  void* wqkv_t;
  void* wo_t;
  void* wcq_t;
  void* wco_t;
  void* w13_t;
  void* w2_t;
  void* wm_t;
  void* wocq_t;
};

// Device buffers of one decoder state (all inside the state buffer).
//   s     [B][d] f32           decoder output s_t
//   ring  [L][B][H][W][hd]     self-attention keys/values; token tau lives in slot tau % W.
//                              W slots hold the W-1 retained entries plus the current one.
//   h, q, qc [B][d] f32        residual stream, self-attention query, cross-attention query
//   hg    [B16][d] dtype       h * gamma of the next RMSNorm (operand of the next projection)
//   ssq   [B][d/32] f32        sums of h^2 over 32-column chunks (that norm's scale)
//   o     [B16][d] dtype       attention output (operand of the output projections)
//   act   [B16][F] dtype       SiLU(f W1) * (f W3)
//   hb    [B16][d] dtype       h in the working dtype (fragment order): operand of the fused
//                              output + cross-query projection
//   pos   [B] int64            tokens each sequence has processed (its position t)
//   part  [B][H][kMaxSplits][hd + 2] f32  partial softmax states of a split memory attention:
//                              per part the unnormalised output (hd), its running max, its sum
// hg, o and act are projection operands in MFMA fragment order, B16 = B rounded up to 16.
struct StateBufs {
  int Bt;  // batch of the whole state: row stride of the per-layer ring blocks
  float* s;
  void* ring_k;
  void* ring_v;
  float* h;
  float* q;
  float* qc;
  void* hg;
  float* ssq;
  void* o;
  void* act;
  void* hb;
  int64_t* pos;
  float* part;
  // rows that take part in the current step (device, one byte per row; NULL: all of them).
  // Other rows compute along but store nothing: their s, ring and position stay as they are.
  const uint8_t* active;
  // the position of every row when the host knows they are all equal, else -1 (kernels then
  // read pos per row); saves a dependent load at the start of each attention block
  int64_t t_uniform;
  // the largest position any row can have (sizes the split of the memory attention)
  int64_t t_max;
};

struct MemBufs {
  void* k;  // [G][B][H][capacity][hd]
  void* v;
  int64_t capacity;
  int Bt;   // batch of the whole memory: row stride of the per-group blocks
};

// The rows [b0, b0 + n) of a state (and of its memory) as a state of n sequences: row-indexed
// buffers are offset, ring/memory blocks keep the whole-batch strides. Sequences are
// independent, so row groups can run on different streams.
StateBufs state_rows(const Dims& D, const StateBufs& S, int b0);
MemBufs memory_rows(const Dims& D, const MemBufs& M, int b0);

// Size of the library-held scratch array of each GPU (rlt_run_parallel_noalloc's workspace).
constexpr size_t kScratchBytes = (size_t)64 << 20;
// The device address of the current device's scratch array (looked up on first use per device).
hipError_t scratch_region(void** out);

// Byte layout of the state buffer; offsets are 256-byte aligned.
struct StateLayout {
  size_t s, ring_k, ring_v, h, q, qc, hg, ssq, o, act, hb, pos, part, total;
};
StateLayout state_layout(const Dims& D, int B);

// ---- launchers (return the first HIP error) -------------------------------------------

// dst rows [row_base + (n / grp) * grp_stride + n % grp] of a [*][K] matrix receive column n
// of src [K][N]; all in dtype.
hipError_t launch_pack_transpose(int dtype, const void* src, int K, int N, void* dst,
                                 int64_t row_base, int grp, int grp_stride, hipStream_t st);

// s = s*, positions 0.
hipError_t launch_reset(const Dims& D, int B, const Packed& P, const StateBufs& S,
                        hipStream_t st);
// Every one of the B positions = t.
hipError_t launch_set_positions(int64_t* pos, int B, int64_t t, hipStream_t st);

// Projects n tokens per sequence into memory entries t0 .. t0+n-1; the encoder outputs of
// sequence b, token i are at e + (b * e_seq + i) * d (elements).
hipError_t launch_memproj(const Dims& D, int B, const Packed& P, const MemBufs& M,
                          const void* e, int64_t e_seq, int64_t t0, int64_t n, const Exec& st);
// The same on the 256 x 256 GEMM (bf16, G * 2 d a multiple of 256), for many tokens.
hipError_t launch_memproj_rows(const Dims& D, int B, const Packed& P, const MemBufs& M,
                               const void* e, int64_t e_seq, int64_t t0, int64_t n,
                               const Exec& st);

// Event timing of selected kernels (owned by a state; see rlt_profile_begin).
struct Profiler {
  struct Rec {
    int kind;
    int ev;       // index of the start event in `events` (the end event follows it), or -1
    int64_t clk;  // with ev = -1: index of the launch's first slot pair in clk_buf
    int64_t nclk; // with ev = -1: slot pairs of the launch (one per workgroup)
    double bytes, flops;
  };
  uint32_t mask = 0;
  int64_t stride = 1;  // decoder-step launches are timed for tokens t0 with t0 % stride == 0
  std::vector<hipEvent_t> events;  // pool, reused across sessions
  std::vector<Rec> recs;
  size_t used = 0;
  // caller-owned device buffer of clk_cap slot pairs (16 bytes each) for self-stamping
  // kernels, one pair per workgroup of each timed launch (or NULL)
  unsigned long long* clk_buf = nullptr;
  int64_t clk_cap = 0, clk_used = 0, clk_dropped = 0;
  bool on(int kind) const { return (mask >> kind) & 1u; }
  // If `kind` is profiled, gives x a fresh pair of timing events for its next launch (or, for
  // a self-stamping kernel of `grid` workgroups while clk_buf is attached, `grid` slot pairs)
  // and records that launch's algorithmic bytes and flops.
  hipError_t arm(int kind, double bytes, double flops, Exec& x, int64_t grid = 0);
  // Sets every clock slot pair to (max, 0) on stream st (a workgroup that left no stamps then
  // shows as a start after its end).
  hipError_t clear_clock(hipStream_t st) const;
  void destroy();
};

// One decoder step of every row of S that is active: row b consumes e_t + b * e_ld (elements)
// at its own position pos[b] (memory must hold entries 0..pos[b]), and its position advances.
// When out != NULL, row b of s is also written to out + b * out_ld (inactive rows: their
// unchanged s). t0 is the largest position, used only to count algorithmic bytes for `prof`.
hipError_t launch_step(const Dims& D, int B, const Packed& P, const StateBufs& S,
                       const MemBufs& M, const void* e_t, int64_t e_ld, int64_t t0,
                       float* out, int64_t out_ld, hipStream_t st, Profiler* prof);

// Workspace of the token-parallel pass (alpha = 0) over n tokens of B sequences; byte offsets.
//   h [B n][d] f32 residual stream; a [R][d] bf16 normed operand (fragment order);
//   q, k, v [B][H][n][hd] bf16; o [R][d], act [R][F] bf16 (fragment order); R = B n rounded up
struct ParLayout {
  size_t h, a, q, k, v, o, act, vt, ssq, total;
};
ParLayout par_layout(const Dims& D, int B, int64_t n);

// The token-parallel pass: memory entries 0..n-1 must be projected; the state must be at
// position 0 (reset). Writes s rows of every token to out (when not NULL; row (b, i) at
// out + b * out_seq + i * d), leaves s = s_n and the ring as n recurrent steps would. bf16 only.
hipError_t launch_parallel(const Dims& D, int B, const Packed& P, const StateBufs& S,
                           const MemBufs& M, const void* e, int64_t e_seq, int64_t n,
                           float* out, int64_t out_seq, void* ws, hipStream_t st,
                           Profiler* prof);

// Parameters of the encoder and the readout around the decoder (inside a head workspace).
//   embed [V][d] dtype (row-major), w_out_t [V][d] dtype (W_out^T in fragment order),
//   enc_gamma [L][2][d], enc_gamma_out [d], out_gamma [d] f32
struct HeadBufs {
  int vocab;
  void* embed;
  void* w_out_t;
  float* enc_gamma;
  float* enc_gamma_out;
  float* out_gamma;
};

// The causal encoder over token ids [B][n] (device int32): writes e [B][n][d] (dtype, row-major).
// Its blocks use the decoder blocks' packed attention and FFN matrices. ws: par_layout(D, B, n)
// bytes. bf16 only.
hipError_t launch_encode(const Dims& D, int B, int64_t n, const Packed& P, const HeadBufs& Hd,
                         const int32_t* tokens, void* e_out, void* ws, hipStream_t st);

// Readout of B rows s [B][d] f32: logits [B][V] f32 = RMSNorm(s; out_gamma) W_out, through
// hg [B16][d] dtype and ssq [B][d/32] f32 scratch.
hipError_t launch_readout_logits(const Dims& D, int B, const HeadBufs& Hd, const float* s,
                                 void* hg, float* ssq, float* logits, hipStream_t st);
// The same logits on the token-parallel 256 x 256 GEMM (bf16, V a multiple of 256): a receives
// bf16(s * gamma / rms(s)) in fragment order (ceil(B / 16) * 16 rows of d).
hipError_t launch_readout_rows(const Dims& D, int B, const HeadBufs& Hd, const float* s, void* a,
                               float* logits, hipStream_t st);
// Sampling from logits [B][V] (row stride V): temperature, top-k, top-p and a uniform u[b] per
// row; token, behaviour log-probability and model log-probability per row.
hipError_t launch_sample(int B, int V, const float* logits, float temperature, int top_k,
                         float top_p, const float* u, int32_t* tokens, float* logp_behaviour,
                         float* logp_model, hipStream_t st);

// Canonical snapshot: row b's retained entries are its tokens pos[b]-n_b .. pos[b]-1 with
// n_b = min(pos[b], W-1), oldest first, zero-padded to W-1. Import sets every position to t.
hipError_t launch_export(const Dims& D, int B, const StateBufs& S, float* s, void* k, void* v,
                         hipStream_t st);
hipError_t launch_import(const Dims& D, int B, const StateBufs& S, int64_t t, const float* s,
                         const void* k, const void* v, hipStream_t st);
// Ring slots from canonical k, v at the positions S.pos already holds.
hipError_t launch_import_caches(const Dims& D, int B, const StateBufs& S, const void* k,
                                const void* v, hipStream_t st);

// ---- kernel-level entry points used by launch_step -----------------------------------------
hipError_t gemm_gate(const Dims& D, int B, const Packed& P, const StateBufs& S, const void* e_t,
                     int64_t e_ld, const Exec& st);
hipError_t gemm_qkv(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                    const Exec& st);
hipError_t gemm_cq(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                   const Exec& st);
// u_save (optional): fp32 [B][2F] copy of the two up-projections (u1 | u3) for the backward pass
hipError_t gemm_w13(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                    const Exec& st, float* u_save = nullptr);
// Fused self-attention output + cross-attention query of layer l (the decoder step's path):
// h1 = h + o W_o (fp32, in S.h, with the 32-column sums of h1^2 in S.ssq) and the unnormalised
// cross query qc = hb diag(g1) W_cq + o W_o diag(g1) W_cq = (h1 * g1) W_cq (fp32, in S.qc); the
// memory attention scales it by 1/rms(h1) (attn_cross with q_unnormalised).
hipError_t gemm_self_out_cq(const Dims& D, int B, int l, const Packed& P, const StateBufs& S,
                            const Exec& st);
// Builds the fused matrices of every layer into P.wocq_t from the unpacked weights (wo, wcq
// [L][d][d], gamma [L][3][d]); tmp: d * d dtype scratch.
hipError_t launch_pack_fused_ocq(const Dims& D, const Packed& P, const void* wo, const void* wcq,
                                 const float* gamma, void* tmp, hipStream_t st);
// h (+)= A W for the output projections: which = 0 (self-attn O), 1 (cross O), 2 (FFN down).
// When dst_s is set the result goes to S.s (and to out rows if out != NULL) instead of h, and
// the positions of the active rows advance: this is the last launch of the step.
hipError_t gemm_residual(const Dims& D, int B, int l, int which, const Packed& P,
                         const StateBufs& S, bool dst_s, float* out, int64_t out_ld,
                         const Exec& st);
// Window attention over the min(t + 1, W) ring slots of each row, memory attention over its
// entries 0..t (t = the row's position).
hipError_t attn_self(const Dims& D, int B, int l, const StateBufs& S, const Exec& st);
// q_unnormalised: S.qc holds (h1 * g1) W_cq and each row's 1/rms(h1) comes from S.ssq.
hipError_t attn_cross(const Dims& D, int B, int l, const StateBufs& S, const MemBufs& M,
                      const Exec& st, bool q_unnormalised = false);
// Whether the memory attention loads its rows with the non-temporal policy (false: ordinary
// loads) for a memory of Bt sequences read up to position t_max.
bool memory_streams(const Dims& D, int Bt, int64_t t_max);
// Parts the memory attention of B rows splits each prefix into when the largest row position is
// t_max (1: one workgroup per sequence and head, no merge launch). The timed main launch has
// B * H * parts workgroups.
int cross_splits(const Dims& D, int B, int64_t t_max);
// Workgroups of an attention launch over `items` (sequence, head, part) items.
int64_t attn_blocks(int64_t items);

// ---- backward pass (backpropagation through time) ----------------------------------------------

// Gradient outputs (device, float32), laid out like the matching rlt_weights fields.
struct GradPtrs {
  float *s_star, *w_gate, *b_gate, *gamma, *wq, *wk, *wv, *wo, *wcq, *wco, *w1, *w3, *w2, *wmk,
      *wmv;
};

// Byte offsets in the workspace of one backward pass over n tokens of B sequences (all 256-byte
// aligned). Tc tokens form one chunk of weight-gradient rows (Mc = Tc * B rows).
struct TrainLayout {
  int64_t Tc, Mc;
  size_t state, mem_k, mem_v, bw, s_hist, xs, ys, zs, qs, qcs, os, ocs, docs, khist, vhist, lse,
      dlt, dres, dn, dattn, u13, gsave, carry, rinv, dkacc, dvacc, ca, cc, cf, cm, yqkv, yo, ycq,
      yco, y13, y2, pg, xg, yg, cspan, part, dkv, o2, tx, ty, total;
};
TrainLayout train_layout(const Dims& D, int B, int64_t n);

// Forward over the n tokens of e [B][n][d] from s* (memory projected inside), keeping what the
// reverse walk needs, then the reverse walk for upstream gradients G [B][n][d]: every field of
// `g` is overwritten with dLoss/dparam for Loss = sum_{b,t} G[b][t] . s_t(b); de [B][n][d]
// (optional) receives dLoss/de; s_traj [B][n][d] (optional) the forward trajectory.
// With `prof`, launches of the kernels it times are timed in the steps of tokens
// i % prof->stride == 0 and everywhere outside the token loops. With `aux` (a second stream,
// and two events for forking to it and joining back), large batches run as two row groups.
// segment > 0: truncation at every segment start of the tensors named by `detach`
// (RLT_DETACH_* bits). With `gs` (a third stream and four events gev: walked[2], done[2]) each
// chunk's weight gradients run there, overlapping the walk of the next chunk.
hipError_t launch_bptt(const Dims& D, int B, int64_t n, const Packed& P, const void* e,
                       const float* G, float* s_traj, const GradPtrs& g, float* de, void* ws,
                       int64_t segment, uint32_t detach, hipStream_t st, hipStream_t aux,
                       hipEvent_t ev_fork, hipEvent_t ev_join, hipStream_t gs,
                       const hipEvent_t* gev, Profiler* prof);

}  // namespace rlt
