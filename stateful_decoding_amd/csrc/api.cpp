// Host side of the C ABI declared in include/rlt.h: argument validation, handle bookkeeping,
// buffer layouts and the sequencing of kernel launches. Validation always completes before
// anything is enqueued, so a rejected call leaves every handle and buffer untouched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"

using namespace rlt;

struct rlt_model {
  rlt_config cfg;
  Dims D;
  Packed P;
  // second stream and fork/join events of rlt_bptt's row groups, created on its first call
  hipStream_t bwd_aux = nullptr;
  hipEvent_t bwd_fork = nullptr, bwd_join = nullptr;
  // the backward pass's weight-gradient stream and its events (walked[2], done[2])
  hipStream_t bwd_grads = nullptr;
  hipEvent_t bwd_gev[4] = {nullptr, nullptr, nullptr, nullptr};
};

struct rlt_state {
  const rlt_model* model;
  int B;
  // tokens processed: every row's position while `ragged` is false; once a step ran with an
  // active mask, the largest position any row can have (an upper bound)
  int64_t t;
  bool ragged;
  StateBufs S;
  Profiler prof;
  // row groups: group g is rows [row0[g], row0[g + 1]); group 0 runs on the caller's stream,
  // group g > 0 on aux[g], forked from and joined back to it with events
  int ngroups;
  int row0[kMaxGroups + 1];
  hipStream_t aux[kMaxGroups];
  hipEvent_t fork, join[kMaxGroups];
};

struct rlt_memory {
  const rlt_model* model;
  int B;
  int64_t len;
  MemBufs M;
};

struct rlt_head {
  const rlt_model* model;
  HeadBufs Hd;
};

namespace {

thread_local std::string g_err;

rlt_status fail(rlt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

rlt_status ok() {
  g_err.clear();
  return RLT_OK;
}

rlt_status hip_fail(hipError_t e, const char* what) {
  return fail(RLT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) % 16) == 0; }

rlt_status check_config(const rlt_config* c) {
  if (!c) return fail(RLT_ERR_ARG, "config is NULL");
  if (c->dtype != RLT_F32 && c->dtype != RLT_BF16)
    return fail(RLT_ERR_DTYPE, "unknown dtype %d", c->dtype);
  if (c->d <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->n_layers <= 0 || c->ffn <= 0 ||
      c->window <= 0 || c->n_groups <= 0)
    return fail(RLT_ERR_SHAPE, "all sizes must be positive");
  if ((int64_t)c->n_heads * c->head_dim != c->d)
    return fail(RLT_ERR_SHAPE, "d (%d) must equal n_heads (%d) * head_dim (%d)", c->d, c->n_heads,
                c->head_dim);
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
    return fail(RLT_ERR_SHAPE, "head_dim %d unsupported (32, 64 or 128)", c->head_dim);
  if (c->d % 64 != 0) return fail(RLT_ERR_SHAPE, "d (%d) must be a multiple of 64", c->d);
  if (c->ffn % 64 != 0) return fail(RLT_ERR_SHAPE, "ffn (%d) must be a multiple of 64", c->ffn);
  if (c->d > 16384 || c->ffn > 65536 || c->n_layers > 4096)
    return fail(RLT_ERR_SHAPE, "sizes beyond the supported range");
  if (c->window > kMaxWindow)
    return fail(RLT_ERR_SHAPE, "window %d exceeds %d", c->window, kMaxWindow);
  if (c->n_groups != 1 && c->n_groups != c->n_layers)
    return fail(RLT_ERR_SHAPE, "n_groups must be 1 or n_layers (%d), got %d", c->n_layers,
                c->n_groups);
  if (!std::isfinite(c->alpha)) return fail(RLT_ERR_ARG, "alpha must be finite");
  if (!std::isfinite(c->eps) || c->eps < 0.f) return fail(RLT_ERR_ARG, "eps must be >= 0");
  return ok();
}

Dims dims_of(const rlt_config& c) {
  Dims D;
  D.d = c.d; D.H = c.n_heads; D.hd = c.head_dim; D.L = c.n_layers; D.F = c.ffn; D.W = c.window;
  D.G = c.n_groups; D.dtype = c.dtype; D.alpha = c.alpha; D.eps = c.eps;
  D.es = c.dtype == RLT_BF16 ? 2 : 4;
  return D;
}

struct ModelLayout {
  size_t w_gate_t, b_gate, s_star, gamma, wqkv_t, wo_t, wcq_t, wco_t, w13_t, w2_t, wm_t, wocq_t,
      fuse_tmp, total;
};

ModelLayout model_layout(const Dims& D) {
  ModelLayout m;
  size_t o = 0;
  const size_t d = D.d, L = D.L, F = D.F, G = D.G, es = D.es;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  m.w_gate_t = take(2 * d * d * es);
  m.b_gate = take(d * 4);
  m.s_star = take(d * 4);
  m.gamma = take(L * 3 * d * 4);
  m.wqkv_t = take(L * 3 * d * d * es);
  m.wo_t = take(L * d * d * es);
  m.wcq_t = take(L * d * d * es);
  m.wco_t = take(L * d * d * es);
  m.w13_t = take(L * 2 * F * d * es);
  m.w2_t = take(L * F * d * es);
  m.wm_t = take(G * 2 * d * d * es);
  m.wocq_t = take(L * 4 * d * d * es);
  m.fuse_tmp = take(d * d * es);
  m.total = o;
  return m;
}

template <typename P>
P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(base) + off);
}

bool valid_batch(int B) { return B >= 1 && B <= (1 << 20); }

constexpr int kMaxVocab = 1 << 22;

struct HeadLayout {
  size_t embed, w_out_t, enc_gamma, enc_gamma_out, out_gamma, total;
};

HeadLayout head_layout(const Dims& D, int V) {
  HeadLayout h;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  h.embed = take((size_t)V * D.d * D.es);
  h.w_out_t = take((size_t)V * D.d * D.es);
  h.enc_gamma = take((size_t)D.L * 2 * D.d * 4);
  h.enc_gamma_out = take((size_t)D.d * 4);
  h.out_gamma = take((size_t)D.d * 4);
  h.total = o;
  return h;
}

bool valid_vocab(int V) { return V >= 64 && V <= kMaxVocab && V % 64 == 0; }

struct ReadoutLayout {
  size_t hg, ssq, logits, total;
};

ReadoutLayout readout_layout(const Dims& D, int V, int B) {
  ReadoutLayout r;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t b16 = ((size_t)B + 15) / 16 * 16;
  r.hg = take(b16 * D.d * D.es);
  r.ssq = take((size_t)B * (D.d / 32) * 4);
  r.logits = take((size_t)B * V * 4);
  r.total = o;
  return r;
}

}  // namespace

namespace rlt {
StateLayout state_layout(const Dims& D, int B) {
  StateLayout s;
  size_t o = 0;
  const size_t b = B, d = D.d, es = D.es, b16 = (b + 15) / 16 * 16;
  auto take = [&](size_t bytes) {
    size_t a = o;
    o = align_up(o + bytes);
    return a;
  };
  const size_t ring = (size_t)D.L * b * D.H * D.W * D.hd * es;
  s.s = take(b * d * 4);
  s.ring_k = take(ring);
  s.ring_v = take(ring);
  s.h = take(b * d * 4);
  s.q = take(b * d * 4);
  s.qc = take(b * d * 4);
  s.hg = take(b16 * d * es);
  s.ssq = take(b * (d / 32) * 4);
  s.o = take(b16 * d * es);
  s.act = take(b16 * D.F * es);
  s.hb = take(b16 * d * es);
  s.pos = take(b * 8);
  s.part = take(b * D.H * kMaxSplits * (D.hd + 2) * 4);
  s.total = o;
  return s;
}
}  // namespace rlt

extern "C" {

const char* rlt_last_error(void) { return g_err.c_str(); }

rlt_status rlt_config_check(const rlt_config* cfg) { return check_config(cfg); }

size_t rlt_model_ws_bytes(const rlt_config* cfg) {
  if (check_config(cfg) != RLT_OK) return 0;
  return model_layout(dims_of(*cfg)).total;
}

rlt_status rlt_model_create(const rlt_config* cfg, const rlt_weights* w, void* ws,
                            size_t ws_bytes, void* stream, rlt_model** out) {
  if (rlt_status s = check_config(cfg)) return s;
  if (!w || !ws || !out) return fail(RLT_ERR_ARG, "weights, workspace and out must be non-NULL");
  const void* ptrs[] = {w->s_star, w->w_gate, w->b_gate, w->gamma, w->wq, w->wk, w->wv, w->wo,
                        w->wcq, w->wco, w->w1, w->w3, w->w2, w->wmk, w->wmv};
  for (const void* p : ptrs)
    if (!p) return fail(RLT_ERR_ARG, "a weight pointer is NULL");
  const Dims D = dims_of(*cfg);
  const ModelLayout m = model_layout(D);
  if (ws_bytes < m.total)
    return fail(RLT_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, m.total);
  if (!aligned(ws)) return fail(RLT_ERR_ARG, "workspace must be 256-byte aligned");

  rlt_model* mdl = new (std::nothrow) rlt_model;
  if (!mdl) return fail(RLT_ERR_ARG, "out of host memory");
  mdl->cfg = *cfg;
  mdl->D = D;
  Packed& P = mdl->P;
  P.w_gate_t = at<char>(ws, m.w_gate_t);
  P.b_gate = at<float>(ws, m.b_gate);
  P.s_star = at<float>(ws, m.s_star);
  P.gamma = at<float>(ws, m.gamma);
  P.wqkv_t = at<char>(ws, m.wqkv_t);
  P.wo_t = at<char>(ws, m.wo_t);
  P.wcq_t = at<char>(ws, m.wcq_t);
  P.wco_t = at<char>(ws, m.wco_t);
  P.w13_t = at<char>(ws, m.w13_t);
  P.w2_t = at<char>(ws, m.w2_t);
  P.wm_t = at<char>(ws, m.wm_t);
  P.wocq_t = at<char>(ws, m.wocq_t);

  hipStream_t st = static_cast<hipStream_t>(stream);
  const int d = D.d, F = D.F, dt = D.dtype;
  const size_t es = D.es;
  hipError_t e = hipSuccess;
  auto src = [&](const void* base, size_t elems) {
    return static_cast<const char*>(base) + elems * es;
  };
  auto dst = [&](void* base, size_t elems) { return static_cast<char*>(base) + elems * es; };
#define RLT_PACK(call)                 \
  if (e == hipSuccess) e = (call)
  RLT_PACK(launch_pack_transpose(dt, w->w_gate, 2 * d, d, P.w_gate_t, 0, d, d, st));
  RLT_PACK(hipMemcpyAsync(P.b_gate, w->b_gate, d * 4, hipMemcpyDeviceToDevice, st));
  RLT_PACK(hipMemcpyAsync(P.s_star, w->s_star, d * 4, hipMemcpyDeviceToDevice, st));
  RLT_PACK(hipMemcpyAsync(P.gamma, w->gamma, (size_t)D.L * 3 * d * 4, hipMemcpyDeviceToDevice, st));
  for (int l = 0; l < D.L && e == hipSuccess; ++l) {
    const size_t dd = (size_t)l * d * d, df = (size_t)l * d * F;
    void* qkv = dst(P.wqkv_t, (size_t)l * 3 * d * d);
    RLT_PACK(launch_pack_transpose(dt, src(w->wq, dd), d, d, qkv, 0, d, d, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->wk, dd), d, d, qkv, d, d, d, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->wv, dd), d, d, qkv, 2 * d, d, d, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->wo, dd), d, d, dst(P.wo_t, dd), 0, d, d, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->wcq, dd), d, d, dst(P.wcq_t, dd), 0, d, d, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->wco, dd), d, d, dst(P.wco_t, dd), 0, d, d, st));
    void* w13 = dst(P.w13_t, (size_t)l * 2 * F * d);
    RLT_PACK(launch_pack_transpose(dt, src(w->w1, df), d, F, w13, 0, 16, 32, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->w3, df), d, F, w13, 16, 16, 32, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->w2, df), F, d, dst(P.w2_t, df), 0, d, d, st));
  }
  for (int g = 0; g < D.G && e == hipSuccess; ++g) {
    const size_t dd = (size_t)g * d * d;
    void* wm = dst(P.wm_t, (size_t)g * 2 * d * d);
    RLT_PACK(launch_pack_transpose(dt, src(w->wmk, dd), d, d, wm, 0, d, d, st));
    RLT_PACK(launch_pack_transpose(dt, src(w->wmv, dd), d, d, wm, d, d, d, st));
  }
  RLT_PACK(launch_pack_fused_ocq(D, P, w->wo, w->wcq, w->gamma, at<char>(ws, m.fuse_tmp), st));
#undef RLT_PACK
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    delete mdl;
    return hip_fail(e, "packing weights");
  }
  *out = mdl;
  return ok();
}

void rlt_model_destroy(rlt_model* model) {
  if (!model) return;
  if (model->bwd_aux) (void)hipStreamDestroy(model->bwd_aux);
  if (model->bwd_fork) (void)hipEventDestroy(model->bwd_fork);
  if (model->bwd_join) (void)hipEventDestroy(model->bwd_join);
  if (model->bwd_grads) (void)hipStreamDestroy(model->bwd_grads);
  for (hipEvent_t ev : model->bwd_gev)
    if (ev) (void)hipEventDestroy(ev);
  delete model;
}

size_t rlt_state_bytes(const rlt_config* cfg, int32_t batch) {
  if (check_config(cfg) != RLT_OK || !valid_batch(batch)) return 0;
  return state_layout(dims_of(*cfg), batch).total;
}

rlt_status rlt_state_create(const rlt_model* model, int32_t batch, void* buf, size_t bytes,
                            void* stream, rlt_state** out) {
  if (!model || !buf || !out) return fail(RLT_ERR_ARG, "model, buffer and out must be non-NULL");
  if (!valid_batch(batch)) return fail(RLT_ERR_SHAPE, "batch %d out of range", batch);
  if (!aligned(buf)) return fail(RLT_ERR_ARG, "state buffer must be 256-byte aligned");
  const StateLayout L = state_layout(model->D, batch);
  if (bytes < L.total)
    return fail(RLT_ERR_CAPACITY, "state buffer has %zu bytes, needs %zu", bytes, L.total);
  rlt_state* s = new (std::nothrow) rlt_state;
  if (!s) return fail(RLT_ERR_ARG, "out of host memory");
  s->model = model;
  s->B = batch;
  s->t = 0;
  s->S.s = at<float>(buf, L.s);
  s->S.ring_k = at<char>(buf, L.ring_k);
  s->S.ring_v = at<char>(buf, L.ring_v);
  s->S.h = at<float>(buf, L.h);
  s->S.q = at<float>(buf, L.q);
  s->S.qc = at<float>(buf, L.qc);
  s->S.hg = at<char>(buf, L.hg);
  s->S.ssq = at<float>(buf, L.ssq);
  s->S.o = at<char>(buf, L.o);
  s->S.act = at<char>(buf, L.act);
  s->S.hb = at<char>(buf, L.hb);
  s->S.pos = at<int64_t>(buf, L.pos);
  s->S.part = at<float>(buf, L.part);
  s->S.active = nullptr;
  s->S.t_uniform = -1;
  s->S.t_max = 0;
  s->S.Bt = batch;
  s->ragged = false;
  s->fork = nullptr;
  for (int g = 0; g < kMaxGroups; ++g) {
    s->aux[g] = nullptr;
    s->join[g] = nullptr;
  }
  int ng = batch / kGroupRows;
  ng = ng < 1 ? 1 : ng > kMaxGroups ? kMaxGroups : ng;
  const int per = ((batch + ng - 1) / ng + 15) / 16 * 16;
  s->ngroups = 0;
  for (int g = 0; g < ng && g * per < batch; ++g) {
    s->row0[g] = g * per;
    s->ngroups = g + 1;
  }
  s->row0[s->ngroups] = batch;
  hipError_t e = hipSuccess;
  if (s->ngroups > 1) e = hipEventCreateWithFlags(&s->fork, hipEventDisableTiming);
  for (int g = 1; g < s->ngroups && e == hipSuccess; ++g) {
    e = hipStreamCreateWithFlags(&s->aux[g], hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&s->join[g], hipEventDisableTiming);
  }
  if (e != hipSuccess) {
    rlt_state_destroy(s);
    return hip_fail(e, "creating the row-group streams");
  }
  e = launch_reset(model->D, batch, model->P, s->S, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    rlt_state_destroy(s);  // also frees the row-group streams and events created above
    return hip_fail(e, "state reset");
  }
  *out = s;
  return ok();
}

rlt_status rlt_state_reset(rlt_state* state, void* stream) {
  if (!state) return fail(RLT_ERR_ARG, "state is NULL");
  hipError_t e = launch_reset(state->model->D, state->B, state->model->P, state->S,
                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "state reset");
  state->t = 0;
  state->ragged = false;
  return ok();
}

rlt_status rlt_state_positions(const rlt_state* state, int64_t* out, void* stream) {
  if (!state || !out) return fail(RLT_ERR_ARG, "state and out must be non-NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(out, state->S.pos, sizeof(int64_t) * (size_t)state->B,
                                hipMemcpyDeviceToHost, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "reading positions");
  return ok();
}

int64_t rlt_state_position(const rlt_state* state) {
  return state && !state->ragged ? state->t : -1;
}
void rlt_state_destroy(rlt_state* state) {
  if (!state) return;
  state->prof.destroy();
  if (state->fork) (void)hipEventDestroy(state->fork);
  for (int g = 0; g < kMaxGroups; ++g) {
    if (state->join[g]) (void)hipEventDestroy(state->join[g]);
    if (state->aux[g]) (void)hipStreamDestroy(state->aux[g]);
  }
  delete state;
}

size_t rlt_memory_bytes(const rlt_config* cfg, int32_t batch, int64_t capacity) {
  if (check_config(cfg) != RLT_OK || !valid_batch(batch) || capacity < 1 ||
      capacity > kMaxCapacity)
    return 0;
  const Dims D = dims_of(*cfg);
  return 2 * align_up((size_t)D.G * batch * D.H * capacity * D.hd * D.es);
}

rlt_status rlt_memory_create(const rlt_model* model, int32_t batch, int64_t capacity, void* buf,
                             size_t bytes, rlt_memory** out) {
  if (!model || !buf || !out) return fail(RLT_ERR_ARG, "model, buffer and out must be non-NULL");
  if (!valid_batch(batch)) return fail(RLT_ERR_SHAPE, "batch %d out of range", batch);
  if (capacity < 1 || capacity > kMaxCapacity)
    return fail(RLT_ERR_CAPACITY, "capacity %lld outside [1, %lld]", (long long)capacity,
                (long long)kMaxCapacity);
  if (!aligned(buf)) return fail(RLT_ERR_ARG, "memory buffer must be 256-byte aligned");
  const Dims& D = model->D;
  const size_t half = align_up((size_t)D.G * batch * D.H * capacity * D.hd * D.es);
  if (bytes < 2 * half)
    return fail(RLT_ERR_CAPACITY, "memory buffer has %zu bytes, needs %zu", bytes, 2 * half);
  rlt_memory* m = new (std::nothrow) rlt_memory;
  if (!m) return fail(RLT_ERR_ARG, "out of host memory");
  m->model = model;
  m->B = batch;
  m->len = 0;
  m->M.k = buf;
  m->M.v = at<char>(buf, half);
  m->M.capacity = capacity;
  m->M.Bt = batch;
  *out = m;
  return ok();
}

int64_t rlt_memory_length(const rlt_memory* mem) { return mem ? mem->len : -1; }

rlt_status rlt_memory_reset(rlt_memory* mem) {
  if (!mem) return fail(RLT_ERR_ARG, "memory is NULL");
  mem->len = 0;
  return ok();
}
void rlt_memory_destroy(rlt_memory* mem) { delete mem; }

rlt_status rlt_memproj(const rlt_model* model, rlt_memory* mem, const void* e, int64_t t0,
                       int64_t n, void* stream) {
  if (!model || !mem || !e) return fail(RLT_ERR_ARG, "model, memory and e must be non-NULL");
  if (mem->model != model) return fail(RLT_ERR_ARG, "memory belongs to another model");
  if (!aligned16(e)) return fail(RLT_ERR_ARG, "e must be 16-byte aligned");
  if (n < 1) return fail(RLT_ERR_ARG, "n must be >= 1");
  if (t0 < 0 || t0 > mem->len)
    return fail(RLT_ERR_NOT_PROJECTED, "t0 %lld leaves a hole (memory length %lld)",
                (long long)t0, (long long)mem->len);
  if (t0 + n > mem->M.capacity)
    return fail(RLT_ERR_CAPACITY, "tokens up to %lld exceed capacity %lld", (long long)(t0 + n),
                (long long)mem->M.capacity);
  hipError_t err = launch_memproj(model->D, mem->B, model->P, mem->M, e, n, t0, n,
                                  static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "memory projection");
  if (t0 + n > mem->len) mem->len = t0 + n;
  return ok();
}

// n decoder steps over e rows (b, i) at e + (b * e_ld + i * d), s rows to out (+ b * out_ld
// + i * d) when out != NULL; every row group on its own stream, all forked from and joined
// back to `st`. Launches are issued step by step, alternating between the groups.
static hipError_t run_steps(const rlt_model* model, rlt_state* state, const rlt_memory* mem,
                            const void* e, int64_t e_ld, int64_t n, float* out, int64_t out_ld,
                            hipStream_t st, const uint8_t* active = nullptr) {
  const Dims& D = model->D;
  const int ng = state->ngroups;
  hipError_t err = hipSuccess;
  if (ng > 1) {
    err = hipEventRecord(state->fork, st);
    for (int g = 0; g < ng && err == hipSuccess; ++g)
      if (state->aux[g]) err = hipStreamWaitEvent(state->aux[g], state->fork, 0);
    if (err != hipSuccess) return err;
  }
  StateBufs Sg[kMaxGroups];
  MemBufs Mg[kMaxGroups];
  StateBufs S = state->S;
  S.active = active;
  for (int g = 0; g < ng; ++g) {
    Sg[g] = state_rows(D, S, state->row0[g]);
    Mg[g] = memory_rows(D, mem->M, state->row0[g]);
  }
  const char* eb = static_cast<const char*>(e);
  for (int64_t i = 0; i < n && err == hipSuccess; ++i) {
    const int64_t t0 = state->t + i;
    for (int g = 0; g < ng; ++g) {
      Sg[g].t_uniform = state->ragged ? -1 : t0;
      Sg[g].t_max = t0;
    }
    for (int g = 0; g < ng && err == hipSuccess; ++g) {
      const int b0 = state->row0[g], rows = state->row0[g + 1] - b0;
      const char* et = eb + ((size_t)b0 * e_ld + (size_t)i * D.d) * D.es;
      float* o = out ? out + (size_t)b0 * out_ld + (size_t)i * D.d : nullptr;
      err = launch_step(D, rows, model->P, Sg[g], Mg[g], et, e_ld, t0, o, out_ld,
                        state->aux[g] ? state->aux[g] : st,
                        t0 % state->prof.stride == 0 ? &state->prof : nullptr);
    }
  }
  for (int g = 0; g < ng && err == hipSuccess; ++g) {
    if (!state->aux[g]) continue;
    err = hipEventRecord(state->join[g], state->aux[g]);
    if (err == hipSuccess) err = hipStreamWaitEvent(st, state->join[g], 0);
  }
  return err;
}

static rlt_status check_step_args(const rlt_model* model, const rlt_state* state,
                                  const rlt_memory* mem) {
  if (!model || !state || !mem) return fail(RLT_ERR_ARG, "model, state and memory must be non-NULL");
  if (state->model != model || mem->model != model)
    return fail(RLT_ERR_ARG, "state or memory belongs to another model");
  if (state->B != mem->B)
    return fail(RLT_ERR_SHAPE, "state batch %d != memory batch %d", state->B, mem->B);
  return ok();
}

rlt_status rlt_decoder_step(const rlt_model* model, rlt_state* state, const rlt_memory* mem,
                            const void* e_t, float* s_out, void* stream) {
  if (rlt_status s = check_step_args(model, state, mem)) return s;
  if (!e_t) return fail(RLT_ERR_ARG, "e_t is NULL");
  if (!aligned16(e_t) || (s_out && !aligned16(s_out)))
    return fail(RLT_ERR_ARG, "e_t and s_out must be 16-byte aligned");
  if (mem->len < state->t + 1)
    return fail(RLT_ERR_NOT_PROJECTED, "token %lld needs memory length %lld, have %lld",
                (long long)(state->t + 1), (long long)(state->t + 1), (long long)mem->len);
  const Dims& D = model->D;
  hipError_t e = run_steps(model, state, mem, e_t, D.d, 1, s_out, D.d,
                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decoder step");
  state->t += 1;
  return ok();
}

rlt_status rlt_decoder_step_ragged(const rlt_model* model, rlt_state* state,
                                   const rlt_memory* mem, const void* e_t, const uint8_t* active,
                                   float* s_out, void* stream) {
  if (rlt_status s = check_step_args(model, state, mem)) return s;
  if (!e_t) return fail(RLT_ERR_ARG, "e_t is NULL");
  if (!aligned16(e_t) || (s_out && !aligned16(s_out)))
    return fail(RLT_ERR_ARG, "e_t and s_out must be 16-byte aligned");
  if (mem->len < state->t + 1)
    return fail(RLT_ERR_NOT_PROJECTED, "positions up to %lld need memory length %lld, have %lld",
                (long long)state->t, (long long)(state->t + 1), (long long)mem->len);
  const Dims& D = model->D;
  hipError_t e = run_steps(model, state, mem, e_t, D.d, 1, s_out, D.d,
                           static_cast<hipStream_t>(stream), active);
  if (e != hipSuccess) return hip_fail(e, "decoder step");
  state->t += 1;
  if (active) state->ragged = true;
  return ok();
}

rlt_status rlt_run_sequence(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                            const void* e, int64_t n, float* s_traj, void* stream) {
  if (rlt_status s = check_step_args(model, state, mem)) return s;
  if (!e) return fail(RLT_ERR_ARG, "e is NULL");
  if (n < 1) return fail(RLT_ERR_ARG, "n must be >= 1");
  if (!aligned16(e) || (s_traj && !aligned16(s_traj)))
    return fail(RLT_ERR_ARG, "e and s_traj must be 16-byte aligned");
  const int64_t t = state->t;
  if (mem->len < t)
    return fail(RLT_ERR_NOT_PROJECTED, "memory length %lld is behind position %lld",
                (long long)mem->len, (long long)t);
  if (t + n > mem->M.capacity)
    return fail(RLT_ERR_CAPACITY, "tokens up to %lld exceed capacity %lld", (long long)(t + n),
                (long long)mem->M.capacity);
  if (state->ragged && mem->len < t + n)
    return fail(RLT_ERR_NOT_PROJECTED, "sequences at different positions: the memory must hold "
                "entries up to %lld already", (long long)(t + n));
  const Dims& D = model->D;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int B = state->B;
  hipError_t err = hipSuccess;
  // project the tokens of [t, t+n) the memory does not hold yet
  if (mem->len < t + n) {
    const int64_t first = mem->len - t;  // index into e of the first missing token
    const int64_t cnt = n - first;
    const void* e_first = static_cast<const char*>(e) + (size_t)first * D.d * D.es;
    const double rows = (double)B * cnt, d = D.d, es = (double)D.es;
    Exec x(st);
    err = state->prof.arm(RLT_K_MEMPROJ, es * (rows * d + D.G * 2 * d * d + rows * D.G * 2 * d),
                          2 * rows * d * D.G * 2 * d, x);
    if (err == hipSuccess) err = launch_memproj(D, B, model->P, mem->M, e_first, n, mem->len, cnt, x);
    if (err != hipSuccess) return hip_fail(err, "memory projection");
    mem->len = t + n;
  }
  err = run_steps(model, state, mem, e, n * D.d, n, s_traj, n * D.d, st);
  if (err != hipSuccess) return hip_fail(err, "decoder step");
  state->t += n;
  return ok();
}

size_t rlt_parallel_ws_bytes(const rlt_config* cfg, int32_t batch, int64_t n) {
  if (check_config(cfg) != RLT_OK || !valid_batch(batch) || n < 1 || n > kMaxCapacity ||
      (int64_t)batch * n > INT32_MAX / 2)
    return 0;
  return par_layout(dims_of(*cfg), batch, n).total;
}

static rlt_status run_parallel(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                               const void* e, int64_t n, float* s_traj, void* ws,
                               size_t ws_bytes, void* stream, bool library_ws);

rlt_status rlt_run_parallel(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                            const void* e, int64_t n, float* s_traj, void* ws, size_t ws_bytes,
                            void* stream) {
  return run_parallel(model, state, mem, e, n, s_traj, ws, ws_bytes, stream, false);
}

rlt_status rlt_run_parallel_noalloc(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                                    const void* e, int64_t n, float* s_traj, void* stream) {
  return run_parallel(model, state, mem, e, n, s_traj, nullptr, kScratchBytes, stream, true);
}

size_t rlt_scratch_bytes(void) { return kScratchBytes; }

// library_ws: the workspace is this device's library-held scratch array (looked up here, after
// validation; ws is ignored), and a pass that does not fit it is refused with
// RLT_ERR_CAPACITY before anything is enqueued.
static rlt_status run_parallel(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                               const void* e, int64_t n, float* s_traj, void* ws,
                               size_t ws_bytes, void* stream, bool library_ws) {
  if (rlt_status s = check_step_args(model, state, mem)) return s;
  const Dims& D = model->D;
  if (D.alpha != 0.f)
    return fail(RLT_ERR_ARG, "the token-parallel pass needs alpha = 0 (the model has %g)",
                (double)D.alpha);
  if (D.dtype != RLT_BF16) return fail(RLT_ERR_DTYPE, "the token-parallel pass is bf16 only");
  if (!e || (!ws && !library_ws)) return fail(RLT_ERR_ARG, "e and ws must be non-NULL");
  if (n < 1) return fail(RLT_ERR_ARG, "n must be >= 1");
  if (!aligned16(e) || (s_traj && !aligned16(s_traj)) || (!library_ws && !aligned(ws)))
    return fail(RLT_ERR_ARG, "e and s_traj must be 16-byte aligned, ws 256-byte aligned");
  if (state->t != 0 || state->ragged)
    return fail(RLT_ERR_ARG, "the token-parallel pass starts from a reset state (position %lld)",
                (long long)state->t);
  const int B = state->B;
  if ((int64_t)B * n > INT32_MAX / 2) return fail(RLT_ERR_SHAPE, "B * n too large");
  const size_t need = par_layout(D, B, n).total;
  if (ws_bytes < need)
    return fail(RLT_ERR_CAPACITY, "%s has %zu bytes, needs %zu",
                library_ws ? "the library's scratch array" : "workspace", ws_bytes, need);
  if (n > mem->M.capacity)
    return fail(RLT_ERR_CAPACITY, "n = %lld exceeds memory capacity %lld", (long long)n,
                (long long)mem->M.capacity);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = hipSuccess;
  if (library_ws && (err = scratch_region(&ws)) != hipSuccess)
    return hip_fail(err, "looking up the scratch array");
  if (mem->len < n) {
    const int64_t first = mem->len, cnt = n - first;
    const void* e_first = static_cast<const char*>(e) + (size_t)first * D.d * D.es;
    const double rows = (double)B * cnt, d = D.d, es = (double)D.es;
    Exec x(st);
    err = state->prof.arm(RLT_K_MEMPROJ, es * (rows * d + D.G * 2 * d * d + rows * D.G * 2 * d),
                          2 * rows * d * D.G * 2 * d, x);
    if (err == hipSuccess) err = launch_memproj(D, B, model->P, mem->M, e_first, n, first, cnt, x);
    if (err != hipSuccess) return hip_fail(err, "memory projection");
    mem->len = n;
  }
  err = launch_parallel(D, B, model->P, state->S, mem->M, e, n, n, s_traj, n * D.d, ws, st,
                        &state->prof);
  if (err != hipSuccess) return hip_fail(err, "token-parallel pass");
  state->t = n;
  return ok();
}

// Starts a session of P: clears its records and, with a clock buffer attached, queues the
// clearing of every slot pair on stream st (ordered before the session's launches on st).
static hipError_t session_start(Profiler& P, hipStream_t st) {
  P.recs.clear();
  P.used = 0;
  P.clk_used = 0;
  P.clk_dropped = 0;
  return P.clear_clock(st);
}

// Ends a session of P: the durations of its timed launches, summed per kind into
// out[RLT_K_COUNT] (zeroed first); *dropped = launches that did not fit the clock buffer.
static hipError_t session_collect(Profiler& P, rlt_kernel_stats* out, int64_t* dropped) {
  for (int k = 0; k < RLT_K_COUNT; ++k) out[k] = rlt_kernel_stats{0, 0.0, 0.0, 0.0};
  hipError_t e = hipSuccess;
  std::vector<unsigned long long> clk;
  double ticks_per_ms = 0.0;
  if (P.clk_used > 0) {
    // self-stamped launches may have run on any of the streams
    int dev = 0, khz = 0;
    e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
    if (e == hipSuccess && khz <= 0) e = hipErrorInvalidValue;
    if (e == hipSuccess) {
      clk.resize(2 * (size_t)P.clk_used);
      e = hipMemcpy(clk.data(), P.clk_buf, clk.size() * 8, hipMemcpyDeviceToHost);
    }
    ticks_per_ms = khz;  // kHz = clock ticks per millisecond
  }
  for (const Profiler::Rec& r : P.recs) {
    if (e != hipSuccess) break;
    float ms = 0.f;
    if (r.ev < 0) {
      // earliest workgroup start to latest workgroup end
      unsigned long long a = ~0ull, b = 0ull;
      for (int64_t w = r.clk; w < r.clk + r.nclk; ++w) {
        a = std::min(a, clk[2 * w]);
        b = std::max(b, clk[2 * w + 1]);
      }
      if (a == ~0ull || b < a) {
        e = hipErrorInvalidValue;  // a workgroup of the launch left no stamps
        break;
      }
      ms = (float)((double)(b - a) / ticks_per_ms);
    } else {
      // launches of different row groups ran on different streams: wait for each one
      e = hipEventSynchronize(P.events[r.ev + 1]);
      if (e == hipSuccess) e = hipEventElapsedTime(&ms, P.events[r.ev], P.events[r.ev + 1]);
      if (e != hipSuccess) break;
    }
    rlt_kernel_stats& o = out[r.kind];
    o.launches += 1;
    o.total_ms += ms;
    o.bytes += r.bytes;
    o.flops += r.flops;
  }
  *dropped = P.clk_dropped;
  P.mask = 0;
  P.recs.clear();
  P.used = 0;
  P.clk_used = 0;
  P.clk_dropped = 0;
  return e;
}

static bool clock_buffer_ok(const void* buf, size_t bytes) {
  return !buf || (bytes >= 16 && reinterpret_cast<uintptr_t>(buf) % 16 == 0);
}

rlt_status rlt_profile_begin(rlt_state* state, uint32_t mask, int32_t token_stride) {
  if (!state) return fail(RLT_ERR_ARG, "state is NULL");
  if (mask >> RLT_K_COUNT) return fail(RLT_ERR_ARG, "mask has bits beyond RLT_K_COUNT");
  if (token_stride < 1) return fail(RLT_ERR_ARG, "token_stride must be >= 1, got %d", token_stride);
  Profiler& P = state->prof;
  P.mask = 0;
  // the state's launches may run on any stream: clear, then wait for the device
  hipError_t e = session_start(P, nullptr);
  if (e == hipSuccess && P.clk_buf) e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "clearing the clock buffer");
  P.stride = token_stride;
  P.mask = mask;
  return ok();
}

rlt_status rlt_profile_clock(rlt_state* state, void* buf, size_t bytes) {
  if (!state) return fail(RLT_ERR_ARG, "state is NULL");
  if (!clock_buffer_ok(buf, bytes))
    return fail(RLT_ERR_ARG, "the clock buffer must be 16-byte aligned and hold one slot pair");
  if (state->prof.mask) return fail(RLT_ERR_ARG, "a timing session is running");
  state->prof.clk_buf = static_cast<unsigned long long*>(buf);
  state->prof.clk_cap = buf ? (int64_t)(bytes / 16) : 0;
  return ok();
}

rlt_status rlt_profile_end(rlt_state* state, rlt_kernel_stats* out) {
  if (!state || !out) return fail(RLT_ERR_ARG, "state and out must be non-NULL");
  int64_t dropped = 0;
  const hipError_t e = session_collect(state->prof, out, &dropped);
  if (e != hipSuccess) return hip_fail(e, "reading kernel timers");
  if (dropped > 0)
    return fail(RLT_ERR_CAPACITY, "the clock buffer holds %lld workgroup slots; %lld more "
                "launches were not timed", (long long)state->prof.clk_cap, (long long)dropped);
  return ok();
}

rlt_status rlt_state_export(const rlt_state* state, float* s, void* k, void* v, int32_t* n_valid,
                            int64_t* position, uint64_t* version, void* stream) {
  if (!state) return fail(RLT_ERR_ARG, "state is NULL");
  const Dims& D = state->model->D;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = launch_export(D, state->B, state->S, s, k, v, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "state export");
  const int64_t keep = D.W - 1;
  if (n_valid) *n_valid = state->ragged ? -1 : (int32_t)(state->t < keep ? state->t : keep);
  if (position) *position = state->ragged ? -1 : state->t;
  if (version) *version = state->model->cfg.version;
  return ok();
}

rlt_status rlt_state_import(rlt_state* state, const float* s, const void* k, const void* v,
                            int64_t position, uint64_t version, void* stream) {
  if (!state || !s || !k || !v) return fail(RLT_ERR_ARG, "state, s, k and v must be non-NULL");
  if (position < 0) return fail(RLT_ERR_ARG, "position must be >= 0");
  if (version != state->model->cfg.version)
    return fail(RLT_ERR_VERSION, "snapshot version %llu != model version %llu",
                (unsigned long long)version, (unsigned long long)state->model->cfg.version);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // stream-ordered: every source is device memory the caller keeps until the stream has
  // passed this point
  hipError_t e = launch_import(state->model->D, state->B, state->S, position, s, k, v, st);
  if (e != hipSuccess) return hip_fail(e, "state import");
  state->t = position;
  state->ragged = false;
  return ok();
}

rlt_status rlt_state_import_ragged(rlt_state* state, const float* s, const void* k,
                                   const void* v, const int64_t* positions, uint64_t version,
                                   void* stream) {
  if (!state || !s || !k || !v || !positions)
    return fail(RLT_ERR_ARG, "state, s, k, v and positions must be non-NULL");
  if (version != state->model->cfg.version)
    return fail(RLT_ERR_VERSION, "snapshot version %llu != model version %llu",
                (unsigned long long)version, (unsigned long long)state->model->cfg.version);
  int64_t lo = positions[0], hi = positions[0];
  for (int b = 1; b < state->B; ++b) {
    lo = positions[b] < lo ? positions[b] : lo;
    hi = positions[b] > hi ? positions[b] : hi;
  }
  if (lo < 0 || hi > kMaxCapacity)
    return fail(RLT_ERR_ARG, "positions must lie in [0, %lld]", (long long)kMaxCapacity);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const Dims& D = state->model->D;
  hipError_t e = hipMemcpyAsync(state->S.s, s, sizeof(float) * (size_t)state->B * D.d,
                                hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(state->S.pos, positions, sizeof(int64_t) * (size_t)state->B,
                       hipMemcpyHostToDevice, st);
  if (e == hipSuccess) e = launch_import_caches(D, state->B, state->S, k, v, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return hip_fail(e, "state import");
  state->t = hi;
  state->ragged = lo != hi;
  return ok();
}

// ---- backward pass ---------------------------------------------------------------------------

size_t rlt_bptt_ws_bytes(const rlt_config* cfg, int32_t batch, int64_t n) {
  if (check_config(cfg) != RLT_OK || !valid_batch(batch) || n < 1 || n > kMaxCapacity ||
      (int64_t)batch * n > INT32_MAX / 2)
    return 0;
  return train_layout(dims_of(*cfg), batch, n).total;
}

rlt_status rlt_bptt(const rlt_model* model, const void* e, int32_t batch, int64_t n,
                    const float* ds, float* s_traj, const rlt_grads* grads, float* de, void* ws,
                    size_t ws_bytes, const rlt_truncation* trunc, const rlt_timing* timing,
                    rlt_kernel_stats* stats, void* stream) {
  if (!model) return fail(RLT_ERR_ARG, "model is NULL");
  if (!e || !ds || !grads || !ws) return fail(RLT_ERR_ARG, "e, ds, grads and ws must be non-NULL");
  float* const gp[] = {grads->s_star, grads->w_gate, grads->b_gate, grads->gamma, grads->wq,
                       grads->wk,     grads->wv,     grads->wo,     grads->wcq,   grads->wco,
                       grads->w1,     grads->w3,     grads->w2,     grads->wmk,   grads->wmv};
  for (float* p : gp)
    if (!p) return fail(RLT_ERR_ARG, "a gradient pointer is NULL");
  if (!valid_batch(batch)) return fail(RLT_ERR_SHAPE, "batch %d out of range", batch);
  if (n < 1 || n > kMaxCapacity)
    return fail(RLT_ERR_SHAPE, "n = %lld must be in [1, %lld]", (long long)n,
                (long long)kMaxCapacity);
  if ((int64_t)batch * n > INT32_MAX / 2) return fail(RLT_ERR_SHAPE, "batch * n too large");
  if (!aligned16(e) || !aligned(ws))
    return fail(RLT_ERR_ARG, "e must be 16-byte aligned, ws 256-byte aligned");
  if (trunc && trunc->segment < 1)
    return fail(RLT_ERR_ARG, "truncation segment must be >= 1, got %lld",
                (long long)trunc->segment);
  if (trunc && (trunc->detach & ~(uint32_t)(RLT_DETACH_STATE | RLT_DETACH_WINDOW)))
    return fail(RLT_ERR_ARG, "unknown detach bits 0x%x", trunc->detach);
  const bool timed = timing && timing->kernels;
  if (timed) {
    if (!stats) return fail(RLT_ERR_ARG, "stats must be non-NULL when timing kernels");
    if (timing->kernels >> RLT_K_COUNT)
      return fail(RLT_ERR_ARG, "timing has kernel bits beyond RLT_K_COUNT");
    if (timing->token_stride < 1)
      return fail(RLT_ERR_ARG, "token_stride must be >= 1, got %d", timing->token_stride);
    if (!clock_buffer_ok(timing->clk, timing->clk_bytes))
      return fail(RLT_ERR_ARG, "the clock buffer must be 16-byte aligned and hold one slot pair");
  }
  const Dims& D = model->D;
  const size_t need = train_layout(D, batch, n).total;
  if (ws_bytes < need)
    return fail(RLT_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  GradPtrs g{grads->s_star, grads->w_gate, grads->b_gate, grads->gamma, grads->wq, grads->wk,
             grads->wv,     grads->wo,     grads->wcq,    grads->wco,   grads->w1, grads->w3,
             grads->w2,     grads->wmk,    grads->wmv};
  hipStream_t st = static_cast<hipStream_t>(stream);
  Profiler prof;
  hipError_t err = hipSuccess;
  if (timed) {
    prof.clk_buf = static_cast<unsigned long long*>(timing->clk);
    prof.clk_cap = timing->clk ? (int64_t)(timing->clk_bytes / 16) : 0;
    err = session_start(prof, st);
    if (err != hipSuccess) return hip_fail(err, "clearing the clock buffer");
    prof.mask = timing->kernels;
    prof.stride = timing->token_stride;
  }
  rlt_model* mm = const_cast<rlt_model*>(model);
  if (batch >= 2 * kGroupRows && !mm->bwd_aux) {
    err = hipStreamCreateWithFlags(&mm->bwd_aux, hipStreamNonBlocking);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&mm->bwd_fork, hipEventDisableTiming);
    if (err == hipSuccess) err = hipEventCreateWithFlags(&mm->bwd_join, hipEventDisableTiming);
    if (err != hipSuccess) return hip_fail(err, "creating the backward pass's second stream");
  }
  if (!mm->bwd_grads) {
    // created as a whole or not at all, so a failed attempt is retried by the next call
    hipStream_t gs = nullptr;
    hipEvent_t gev[4] = {nullptr, nullptr, nullptr, nullptr};
    err = hipStreamCreateWithFlags(&gs, hipStreamNonBlocking);
    for (int i = 0; i < 4 && err == hipSuccess; ++i)
      err = hipEventCreateWithFlags(&gev[i], hipEventDisableTiming);
    if (err != hipSuccess) {
      if (gs) (void)hipStreamDestroy(gs);
      for (hipEvent_t ev : gev)
        if (ev) (void)hipEventDestroy(ev);
      return hip_fail(err, "creating the backward pass's gradient stream");
    }
    mm->bwd_grads = gs;
    for (int i = 0; i < 4; ++i) mm->bwd_gev[i] = gev[i];
  }
  err = launch_bptt(D, batch, n, model->P, e, ds, s_traj, g, de, ws, trunc ? trunc->segment : 0,
                    trunc ? trunc->detach : 0u, st,
                    batch >= 2 * kGroupRows ? mm->bwd_aux : nullptr, mm->bwd_fork, mm->bwd_join,
                    mm->bwd_grads, mm->bwd_gev, timed ? &prof : nullptr);
  int64_t dropped = 0;
  if (timed) {
    if (err == hipSuccess) err = hipStreamSynchronize(st);
    if (err == hipSuccess) err = session_collect(prof, stats, &dropped);
    prof.destroy();
  }
  if (err != hipSuccess) return hip_fail(err, "backward pass");
  if (dropped > 0)
    return fail(RLT_ERR_CAPACITY, "the clock buffer holds %lld workgroup slots; %lld more "
                "launches were not timed", (long long)prof.clk_cap, (long long)dropped);
  return ok();
}

// ---- encoder and readout around the decoder ----------------------------------------------------

size_t rlt_head_ws_bytes(const rlt_config* cfg, int32_t vocab) {
  if (check_config(cfg) != RLT_OK || !valid_vocab(vocab)) return 0;
  return head_layout(dims_of(*cfg), vocab).total;
}

rlt_status rlt_head_create(const rlt_model* model, int32_t vocab, const rlt_head_weights* w,
                           void* ws, size_t ws_bytes, void* stream, rlt_head** out) {
  if (!model || !w || !ws || !out)
    return fail(RLT_ERR_ARG, "model, weights, workspace and out must be non-NULL");
  if (!w->embed || !w->enc_gamma || !w->enc_gamma_out || !w->out_gamma || !w->w_out)
    return fail(RLT_ERR_ARG, "a head weight pointer is NULL");
  if (!valid_vocab(vocab))
    return fail(RLT_ERR_SHAPE, "vocab %d must be a multiple of 64 in [64, %d]", vocab, kMaxVocab);
  if (!aligned(ws)) return fail(RLT_ERR_ARG, "workspace must be 256-byte aligned");
  const Dims& D = model->D;
  const HeadLayout L = head_layout(D, vocab);
  if (ws_bytes < L.total)
    return fail(RLT_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  rlt_head* h = new (std::nothrow) rlt_head;
  if (!h) return fail(RLT_ERR_ARG, "out of host memory");
  h->model = model;
  h->Hd.vocab = vocab;
  h->Hd.embed = at<char>(ws, L.embed);
  h->Hd.w_out_t = at<char>(ws, L.w_out_t);
  h->Hd.enc_gamma = at<float>(ws, L.enc_gamma);
  h->Hd.enc_gamma_out = at<float>(ws, L.enc_gamma_out);
  h->Hd.out_gamma = at<float>(ws, L.out_gamma);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t d = D.d;
  hipError_t e = hipMemcpyAsync(h->Hd.embed, w->embed, (size_t)vocab * d * D.es,
                                hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess)
    e = launch_pack_transpose(D.dtype, w->w_out, (int)d, vocab, h->Hd.w_out_t, 0, vocab, vocab,
                              st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->Hd.enc_gamma, w->enc_gamma, (size_t)D.L * 2 * d * 4,
                       hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->Hd.enc_gamma_out, w->enc_gamma_out, d * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess)
    e = hipMemcpyAsync(h->Hd.out_gamma, w->out_gamma, d * 4, hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "packing the head weights");
  }
  *out = h;
  return ok();
}

void rlt_head_destroy(rlt_head* head) { delete head; }

size_t rlt_encode_ws_bytes(const rlt_config* cfg, int32_t batch, int64_t n) {
  if (check_config(cfg) != RLT_OK || cfg->dtype != RLT_BF16 || !valid_batch(batch) || n < 1 ||
      n > kMaxCapacity || (int64_t)batch * n > INT32_MAX / 2)
    return 0;
  return par_layout(dims_of(*cfg), batch, n).total;
}

rlt_status rlt_encode(const rlt_model* model, const rlt_head* head, const int32_t* tokens,
                      int32_t batch, int64_t n, void* e, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!model || !head || !tokens || !e || !ws)
    return fail(RLT_ERR_ARG, "model, head, tokens, e and ws must be non-NULL");
  if (head->model != model) return fail(RLT_ERR_ARG, "head belongs to another model");
  const Dims& D = model->D;
  if (D.dtype != RLT_BF16) return fail(RLT_ERR_DTYPE, "the encoder is bf16 only");
  if (!valid_batch(batch)) return fail(RLT_ERR_SHAPE, "batch %d out of range", batch);
  if (n < 1 || n > kMaxCapacity)
    return fail(RLT_ERR_SHAPE, "n = %lld must be in [1, %lld]", (long long)n,
                (long long)kMaxCapacity);
  if ((int64_t)batch * n > INT32_MAX / 2) return fail(RLT_ERR_SHAPE, "batch * n too large");
  if (reinterpret_cast<uintptr_t>(tokens) % 4 != 0 || !aligned16(e) || !aligned(ws))
    return fail(RLT_ERR_ARG, "tokens must be 4-byte, e 16-byte and ws 256-byte aligned");
  const size_t need = par_layout(D, batch, n).total;
  if (ws_bytes < need)
    return fail(RLT_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  hipError_t err = launch_encode(D, batch, n, model->P, head->Hd, tokens, e, ws,
                                 static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return hip_fail(err, "encoder");
  return ok();
}

size_t rlt_readout_ws_bytes(const rlt_config* cfg, int32_t vocab, int32_t batch) {
  if (check_config(cfg) != RLT_OK || !valid_vocab(vocab) || !valid_batch(batch)) return 0;
  return readout_layout(dims_of(*cfg), vocab, batch).total;
}

rlt_status rlt_readout(const rlt_model* model, const rlt_head* head, const float* s,
                       int32_t batch, const rlt_sampling* sp, const float* u, int32_t* tokens,
                       float* logp_behaviour, float* logp_model, float* logits, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!model || !head || !s || !sp || !u || !tokens || !logp_behaviour || !logp_model || !ws)
    return fail(RLT_ERR_ARG, "model, head, s, sampling, u, tokens, log-probability outputs and "
                "ws must be non-NULL");
  if (head->model != model) return fail(RLT_ERR_ARG, "head belongs to another model");
  if (!valid_batch(batch)) return fail(RLT_ERR_SHAPE, "batch %d out of range", batch);
  if (!std::isfinite(sp->temperature) || sp->temperature < 0.f)
    return fail(RLT_ERR_ARG, "temperature must be finite and >= 0");
  if (sp->top_k < 0) return fail(RLT_ERR_ARG, "top_k must be >= 0");
  if (!(sp->top_p > 0.f && sp->top_p <= 1.f)) return fail(RLT_ERR_ARG, "top_p must be in (0, 1]");
  if (!aligned16(s) || (logits && !aligned16(logits)) || !aligned(ws))
    return fail(RLT_ERR_ARG, "s and logits must be 16-byte aligned, ws 256-byte aligned");
  const Dims& D = model->D;
  const int V = head->Hd.vocab;
  const ReadoutLayout L = readout_layout(D, V, batch);
  if (ws_bytes < L.total)
    return fail(RLT_ERR_CAPACITY, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* lg = logits ? logits : at<float>(ws, L.logits);
  hipError_t err = launch_readout_logits(D, batch, head->Hd, s, at<char>(ws, L.hg),
                                         at<float>(ws, L.ssq), lg, st);
  if (err == hipSuccess)
    err = launch_sample(batch, V, lg, sp->temperature, sp->top_k, sp->top_p, u, tokens,
                        logp_behaviour, logp_model, st);
  if (err != hipSuccess) return hip_fail(err, "readout");
  return ok();
}

}  // extern "C"
