/*
 * rlt.h - C ABI of the MI355X (gfx950) Recurrent Looped Transformer decoder-step library.
 *
 * The library computes the per-token recurrent decoder transition H_{t-1} -> H_t of the
 * Recurrent Looped Transformer for B independent sequences at once, plus the token-parallel
 * projection of encoder outputs into the key/value memory that feeds it. Source of the
 * method: "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", section
 * "Architecture: encoder memory meets recurrent decoder" (state H_t = (s_t, C_t^D), gated
 * merge, per-block sliding-window self-attention + cross-attention to M_{<=t} + FFN, window W
 * counting the current token, learned start state s*), and its section "Three design
 * principles and their caveats" (memory projection runs token-parallel; transitions of
 * independent sequences share one batched kernel; no parallel scan over tokens).
 *
 * Formulas (the pages state none; these are the readings the library implements):
 *   u = alpha * s_{t-1};  g = sigmoid([e_t ; u] W_g + b_g);  h = g*e_t + (1-g)*u
 *   for each block l:  h += SWA(RMSNorm(h; gamma_l0))      window: this token + W-1 past
 *                      h += Cross(RMSNorm(h; gamma_l1))    memory entries 1..t of group g(l)
 *                      h += (SiLU(f W1) * (f W3)) W2,  f = RMSNorm(h; gamma_l2)
 *   s_t = h.   RMSNorm(x; gamma) = gamma * x / sqrt(mean(x^2) + eps).
 *   Attention is multi-head (H heads of hd = d/H), softmax scale 1/sqrt(hd), no biases,
 *   no positional encoding. Memory: K_j = e_j W_mK^(g), V_j = e_j W_mV^(g), g(l) = 0 when
 *   G = 1 and g(l) = l when G = L.
 *
 * Conventions for every call:
 *   - Device memory is allocated by the caller and borrowed by handles; the library never
 *     allocates device memory. Handles are host objects owned by the library and freed by
 *     the matching *_destroy (which never frees caller memory).
 *   - "dtype" arrays hold float32 (RLT_F32) or bfloat16 (RLT_BF16) elements, row-major.
 *     s, s*, b_g and the gains are always float32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Work is
 *     enqueued on it and the call returns without waiting, except where stated.
 *   - Every call validates all arguments before enqueuing anything; on error it returns a
 *     non-zero rlt_status, mutates nothing, and rlt_last_error() describes the problem.
 *     RLT_ERR_HIP reports a failed HIP call (launch or copy); state contents are then
 *     undefined.
 *   - Handles are not thread-safe. Distinct states on distinct streams may run concurrently.
 */
#ifndef RLT_H
#define RLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rlt_status {
  RLT_OK = 0,
  RLT_ERR_ARG = 1,           /* NULL handle/pointer, non-finite alpha, bad count      */
  RLT_ERR_SHAPE = 2,         /* sizes the library does not support or that disagree  */
  RLT_ERR_DTYPE = 3,         /* unknown dtype                                        */
  RLT_ERR_CAPACITY = 4,      /* caller buffer too small, or past the memory capacity */
  RLT_ERR_NOT_PROJECTED = 5, /* a step needs memory entries that are not projected   */
  RLT_ERR_HIP = 6,           /* a HIP runtime call failed                            */
  RLT_ERR_VERSION = 7        /* snapshot from a model with another version tag       */
} rlt_status;

typedef enum rlt_dtype { RLT_F32 = 0, RLT_BF16 = 1 } rlt_dtype;

/* Model shape. Supported: d = n_heads * head_dim, head_dim in {32, 64, 128}, d % 64 == 0,
 * ffn % 64 == 0, 1 <= window <= 1024, n_groups in {1, n_layers}, eps >= 0, alpha finite.
 * `version` is a caller-chosen tag of the weights, stored in snapshots and checked on import. */
typedef struct rlt_config {
  int32_t d;
  int32_t n_heads;
  int32_t head_dim;
  int32_t n_layers;   /* L_D */
  int32_t ffn;        /* F   */
  int32_t window;     /* W, counts the current token */
  int32_t n_groups;   /* G   */
  int32_t dtype;      /* rlt_dtype */
  float alpha;        /* feedback scale */
  float eps;          /* RMSNorm epsilon */
  uint64_t version;
} rlt_config;

/* Device pointers to the weights, in the math convention y = x W (row-major [in][out]).
 * Matrices are `dtype`; the rest float32. Only read during rlt_model_create. */
typedef struct rlt_weights {
  const float* s_star; /* [d]        learned start state s*                               */
  const void* w_gate;  /* [2d][d]    rows 0..d-1 multiply e_t, rows d..2d-1 multiply u     */
  const float* b_gate; /* [d]                                                              */
  const float* gamma;  /* [L][3][d]  gains before self-attention, cross-attention, FFN    */
  const void* wq;      /* [L][d][d]  */
  const void* wk;      /* [L][d][d]  */
  const void* wv;      /* [L][d][d]  */
  const void* wo;      /* [L][d][d]  */
  const void* wcq;     /* [L][d][d]  cross-attention query projection                     */
  const void* wco;     /* [L][d][d]  cross-attention output projection                    */
  const void* w1;      /* [L][d][F]  FFN gate branch (through SiLU)                       */
  const void* w3;      /* [L][d][F]  FFN linear branch                                    */
  const void* w2;      /* [L][F][d]  FFN down projection                                  */
  const void* wmk;     /* [G][d][d]  memory key projection                                */
  const void* wmv;     /* [G][d][d]  memory value projection                              */
} rlt_weights;

typedef struct rlt_model rlt_model;
typedef struct rlt_state rlt_state;
typedef struct rlt_memory rlt_memory;

/* Thread-local description of the last error (empty string if none). Never NULL. */
const char* rlt_last_error(void);

/* Validates a configuration without touching the GPU. */
rlt_status rlt_config_check(const rlt_config* cfg);

/* --- model ------------------------------------------------------------------------------ */

/* Bytes of device workspace rlt_model_create needs for the packed weights (0 if the
 * configuration is invalid). */
size_t rlt_model_ws_bytes(const rlt_config* cfg);

/* Packs the weights into `ws` (device, >= rlt_model_ws_bytes, 256-byte aligned) in the
 * layouts the kernels read, on `stream`, and waits for that stream: on return the caller may
 * free the source weights. `ws` must stay alive until rlt_model_destroy. */
rlt_status rlt_model_create(const rlt_config* cfg, const rlt_weights* w, void* ws,
                            size_t ws_bytes, void* stream, rlt_model** out);
void rlt_model_destroy(rlt_model* model);

/* --- decoder state H_t = (s_t, C_t^D) ------------------------------------------------- */

/* Bytes of device memory for the state of B sequences: s [B][d] float32, the per-layer
 * self-attention caches, and the working buffers of one decoder step. The state is
 * H_t = (s_t, C_t^D) of "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets",
 * "Architecture: encoder memory meets recurrent decoder". 0 if the configuration or batch
 * (1 .. 2^20) is invalid. */
size_t rlt_state_bytes(const rlt_config* cfg, int32_t batch);

/* Binds `buf` (device, >= rlt_state_bytes, 256-byte aligned) as the state of `batch`
 * sequences and resets it on `stream` (see rlt_state_reset). RLT_ERR_CAPACITY if `buf` is too
 * small, RLT_ERR_ARG if misaligned or NULL. The buffer stays owned by the caller and must
 * outlive the handle. */
rlt_status rlt_state_create(const rlt_model* model, int32_t batch, void* buf, size_t bytes,
                            void* stream, rlt_state** out);

/* s_0 = s* for every sequence, empty caches, position t = 0 (before the first token): the
 * one-time initialisation by the learned start state and an empty cache of the architecture
 * section; nothing resets the state afterwards (no reset at the prompt-response boundary). */
rlt_status rlt_state_reset(rlt_state* state, void* stream);

/* Number of tokens every sequence of the state has processed (t), or -1 once a step with an
 * active mask has run (rlt_decoder_step_ragged): then the sequences may be at different
 * positions, which rlt_state_positions reads. */
int64_t rlt_state_position(const rlt_state* state);

/* Waits for `stream` and copies the B per-sequence positions (int64, host array `out`). */
rlt_status rlt_state_positions(const rlt_state* state, int64_t* out, void* stream);
void rlt_state_destroy(rlt_state* state);

/* --- encoder memory M ----------------------------------------------------------------- */

/* Bytes for the key and value memory M of B sequences up to `capacity` tokens: K and V, each
 * [G][B][H][capacity][hd] dtype, shared by all blocks (G = 1) or one per block (G = L_D), as
 * the architecture section allows. 1 <= capacity <= 2^20; 0 if invalid. */
size_t rlt_memory_bytes(const rlt_config* cfg, int32_t batch, int64_t capacity);

/* Binds `buf` (device, >= rlt_memory_bytes, 256-byte aligned) as empty memory (length 0).
 * RLT_ERR_CAPACITY if `buf` or `capacity` is out of range, RLT_ERR_ARG if misaligned. The
 * buffer stays owned by the caller and must outlive the handle. */
rlt_status rlt_memory_create(const rlt_model* model, int32_t batch, int64_t capacity, void* buf,
                             size_t bytes, rlt_memory** out);

/* Number of tokens whose keys/values have been projected (entries 0..length-1). */
int64_t rlt_memory_length(const rlt_memory* mem);

/* Marks the memory empty (length 0) so it can be projected again from token 0; host-only. */
rlt_status rlt_memory_reset(rlt_memory* mem);
void rlt_memory_destroy(rlt_memory* mem);

/* Token-parallel memory projection of tokens t0 .. t0+n-1 (0-based) from encoder outputs
 * e [B][n][d] dtype (device): K_j = e_j W_mK^(g), V_j = e_j W_mV^(g) for every group g, the
 * prefix-restricted key/value memory M_{<=t} the decoder reads ("RLT Runs 96 Blocks Per Token
 * With Recurrent State, No Resets", "Architecture: encoder memory meets recurrent decoder";
 * run token-parallel per "Three design principles and their caveats"). Requires
 * 0 <= t0 <= length (no holes, else RLT_ERR_NOT_PROJECTED), n >= 1 (RLT_ERR_ARG) and
 * t0 + n <= capacity (RLT_ERR_CAPACITY); afterwards length = max(length, t0 + n). e must
 * stay valid until `stream` has passed the call. */
rlt_status rlt_memproj(const rlt_model* model, rlt_memory* mem, const void* e, int64_t t0,
                       int64_t n, void* stream);

/* --- the recurrent transition --------------------------------------------------------- */

/* One decoder step for every sequence, the transition H_t -> H_{t+1} ("RLT Runs 96 Blocks Per
 * Token With Recurrent State, No Resets", "Architecture: encoder memory meets recurrent
 * decoder": gated merge of e with the previous output, then per block window self-attention,
 * cross-attention to M_{<=t+1} and FFN; the window keeps W-1 past entries): consumes
 * e_t [B][d] dtype (device) for token t+1 (1-based), where t = rlt_state_position; needs
 * memory length >= t+1 (else RLT_ERR_NOT_PROJECTED). Writes s_{t+1} to s_out [B][d] float32
 * (device) unless NULL, and advances the position. The state and the memory must belong to
 * `model` (RLT_ERR_ARG) and have the same batch (RLT_ERR_SHAPE); e_t and s_out 16-byte
 * aligned (RLT_ERR_ARG). */
rlt_status rlt_decoder_step(const rlt_model* model, rlt_state* state, const rlt_memory* mem,
                            const void* e_t, float* s_out, void* stream);

/* Ragged "ready updates": one decoder step for the sequences whose byte in `active` (device,
 * [B] uint8, non-zero = active; NULL = all) is set, each at its own position: sequence b
 * consumes e_t row b as its token pos_b + 1 and advances; the others keep s, their window and
 * their position, and their s_out row receives their unchanged s. Sequences that are ready
 * share one batched launch per kernel ("RLT Runs 96 Blocks Per Token With Recurrent State, No
 * Resets", "Three design principles and their caveats": ready updates of independent
 * sequences share one batched kernel). The memory must hold entries up to the largest
 * position any sequence can have (the number of steps run since reset), else
 * RLT_ERR_NOT_PROJECTED. After such a step rlt_state_position returns -1. */
rlt_status rlt_decoder_step_ragged(const rlt_model* model, rlt_state* state,
                                   const rlt_memory* mem, const void* e_t, const uint8_t* active,
                                   float* s_out, void* stream);

/* n consecutive steps over e [B][n][d] dtype (device), the encoder outputs of tokens
 * t+1 .. t+n: the sequential chain of transitions, which no parallel scan replaces ("RLT Runs
 * 96 Blocks Per Token With Recurrent State, No Resets", "Three design principles and their
 * caveats"). First projects every one of those tokens that the memory does not hold yet
 * (same as rlt_memproj on the missing range; requires t <= length, else
 * RLT_ERR_NOT_PROJECTED, and t + n <= capacity, else RLT_ERR_CAPACITY), then runs n steps.
 * s_traj [B][n][d] float32 (device) receives every s unless NULL. The result equals
 * rlt_memproj followed by n calls of rlt_decoder_step, bitwise; so does any split of the n
 * tokens into consecutive calls (the split invariance of the same section). */
rlt_status rlt_run_sequence(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                            const void* e, int64_t n, float* s_traj, void* stream);

/* --- token-parallel pass for alpha = 0 -------------------------------------------------- */
/* With feedback scale alpha = 0 the gated merge does not read s_{t-1} (h_t = g(e_t) * e_t),
 * so the decoder blocks couple tokens only through causal attention - the window of W-1
 * previous tokens of each layer and the memory prefix 1..t - and all n tokens can run layer by
 * layer at once, as the feedback-off control of the independent evaluation did ("RLT Runs 96
 * Blocks Per Token With Recurrent State, No Resets", "Three design principles and their
 * caveats": a parallel decoder pass is not equivalent to the recurrence unless the feedback is
 * off; "16 per-token recurrence, no quality gain": the feedback-off variant trained at 66.0K
 * tokens/s against 8.4K for the recurrence). */

/* Device workspace bytes of rlt_run_parallel for B sequences and n tokens (0 if invalid). */
size_t rlt_parallel_ws_bytes(const rlt_config* cfg, int32_t batch, int64_t n);

/* Same contract as rlt_run_sequence from a reset state (position 0): projects the memory of
 * tokens 1..n it does not hold yet, writes every s_t to s_traj [B][n][d] float32 unless NULL,
 * and leaves the state as n decoder steps would (s_n, the last W-1 keys/values per layer,
 * position n), so decoding can continue with rlt_decoder_step. Results equal the recurrent
 * path up to rounding (the projections run as large MFMA GEMMs on RMS-normalised bf16 rows and
 * the attentions as causal flash attention with bf16 queries). Requires alpha == 0
 * (RLT_ERR_ARG), dtype bf16 (RLT_ERR_DTYPE), position 0 (RLT_ERR_ARG), n <= memory capacity
 * (RLT_ERR_CAPACITY) and `ws` (device, 256-byte aligned, >= rlt_parallel_ws_bytes; its contents
 * are scratch, owned by the caller) (RLT_ERR_CAPACITY). */
rlt_status rlt_run_parallel(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                            const void* e, int64_t n, float* s_traj, void* ws, size_t ws_bytes,
                            void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, serving loops
 * that must not call the allocator, harnesses that forbid it): rlt_run_parallel with the
 * workspace taken from a scratch array the library holds on each GPU for the life of the
 * process (rlt_scratch_bytes() bytes, 64 MiB). The call allocates nothing. A pass whose
 * workspace (rlt_parallel_ws_bytes) exceeds the array fails with RLT_ERR_CAPACITY before
 * anything is enqueued; every other argument and error is as for rlt_run_parallel. All calls
 * on one GPU share that GPU's array and it keeps the last call's contents: calls that overlap
 * on one GPU (several host threads, or several streams whose work runs concurrently) race on
 * it and must be ordered by the caller. */
rlt_status rlt_run_parallel_noalloc(const rlt_model* model, rlt_state* state, rlt_memory* mem,
                                    const void* e, int64_t n, float* s_traj, void* stream);

/* Bytes of the library-held scratch array of each GPU. */
size_t rlt_scratch_bytes(void);

/* --- backward pass ("RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", section
 * "Training and serving implications": training backpropagates through the whole sequence,
 * and the gradient between consecutive states also runs through the decoder's self-attention
 * keys/values; "16 per-token recurrence, no quality gain": a backward pass that walks the
 * tokens in reverse) ------------------------------------------------------------------------ */

/* Truncated backpropagation for rlt_bptt ("RLT Runs 96 Blocks Per Token With Recurrent State,
 * No Resets", "Training and serving implications": detaching s_t alone leaves gradient paths
 * open through the decoder's keys/values, so a truncated scheme must name every detached
 * tensor). The tokens form segments of `segment` tokens; at every segment start the tensors
 * named in `detach` carry no gradient back into the previous segment. The memory is never
 * detached. */
enum {
  RLT_DETACH_STATE = 1,  /* the carried output s (the gated merge's feedback input)     */
  RLT_DETACH_WINDOW = 2  /* self-attention keys/values of earlier tokens in the window */
};
typedef struct rlt_truncation {
  int64_t segment;  /* >= 1 */
  uint32_t detach;  /* RLT_DETACH_* bits */
} rlt_truncation;

/* Optional kernel timing of rlt_bptt (see rlt_kernel and rlt_kernel_stats below). */
typedef struct rlt_timing {
  uint32_t kernels;     /* bit (1 << rlt_kernel) per kernel to time */
  int32_t token_stride; /* >= 1 */
  void* clk;            /* NULL (events), or a device buffer, 16-byte aligned, in which the
                         * backward attention kernels (RLT_K_BWD_SELF, RLT_K_BWD_CROSS) time
                         * themselves as with rlt_profile_clock: 16 * H bytes per sequence of
                         * each timed launch; too small: RLT_ERR_CAPACITY after the pass */
  size_t clk_bytes;
} rlt_timing;
struct rlt_kernel_stats;

/* Gradient outputs of rlt_bptt: device float32 buffers (caller-owned), one per parameter, each
 * laid out like the matching rlt_weights field. */
typedef struct rlt_grads {
  float* s_star; /* [d]        */
  float* w_gate; /* [2d][d]    */
  float* b_gate; /* [d]        */
  float* gamma;  /* [L][3][d]  */
  float* wq;     /* [L][d][d]  */
  float* wk;
  float* wv;
  float* wo;
  float* wcq;
  float* wco;
  float* w1;     /* [L][d][F]  */
  float* w3;     /* [L][d][F]  */
  float* w2;     /* [L][F][d]  */
  float* wmk;    /* [G][d][d]  */
  float* wmv;    /* [G][d][d]  */
} rlt_grads;

/* Device workspace bytes of rlt_bptt for B sequences of n tokens (0 if invalid). The workspace
 * holds what the reverse walk needs from the forward pass (about
 * n * B * L * d * (20 + 5 * element size) bytes), the memory, and backward copies of the
 * weights. */
size_t rlt_bptt_ws_bytes(const rlt_config* cfg, int32_t batch, int64_t n);

/* Backpropagation through time over whole sequences. Runs the decoder from the start state
 * (s*, empty caches) over e [B][n][d] (dtype, device, 16-byte aligned), projecting the memory
 * of all n tokens itself, then walks the tokens in reverse for the upstream gradients
 * ds [B][n][d] float32 (device): ds[b][t] = dLoss/ds_t of sequence b. Every buffer of `grads`
 * is overwritten with dLoss/dparameter (float32, summed over the batch); de [B][n][d] float32
 * (device, or NULL to skip) receives dLoss/de through the gated merge and the memory
 * projection; s_traj [B][n][d] float32 (device, or NULL) receives the forward trajectory.
 * Gradients through the self-attention keys/values of later tokens are included; `trunc`
 * (NULL: full backpropagation) truncates them and the state's at segment starts as it names
 * (RLT_ERR_ARG for a segment < 1 or unknown bits). Independent
 * of any rlt_state or rlt_memory. `ws`: device, 256-byte aligned, >= rlt_bptt_ws_bytes bytes,
 * scratch owned by the caller (RLT_ERR_CAPACITY if smaller). Asynchronous on `stream`, unless
 * `timing` is non-NULL with kernels != 0: then the launches of those kernels (rlt_kernel bits)
 * are timed with events, in the forward and reverse steps of tokens t with
 * t % token_stride == 0 and in every launch outside the token loops, and the call waits for the
 * stream and writes RLT_K_COUNT entries to `stats` (host array, required then).
 * Batches of 256 or more sequences run as two row groups, the second on a stream the model
 * creates on first use, and the weight gradients of each chunk of tokens run on a third such
 * stream while the walk goes on; both are kept until rlt_model_destroy. Calls of rlt_bptt on
 * one model must not overlap (they share those streams and their events); other calls on the
 * model may. */
rlt_status rlt_bptt(const rlt_model* model, const void* e, int32_t batch, int64_t n,
                    const float* ds, float* s_traj, const rlt_grads* grads, float* de, void* ws,
                    size_t ws_bytes, const rlt_truncation* trunc, const struct rlt_timing* timing,
                    struct rlt_kernel_stats* stats, void* stream);

/* --- encoder and readout around the decoder ------------------------------------------------
 * "RLT Runs 96 Blocks Per Token With Recurrent State, No Resets", "Architecture: encoder memory
 * meets recurrent decoder": a causal encoder processes the tokens in parallel and produces the
 * e_t the memory is projected from; in the tied configuration its blocks share the decoder
 * blocks' attention and FFN weights; the next-token distribution is read from s_t. Same page,
 * "Three design principles and their caveats" (model-RL co-design): the sampler records each
 * action's behaviour log-probability under the distribution it sampled from, temperature and
 * truncation included. Readings (the pages give no formulas):
 *   x_0 = E[token];  encoder block l: x += Attn_causal(RMSNorm(x; g_l0)) W_o[l] (positions
 *   1..t, W_q/W_k/W_v/W_o of decoder block l), x += FFN_l(RMSNorm(x; g_l1)) (decoder block l's
 *   W_1, W_3, W_2);  e = RMSNorm(x; g_out).  logits = RMSNorm(s; gamma_out) W_out.
 *   Sampling: q = softmax(logits / temperature); order tokens by descending logit, ties by
 *   ascending id; top-k keeps the first k (0: all), top-p the shortest prefix of those whose
 *   mass reaches top_p times their mass (1: all); pi = q on the kept tokens, renormalised; the
 *   action is the first kept token, in ascending id, at which the running sum of pi exceeds u.
 *   temperature 0 = greedy (first maximal logit, probability 1). */

/* Head weights (device pointers, only read during rlt_head_create). */
typedef struct rlt_head_weights {
  const void* embed;          /* [V][d] dtype      token embedding E                          */
  const float* enc_gamma;     /* [L][2][d]         encoder gains before attention and FFN     */
  const float* enc_gamma_out; /* [d]               gain of the norm that gives e               */
  const float* out_gamma;     /* [d]               gain of the readout's norm of s             */
  const void* w_out;          /* [d][V] dtype      readout matrix                              */
} rlt_head_weights;
typedef struct rlt_head rlt_head;

/* Bytes of device workspace rlt_head_create needs for vocabulary size V (0 if invalid: V must
 * be a multiple of 64 in [64, 2^22]). */
size_t rlt_head_ws_bytes(const rlt_config* cfg, int32_t vocab);

/* Copies and packs the head weights into `ws` (device, 256-byte aligned, >= rlt_head_ws_bytes)
 * on `stream` and waits for it, so the sources may be freed on return. The encoder uses the
 * model's packed attention and FFN matrices, so the head is bound to `model`. */
rlt_status rlt_head_create(const rlt_model* model, int32_t vocab, const rlt_head_weights* w,
                           void* ws, size_t ws_bytes, void* stream, rlt_head** out);
void rlt_head_destroy(rlt_head* head);

/* Device workspace bytes of rlt_encode for B sequences of n tokens (0 if invalid, or for fp32
 * models: the encoder is bf16 only). */
size_t rlt_encode_ws_bytes(const rlt_config* cfg, int32_t batch, int64_t n);

/* Token-parallel causal encoder: token ids [B][n] int32 (device, 4-byte aligned; ids outside
 * [0, V) embed as zero vectors) -> e [B][n][d] dtype (device, 16-byte aligned), ready for
 * rlt_memproj / rlt_run_sequence. ws: device, 256-byte aligned, >= rlt_encode_ws_bytes
 * (RLT_ERR_CAPACITY), scratch owned by the caller. bf16 models only (RLT_ERR_DTYPE).
 * Asynchronous on `stream`. */
rlt_status rlt_encode(const rlt_model* model, const rlt_head* head, const int32_t* tokens,
                      int32_t batch, int64_t n, void* e, void* ws, size_t ws_bytes,
                      void* stream);

/* Sampling parameters: temperature >= 0 (0 = greedy), top_k >= 0 (0 = off), top_p in (0, 1]
 * (1 = off). */
typedef struct rlt_sampling {
  float temperature;
  int32_t top_k;
  float top_p;
} rlt_sampling;

/* Device workspace bytes of rlt_readout for B rows (0 if invalid). */
size_t rlt_readout_ws_bytes(const rlt_config* cfg, int32_t vocab, int32_t batch);

/* Readout and sampling of B rows s [B][d] float32 (device; e.g. s_out of a decoder step): the
 * logits (float32 [B][V] into `logits` when non-NULL, else into ws), then per row b, with the
 * uniform u[b] in [0, 1) (device float32 [B], drawn by the caller), the action tokens[b]
 * (device int32), its behaviour log-probability log pi(action) under the tempered, truncated
 * distribution logp_behaviour[b] (0 when greedy) and its model log-probability
 * log softmax(logits)(action) at temperature 1 without truncation logp_model[b] (device float32
 * [B] each). Every decision (truncation sets, inverse CDF) is taken on exact integers: fixed-point
 * probabilities (2^-40 units) and an order-preserving key of each logit. RLT_ERR_ARG for
 * parameters out of range or NULL outputs; ws: device, 256-byte aligned,
 * >= rlt_readout_ws_bytes (RLT_ERR_CAPACITY). Asynchronous on `stream`. */
rlt_status rlt_readout(const rlt_model* model, const rlt_head* head, const float* s,
                       int32_t batch, const rlt_sampling* sampling, const float* u,
                       int32_t* tokens, float* logp_behaviour, float* logp_model, float* logits,
                       void* ws, size_t ws_bytes, void* stream);

/* --- snapshots ("exact prefix snapshot" of the serving section of the same page) ------ */

/* Copies the state to caller buffers in canonical order and waits for the stream:
 *   s [B][d] float32 (device); k, v [L][B][W-1][d] dtype (device), per layer and sequence
 *   the retained entries oldest first (sequence b keeps min(t_b, W-1) of them, t_b its own
 *   position), zero padded; *n_valid = min(t, W-1) and *position = t when every sequence is
 *   at the same position t, else both -1 (see rlt_state_positions); *version = the model's
 *   version tag. Any output pointer may be NULL to skip it. */
rlt_status rlt_state_export(const rlt_state* state, float* s, void* k, void* v,
                            int32_t* n_valid, int64_t* position, uint64_t* version,
                            void* stream);

/* Loads a snapshot in the layout rlt_state_export writes (k/v rows beyond min(t, W-1) are
 * ignored). Fails with RLT_ERR_VERSION, changing nothing, if `version` differs from the
 * model's tag. Stream-ordered, like the steps: s, k and v (device) must stay valid until
 * `stream` has passed the call. */
rlt_status rlt_state_import(rlt_state* state, const float* s, const void* k, const void* v,
                            int64_t position, uint64_t version, void* stream);

/* The same for a snapshot whose sequences are at different positions: `positions` is a host
 * array of B positions (as rlt_state_positions reads them, each in [0, 2^20]); sequence b's
 * canonical k/v rows hold its min(positions[b], W-1) retained entries. Waits for the stream,
 * so that the host array may be reused on return (the one import that synchronises).
 * Together with rlt_state_export and rlt_state_positions this splits and resumes a batch of
 * ragged sequences ("exact prefix snapshot"). */
rlt_status rlt_state_import_ragged(rlt_state* state, const float* s, const void* k,
                                   const void* v, const int64_t* positions, uint64_t version,
                                   void* stream);

/* --- kernel timing --------------------------------------------------------------------- */

/* Kernels of one decoder step (and the memory projection run by rlt_run_sequence). */
typedef enum rlt_kernel {
  RLT_K_GATE = 0,        /* gated merge: [e_t ; alpha s] W_g, sigmoid, merge            */
  RLT_K_QKV = 1,         /* RMSNorm + q/k/v projection, k/v into the ring cache          */
  RLT_K_SELF_ATTN = 2,   /* sliding-window attention over the ring cache                 */
  RLT_K_SELF_OUT = 3,    /* self-attention output projection + residual                  */
  RLT_K_CROSS_Q = 4,     /* RMSNorm + cross-attention query projection                   */
  RLT_K_CROSS_ATTN = 5,  /* attention over memory entries 1..t                            */
  RLT_K_CROSS_OUT = 6,   /* cross-attention output projection + residual                 */
  RLT_K_FFN_UP = 7,      /* RMSNorm + W1/W3 projection + SiLU product                     */
  RLT_K_FFN_DOWN = 8,    /* W2 projection + residual                                      */
  RLT_K_MEMPROJ = 9,     /* memory projection                                             */
  RLT_K_PAR_GEMM = 10,   /* token-parallel pass: every projection (all rows at once)      */
  RLT_K_PAR_SELF = 11,   /* token-parallel pass: window attention                          */
  RLT_K_PAR_CROSS = 12,  /* token-parallel pass: memory-prefix attention                   */
  RLT_K_PAR_OTHER = 13,  /* token-parallel pass: RMSNorm rows, ring hand-off, final s      */
  RLT_K_BWD_PROJ = 14,   /* backward pass: per-token projections against transposed weights */
  RLT_K_BWD_SELF = 15,   /* backward pass: window attention backward, key/value gradients    */
  RLT_K_BWD_CROSS = 16,  /* backward pass: memory-prefix attention backward (query gradient) */
  RLT_K_BWD_MEM = 17,    /* backward pass: memory key/value gradients after the walk         */
  RLT_K_BWD_WGRAD = 18,  /* backward pass: weight-gradient GEMMs over chunks of rows         */
  RLT_K_BWD_OTHER = 19,  /* backward pass: RMSNorm rows and backward, saves, sums, repacking */
  RLT_K_COUNT = 20
} rlt_kernel;

typedef struct rlt_kernel_stats {
  int64_t launches;  /* launches timed                                                   */
  double total_ms;   /* sum over launches of the kernel's duration (HIP events, or the     *
                      * kernel's own clock stamps, see rlt_profile_clock)                 */
  double bytes;      /* algorithmic bytes: each operand read once, each result written once */
  double flops;      /* algorithmic floating-point operations                            */
} rlt_kernel_stats;

/* Starts timing, for this state, launches of the kernels whose bit (1 << rlt_kernel) is set in
 * `mask`: each timed launch records a pair of HIP events at the start and at the end of its
 * kernel (hipExtLaunchKernel), on the stream it runs on, except the attention kernels while a
 * clock buffer is attached (rlt_profile_clock), which time themselves. Decoder
 * launches are timed in the steps of tokens t (0-based position before the step) with
 * t % token_stride == 0 (token_stride >= 1; 1 = every step), memory projections always.
 * Events are pooled by the state and kept until rlt_state_destroy. */
rlt_status rlt_profile_begin(rlt_state* state, uint32_t mask, int32_t token_stride);

/* Stops timing, waits for the recorded events (and, when clock slots were used, for the
 * device) and writes RLT_K_COUNT entries to `out` (host array, indexed by rlt_kernel).
 * RLT_ERR_CAPACITY (after writing `out`) when the clock buffer was too small for the launches
 * to be timed. */
rlt_status rlt_profile_end(rlt_state* state, rlt_kernel_stats* out);

/* Attaches a caller-owned device buffer (16-byte aligned; NULL detaches) in which later timing
 * sessions of this state time the two attention kernels (RLT_K_SELF_ATTN, RLT_K_CROSS_ATTN)
 * by their own clock instead of by events: every workgroup writes the GPU's constant-rate wall
 * clock to a slot pair of its own when it starts and when all its waves are done, and
 * rlt_profile_end takes each launch's earliest start and latest end. Nothing is queued around
 * the launch that could change how concurrent streams overlap, and no two workgroups write the
 * same address. The kernels run one workgroup per (sequence, head): a timed launch takes
 * 16 * H bytes per sequence of its batch; a memory attention whose batch has fewer than 128
 * sequence-head pairs splits each prefix into up to 16 slices of at least 256 entries, one
 * workgroup each (16 * H * slices bytes per sequence), and merges them in a second, untimed
 * launch. rlt_profile_begin clears the slots (it waits for the
 * device); launches that no longer fit are not timed and make rlt_profile_end return
 * RLT_ERR_CAPACITY. Not while a session runs (RLT_ERR_ARG). The buffer must stay allocated
 * while attached. */
rlt_status rlt_profile_clock(rlt_state* state, void* buf, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* RLT_H */
