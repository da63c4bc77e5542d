/*
 * moe.h -- C ABI of libmoe.so: the forward pass of one mixture-of-experts
 * feed-forward layer on an AMD Instinct MI355X (gfx950).
 *
 * The layer, as the pages define it: a router scores every expert per token,
 * keeps the k best and weights them (softmax over all experts then top-k,
 * optionally renormalized, or top-k then softmax over the chosen k); tokens
 * are grouped by expert, optionally capped at a capacity C; each expert is a
 * SwiGLU MLP; an optional shared expert runs on every token; the outputs are
 * summed back in token order, weighted by the gate weights; balance
 * statistics f_i, P_i, L_aux and the demand max/mean load are reported.
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must point to device memory (HBM) of
 *     the current device; the caller owns and allocates every buffer.  The
 *     library allocates nothing; its only state is a per-device cache of the
 *     compute-unit count (read once with hipDeviceGetAttribute).
 *   - Tensors are dense, row-major.  Rows of x and of the weights must start on
 *     16-byte boundaries (true when the base is 16-byte aligned and d, F are
 *     multiples of 8).
 *   - dtype (MOE_F32 or MOE_BF16) is the storage type of x, every weight
 *     matrix, the hidden activations a, y_perm, shared_y and y.  Router scores
 *     (logits), gate weights and statistics are float32.  Accumulation is
 *     float32.  bfloat16 results are rounded to nearest, ties to even.
 *   - Weights are held (out_features, in_features), as torch.nn.Linear holds
 *     them: W_r[E][d]; per expert gate[F][d], up[F][d], down[d][F].  The
 *     Residual Stream's MoE listing ("An MoE tiny GPT") stacks the expert
 *     matrices the other way round, gate and up as (E, d, F) and down as
 *     (E, F, d), and multiplies h @ gate[e]: a caller holding tensors in that
 *     order transposes each expert's matrices once (torch:
 *     gate.transpose(1, 2).contiguous(), the same for up and down) before
 *     passing them here.  K-contiguous rows let both MFMA operands load as
 *     16-byte vectors along the reduction.
 *   - Calls are asynchronous on `stream` (0 = the null stream) and never
 *     synchronize the host.  Arguments are checked on the host before
 *     anything is enqueued; on a bad argument a negative moe_status is
 *     returned and nothing runs.  A failed launch returns MOE_ERR_HIP.
 *     moe_last_error() describes the last failure on the calling thread.
 *   - T = 0 (no tokens) is a valid call that enqueues nothing.
 *   - Kernels never trap.  Values read from device memory that the host cannot
 *     check (expert ids, offsets) are clamped or skipped as stated per call.
 *
 * Limits: 1 <= k <= E <= 256.  d and F multiples of 8 (MOE_F32) or of 128
 * (MOE_BF16); other sizes return MOE_ERR_UNSUPPORTED.  The grouped GEMMs
 * address each operand (x or a, one expert's weights) with 32-bit byte
 * offsets: an operand over 4 GiB returns MOE_ERR_UNSUPPORTED.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* NULL pointer, negative size, k > E, unknown enum, ... */
  MOE_ERR_UNSUPPORTED = -2, /* valid but outside the sizes the kernels handle */
  MOE_ERR_WORKSPACE = -3,   /* workspace NULL or smaller than the *_workspace_bytes value */
  MOE_ERR_HIP = -4          /* a HIP launch or runtime call failed */
};

enum moe_dtype { MOE_F32 = 0, MOE_BF16 = 1 };

enum moe_score_mode {
  MOE_SOFTMAX_THEN_TOPK = 0, /* p = softmax over all E scores; weights = p of the chosen k */
  MOE_TOPK_THEN_SOFTMAX = 1, /* weights = softmax over the chosen k scores */
  MOE_SIGMOID_THEN_TOPK = 2  /* g = sigmoid(score); weights = g of the chosen k over their sum */
};

#define MOE_MAX_EXPERTS 256
#define MOE_NEAR_TIE_GAP 1e-4

/*
 * moe_route -- router GEMM, top-k selection and gate weights.
 * Sources: Latent "Mixture of experts", "Where the experts live" (s = W_r x and
 * the gate equation); The Residual Stream "Mixture of Experts: More Parameters,
 * Same FLOPs", "The router" (renormalized top-k equation, worked example;
 * DeepSeek-V3's sigmoid scores normalized over the chosen experts) and "Keeping
 * the load even" (bias balancing: a per-expert bias that chooses but never
 * weights); Transformers & Math 17.2 (the two softmax orders); ML Interview
 * Notes, the Router listing.
 *
 *   x           device [T][d] dtype        token vectors
 *   w_router    device [E][d] dtype        router weight (nn.Linear(d, E) layout)
 *   logit_bias  device [E] float32 or NULL added to every token's scores before
 *                                         selection and softmax
 *   select_bias device [E] float32 or NULL added only to the selection keys:
 *                                         softmax(s) + b (MOE_SOFTMAX_THEN_TOPK),
 *                                         s + b (MOE_TOPK_THEN_SOFTMAX) or
 *                                         sigmoid(s) + b (MOE_SIGMOID_THEN_TOPK);
 *                                         never in the weights or the logits.
 *                                         Without it the key is s, or sigmoid(s).
 *   logits      device [T][E] float32 out  s = x W_r^T (+ logit_bias), float32
 *                                         accumulation (the summation order depends
 *                                         on T: up to 2048 bf16 tokens take a
 *                                         split-d kernel; results are deterministic
 *                                         for given T)
 *   topk_idx    device [T][k] int32 out    the k highest keys, best first; equal
 *                                         keys go to the lower expert index
 *   topk_w      device [T][k] float32 out  gate weights by `mode` from the scores;
 *                                         with MOE_SOFTMAX_THEN_TOPK and renorm != 0
 *                                         they are divided by their sum (renorm is
 *                                         ignored by the other two modes; sigmoid
 *                                         weights are always normalized)
 *   near_tie    device [T] int32 out       1 where the k-th best key exceeds the
 *                                         (k+1)-th by less than MOE_NEAR_TIE_GAP
 *                                         (0 when k = E)
 */
int moe_route(const void* x, const void* w_router, const float* logit_bias, const float* select_bias, int dtype,
              int T, int d, int E, int k, int mode, int renorm,
              float* logits, int32_t* topk_idx, float* topk_w, int32_t* near_tie,
              hipStream_t stream);

/*
 * moe_bias_update -- one step of bias balancing.
 * Source: The Residual Stream, "Keeping the load even" (after every step, raise
 * an expert's bias by a fixed amount if it got fewer than its share of tokens,
 * lower it if it got more) and the MoE listing's update.
 *
 *   counts      device [E] int32           demand counts of the step (moe_permute)
 *   T, k, E                                the step's tokens, slots, experts
 *   rate        the fixed step
 *   select_bias device [E] float32 in/out  b_e += rate * sign(T k - E counts_e),
 *                                         in float32 (the share T k / E is compared
 *                                         exactly, in integers)
 * T = 0 leaves the bias unchanged.  A NaN rate returns MOE_ERR_INVALID_ARG.
 */
int moe_bias_update(const int32_t* counts, int T, int k, int E, float rate, float* select_bias,
                    hipStream_t stream);

/*
 * moe_permute -- per-expert histogram, capacity, stable permutation, gather.
 * Sources: ML Interview Notes, MoELayer listing (per-expert (token, slot) pairs)
 * and "Capacity factor" (tokens arriving at a full expert are dropped);
 * Transformers & Math 17.5 (capacity, dropped tokens keep their other experts);
 * Understanding Data, "The maths", "Capacity".
 *
 * Assignment (t, j) goes to expert e = topk_idx[t][j].  Assignments reach their
 * experts in ascending order of t*k + j; rank(t, j) is the number of earlier
 * assignments to the same expert.  With capacity >= 0 an assignment is kept
 * iff rank < capacity; capacity < 0 means dropless.  Expert ids outside [0, E)
 * are ignored (counted nowhere, row -1).
 *
 *   counts     device [E] int32 out       demand per expert, before the cap
 *   offsets    device [E+1] int32 out     offsets[0] = 0, offsets[e+1] =
 *                                        offsets[e] + min(counts[e], capacity)
 *   row_of     device [T][k] int32 out    offsets[e] + rank, or -1 when dropped
 *   perm_token device [T*k] int32 out     token of each row; rows >= offsets[E]
 *                                        are left untouched
 *   x_perm     device [T*k][d] dtype out  x_perm[r] = x[perm_token[r]] for
 *                                        r < offsets[E]; may be NULL (then x may
 *                                        be NULL too): no copy is made, and the
 *                                        expert GEMM gathers rows through
 *                                        perm_token instead (row_index below)
 *   workspace  device, >= moe_permute_workspace_bytes(T, k, E) bytes, scratch
 */
int moe_permute(const int32_t* topk_idx, int T, int k, int E, int64_t capacity,
                const void* x, int dtype, int d,
                int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* perm_token,
                void* x_perm, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_permute_padded -- the same dispatch in a capacity-padded layout: each
 * expert owns `capacity` (C) slots, as in the fixed-size buffers an
 * expert-parallel exchange sends.
 * Sources: Transformers & Math 17.5 (each expert processes at most C tokens);
 * Understanding Data, "The maths", "Capacity"; The Residual Stream, "What
 * experts cost at serving time" (experts spread over devices).
 *
 * Arguments as moe_permute, except:
 *   capacity   C >= 1 (required); E * C <= 2^31 - 1
 *   offsets    device [E+1] int32 out    e * C (the group bounds for the grouped
 *                                        GEMMs over all E * C slots)
 *   row_of     device [T][k] int32 out   slot e * C + rank of the assignment,
 *                                        -1 when dropped
 *   slot_token device [E*C] int32 out    token of each slot; -1 for the slots past
 *                                        an expert's kept count min(counts_e, C)
 *   x_slots    device [E*C][d] or NULL   x[slot_token[s]], zero rows for padding
 * Padding slots take part in the grouped GEMMs (their outputs are computed and
 * never read by moe_combine).
 */
int moe_permute_padded(const int32_t* topk_idx, int T, int k, int E, int64_t capacity, const void* x, int dtype,
                       int d, int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* slot_token,
                       void* x_slots, void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t moe_permute_workspace_bytes(int T, int k, int E);

/*
 * moe_permute_noalloc -- moe_permute with no workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Arguments, results and
 * errors as moe_permute (same kernels, bit-identical results).
 *
 * The scratch moe_permute takes as `workspace` lives instead in one
 * MOE_NOALLOC_SCRATCH_BYTES array in the library's device memory, one copy per
 * GPU, held from the library's load until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree); its first call on a device looks up that
 * device's copy (hipGetSymbolAddress) with the device current.
 *   - Sizes whose moe_permute_workspace_bytes(T, k, E) exceeds
 *     MOE_NOALLOC_SCRATCH_BYTES (4 MiB: T*k up to 2^20 assignments at E = 256,
 *     2^21 at E = 128) return MOE_ERR_UNSUPPORTED before anything is enqueued.
 *   - Every call on one GPU shares that GPU's array, which keeps the last call's
 *     contents; each call writes every word it reads first, so nothing needs
 *     clearing.  Calls that overlap on one GPU (different streams, or host
 *     threads) race on the array and must be ordered by the caller.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
int moe_permute_noalloc(const int32_t* topk_idx, int T, int k, int E, int64_t capacity,
                        const void* x, int dtype, int d,
                        int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* perm_token,
                        void* x_perm, hipStream_t stream);

/*
 * moe_capacity -- C = ceil(phi * k * T / E), evaluated exactly on the binary
 * value of phi (Transformers & Math 17.5 equation; Understanding Data,
 * "Capacity").  Returns -1 (dropless) when phi is not finite or negative, or
 * when T < 0, k < 1 or E < 1.
 */
int64_t moe_capacity(int64_t T, int k, int E, double phi);

/*
 * moe_grouped_gate_up -- first half of G SwiGLU experts as one variable-size
 * grouped GEMM: for each group g and each row r in [offsets[g], offsets[g+1]),
 *     a[r] = SiLU(h_r gate[g]^T) * (h_r up[g]^T),  SiLU(z) = z/(1+e^-z)
 * where h_r = x[r], or h_r = x[row_index[r]] when row_index is given.
 * Sources: The Residual Stream, "An MoE tiny GPT" listing (F.silu(h @ gate) *
 * (h @ up)); ML Interview Notes "Capacity factor" (dropless routing with
 * variable-size grouped GEMMs).
 *
 *   x        device [max_rows][d] dtype (row_index NULL) or [src_rows][d]
 *   row_index device [max_rows] int32 or NULL: the dispatch permutation
 *                                        (perm_token of moe_permute), values
 *                                        clamped to [0, src_rows); lets the GEMM
 *                                        gather token rows itself
 *   src_rows number of rows of x when row_index is given (ignored otherwise)
 *   offsets  device [G+1] int32           group row ranges; values are clamped to
 *                                        [0, max_rows]; rows outside every range
 *                                        are not written
 *   w_gate, w_up device [G][F][d] dtype
 *   a        device [max_rows][F] dtype out
 * G in [1, 256].  max_rows >= 0 bounds the launch; the true row count is read
 * from offsets on the device, so no host round trip is needed.
 */
int moe_grouped_gate_up(const void* x, const int32_t* row_index, int src_rows,
                        const int32_t* offsets, int G, int max_rows,
                        int d, int F, const void* w_gate, const void* w_up, int dtype,
                        void* a, hipStream_t stream);

/*
 * moe_grouped_down -- second half: y_perm[r] = a[r] down[g]^T for r in group g.
 *   a        device [max_rows][F] dtype
 *   w_down   device [G][d][F] dtype
 *   y_perm   device [max_rows][d] dtype out
 */
int moe_grouped_down(const void* a, const int32_t* offsets, int G, int max_rows,
                     int F, int d, const void* w_down, int dtype, void* y_perm,
                     hipStream_t stream);

/*
 * moe_grouped_swiglu -- moe_grouped_gate_up then moe_grouped_down: G SwiGLU
 * experts (SiLU(h gate^T) * (h up^T)) down^T over their row groups.  The shared
 * expert of a layer is this call with G = 1, offsets = {0, T}, x the tokens and
 * no row index (Transformers & Math 17.3; ML Interview Notes, MoELayer,
 * always-on experts).
 */
int moe_grouped_swiglu(const void* x, const int32_t* row_index, int src_rows,
                       const int32_t* offsets, int G, int max_rows,
                       int d, int F, const void* w_gate, const void* w_up,
                       const void* w_down, int dtype, void* a, void* y_perm,
                       hipStream_t stream);

/*
 * moe_combine -- y[t] = sum over j with row_of[t][j] >= 0 of
 *                topk_w[t][j] * y_perm[row_of[t][j]]  (+ shared_y[t]).
 * Sources: Transformers & Math 17.2 equation (routed sum plus the shared
 * expert, unweighted); ML Interview Notes, MoELayer (out[tok] += weights *
 * expert(x)); Transformers & Math 17.5 (a dropped slot adds nothing and the
 * other weights are kept as they are).
 * The sum runs in slot order in float32 and is rounded once: the result is
 * deterministic.  row_of values outside [0, y_rows) count as dropped.
 *
 *   y_perm   device [y_rows][d] dtype: T*k rows for the compact layout
 *            (moe_permute), E*C for the padded one (moe_permute_padded).
 *            With y_rows = 0 every slot counts as dropped, no row is read and
 *            y_perm may be NULL (y is then shared_y, or zeros).
 *   row_of   device [T][k] int32; topk_w device [T][k] float32;
 *   shared_y device [T][d] dtype or NULL;
 *   y        device [T][d] dtype out (every row written)
 */
int moe_combine(const void* y_perm, int y_rows, const int32_t* row_of, const float* topk_w,
                const void* shared_y, int dtype, int T, int k, int d, void* y,
                hipStream_t stream);

/*
 * moe_grouped_down_combine -- moe_grouped_down and moe_combine in one call, with
 * the weighted sum done in the down GEMM's epilogue: each product row r, rounded
 * to dtype as y_perm would hold it, is multiplied by its slot's gate weight and
 * added with float32 atomics to an accumulator row of token perm_token[r]; y is
 * then accumulator + shared_y, rounded once.  No y_perm is written or read.
 * Sources: ML Interview Notes, MoELayer (out[tok] += weights * expert(x), a
 * weighted scatter-add); The Residual Stream, "An MoE tiny GPT" (index_add_ of
 * the weighted expert outputs); Transformers & Math 17.2 equation (plus the
 * shared expert, unweighted).
 * The result equals moe_grouped_down followed by moe_combine up to the order of
 * the float32 additions, which atomics do not fix: y may differ from run to run
 * in the last bit of a sum before rounding (at most one dtype ulp after it).
 *
 *   a, offsets, G, max_rows, F, d, w_down, dtype   as for moe_grouped_down
 *   perm_token device [max_rows] int32: the token of each row (moe_permute's
 *            perm_token, or moe_permute_padded's slot_token, -1 for padding);
 *            rows whose value lies outside [0, T) add nothing.  It must be the
 *            inverse of row_of, as those calls write it.
 *   row_of, topk_w, shared_y, T, k, y              as for moe_combine (y_rows =
 *            max_rows: row_of values outside [0, max_rows) count as dropped)
 *   workspace device, >= moe_down_combine_workspace_bytes(T, d, max_rows) bytes:
 *            the float32 accumulator [T][d] and one weight per row; zeroed and
 *            written by the call itself
 * Calls on one stream are ordered; two calls that share a workspace must not
 * run concurrently.
 */
int moe_grouped_down_combine(const void* a, const int32_t* offsets, int G, int max_rows, int F, int d,
                             const void* w_down, int dtype, const int32_t* perm_token, const int32_t* row_of,
                             const float* topk_w, int T, int k, const void* shared_y, void* y, void* workspace,
                             size_t workspace_bytes, hipStream_t stream);
size_t moe_down_combine_workspace_bytes(int T, int d, int max_rows);

/*
 * moe_stats -- balance statistics.
 * Sources: Transformers & Math 17.4 equation (L_aux = alpha N_E sum f_i P_i);
 * The Residual Stream "Keeping the load even" and the MoE listing (f = counts /
 * counts.sum(), P = mean router probability); Latent "Keeping the load
 * balanced"; Understanding Data "Load imbalance" (measured on demand).
 *
 *   counts   device [E] int32            demand per expert (moe_permute output)
 *   logits   device [T][E] float32       router scores (moe_route output)
 *   f        device [E] float32 out      counts[i] / (T k), one float32 division
 *   P        device [E] float32 out      mean over tokens of softmax(logits[t])[i]
 *   l_aux    device [1] float32 out      alpha * E * sum_i f_i P_i
 *   max_over_mean device [1] float32 out E * max_i counts[i] / (T k)
 *   workspace device, >= moe_stats_workspace_bytes(T, E) bytes, scratch
 * With T = 0 nothing is written.
 */
int moe_stats(const int32_t* counts, const float* logits, int T, int k, int E, float alpha,
              float* f, float* P, float* l_aux, float* max_over_mean,
              void* workspace, size_t workspace_bytes, hipStream_t stream);

size_t moe_stats_workspace_bytes(int T, int E);

/*
 * moe_layer_forward -- the whole layer in one call: moe_route, moe_permute
 * (compact layout, no x_perm), moe_grouped_gate_up (rows gathered through
 * perm_token), moe_grouped_down, the shared expert (moe_grouped_swiglu with
 * G = 1, when F_shared > 0), moe_combine and moe_stats, in that order, with the
 * arguments of the struct below.  Every call's checks run first; on a bad
 * argument nothing is enqueued and the status and moe_last_error() are those of
 * the first call that rejects it.
 * With bf16, T <= 64 and T k <= 512 (decode batches) the selection, the
 * dispatch and the statistics run as one block after the score kernel, with no
 * launch between them.  With bf16, 64 < E <= 128, k = 8 and T >= 4096 the
 * router's blocks also write the dispatch's per-block histograms and the
 * statistics' partial sums.  Either way the results are bit-identical to the
 * separate calls.
 * Sources: the five steps as each call cites them; Transformers & Math 17.2
 * equation for the layer sum.
 *
 * Every pointer is a device pointer, with the shape and meaning given for the
 * call that takes it; R = T k.
 */
typedef struct moe_layer_args {
  int dtype, T, d, E, k, F;
  int F_shared;                 /* 0: no shared expert */
  int mode, renorm;             /* as for moe_route */
  int64_t capacity;             /* moe_capacity(T, k, E, phi), < 0: dropless */
  float alpha;                  /* L_aux coefficient */
  const void* x;                /* [T][d] */
  const void* w_router;         /* [E][d] */
  const float* logit_bias;      /* [E] or NULL */
  const float* select_bias;     /* [E] or NULL */
  const void* w_gate;           /* [E][F][d] */
  const void* w_up;             /* [E][F][d] */
  const void* w_down;           /* [E][d][F] */
  const void* shared_gate;      /* [F_shared][d], with F_shared > 0 */
  const void* shared_up;        /* [F_shared][d] */
  const void* shared_down;      /* [d][F_shared] */
  const int32_t* shared_offsets;  /* [2] = {0, T}, with F_shared > 0 */
  float* logits;                /* [T][E] out */
  int32_t* topk_idx;            /* [T][k] out */
  float* topk_w;                /* [T][k] out */
  int32_t* near_tie;            /* [T] out */
  int32_t* counts;              /* [E] out */
  int32_t* offsets;             /* [E+1] out */
  int32_t* row_of;              /* [T][k] out */
  int32_t* perm_token;          /* [R] out */
  void* a;                      /* [R][F] out */
  void* y_perm;                 /* [R][d] out */
  void* shared_a;               /* [T][F_shared] out, with F_shared > 0 */
  void* shared_y;               /* [T][d] out, with F_shared > 0 */
  void* y;                      /* [T][d] out */
  float* f;                     /* [E] out */
  float* P;                     /* [E] out */
  float* l_aux;                 /* [1] out */
  float* max_over_mean;         /* [1] out */
  void* permute_workspace;      /* >= moe_permute_workspace_bytes(T, k, E) */
  size_t permute_workspace_bytes;
  void* stats_workspace;        /* >= moe_stats_workspace_bytes(T, E) */
  size_t stats_workspace_bytes;
  /* Optional: with side_stream, fork_event and join_event all given, the
   * statistics run on side_stream after the work before the combine, and
   * `stream` waits for them before the call returns its last operation.  Not in
   * the decode form above, nor where the router computes the statistics' partial
   * sums itself (bf16, 64 < E <= 128, k = 8, T >= 4096): there their final
   * reduction runs on `stream` right after the dispatch.  The events are the
   * caller's (hipEventCreate...). */
  hipStream_t side_stream;
  hipEvent_t fork_event;
  hipEvent_t join_event;
  /* Optional timing marks, each recorded on `stream` if not NULL: before the
   * gate/up GEMM, after it, after the down GEMM, after the shared expert. */
  hipEvent_t marks[4];
} moe_layer_args;

int moe_layer_forward(const moe_layer_args* args, hipStream_t stream);
/* sizeof(moe_layer_args), for bindings that lay the struct out themselves. */
size_t moe_layer_args_size(void);

/* Human-readable name of a moe_status value. */
const char* moe_status_string(int status);

/* Description of the last failure on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
