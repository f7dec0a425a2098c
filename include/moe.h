/*
 * moe.h -- C ABI of libmoe.so: the routed Mixture-of-Experts layer of a
 * fine-grained MoE at inference, with decoupled top-k1/k2 weights, on one
 * AMD Instinct MI355X (gfx950).
 *
 * The method ("Paper of the Week #3 - Half the FLOPs Is Not Half the Time",
 * section "The Receipt", Eq. 2): a token runs its k1 most probable experts and
 * weights each by its probability divided by the probability mass of its k2
 * most probable experts,
 *
 *     w_i = p_i / sum_{j in Top-k2} p_j      for i in Top-k1,
 *
 * so k2 = k1 is standard top-k renormalisation and k2 = E is none.  The
 * router method of the same page (section "Ship It - Code of the Week")
 * computes the probabilities in fp32 from a linear router and keeps
 * min(k2, E) candidates.  An expert is a gated MLP whose channel c owns one
 * gate row, one up row and one down column ("Channel Selection for
 * Mixture-of-Experts Decoding Needs No Calibration Data", section 2
 * "Background"); the activation is silu on the gate times the up projection.
 *
 * Numerical contract of the route (softmax, ranking, Eq. 2), fp32 throughout:
 *   m = max_e l_e;  d_e = l_e - m;  e_e = exp(d_e) evaluated as
 *   2^n * P7(r) with n = rint(d * log2 e), r = d - n ln2 (Cody & Waite's
 *   two-constant reduction) and P7 the degree-7 Taylor polynomial by Horner
 *   with fused multiply-adds, and e_e = 0 for d_e < -80;
 *   S = pairwise sum of e over the next power of two (zero padded);
 *   p_e = e_e / S (IEEE division);  ranking by p descending, lower index
 *   first on equal p;  M = sum of the first min(k2,E) ranked p, left to right;
 *   w_r = p_r / M, or w_r = p_r when k2 >= E.
 * Given identical logits the ids and weights are reproducible bit for bit.
 *
 * Conventions for every entry point:
 *  - all tensors are row-major and contiguous, in device memory of the
 *    current HIP device, owned by the caller; the library keeps no pointer
 *    after returning and allocates no device memory (its one device buffer
 *    is the fixed scratch array of moe_forward_noalloc, which each device the
 *    library runs on holds until the process ends);
 *  - `stream` is a hipStream_t (NULL = the null stream); all work is enqueued
 *    on it with no host synchronisation; outputs are overwritten;
 *  - argument errors are returned before anything is launched; a failed launch
 *    returns MOE_EHIP (text in moe_last_error_str()); device faults surface at
 *    the caller's next synchronisation, as usual for HIP;
 *  - logits must be finite (a precondition: with a non-finite logit the
 *    outputs for that token are unspecified);
 *  - entry points never throw and are safe to call from several host threads;
 *  - with MOE_DEBUG set in the environment (to anything but "0"), every
 *    moe_forward* call also waits for its work and returns the device status
 *    of moe_workspace_status (so it cannot be captured in a HIP graph).
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 2
#define MOE_MAX_EXPERTS 1024

typedef enum {
    MOE_OK = 0,
    MOE_EINVAL = 1,     /* a size or k argument out of range, or a NULL pointer */
    MOE_EALIGN = 2,     /* a pointer without the required alignment */
    MOE_EWORKSPACE = 3, /* workspace NULL, misaligned or too small */
    MOE_ENOTSUP = 4,    /* unsupported dtype combination or shape for a path */
    MOE_EHIP = 5,       /* a HIP runtime call failed */
    MOE_EDEVICE = 6     /* a wait inside a kernel gave up (moe_workspace_status) */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* moe_forward flags: force one of the execution paths (0 = choose by batch
 * size and shape: one token runs as a single launch whose workgroups hand the
 * route and the activations over through the workspace; decode batches take
 * GROUPED, large batches PREFILL).  All paths compute the same layer; they
 * differ in kernels:
 *   GROUPED router, route, per-expert plan, gate/up, down and combine kernels
 *           (grouped GEMVs that read each activated expert once); with one
 *           token it replaces the single launch;
 *   PREFILL the same steps with the expert projections as bf16 MFMA grouped
 *           GEMMs (chosen from 512 assignments T*k1 on, when the activated
 *           experts average two rows or more).
 * A forced path that cannot take the call's shapes returns MOE_ENOTSUP.  Bit
 * value 1 is not a flag (MOE_EINVAL). */
#define MOE_FLAG_FORCE_GROUPED 2u
#define MOE_FLAG_FORCE_PREFILL 4u

/* moe_forward flag: the bf16 router -- the router method of "Paper of the
 * Week #3" (section "Ship It - Code of the Week") as it runs on a bf16 model,
 * where the linear layer runs in the model's dtype and the weights are cast
 * back to the logits' dtype.  With it:
 *   Wr is bf16 [E, H] and br must be NULL (MOE_EINVAL otherwise);
 *   logits[t, e] = bf16(x[t] . Wr[e]): fp32 accumulation of the exact bf16
 *       products, rounded once to bf16 (nearest, ties to even);
 *   the softmax, ranking and Eq. 2 run in fp32 on those logits, exactly as
 *       without the flag;
 *   each weight is then rounded to bf16, and the experts are scaled by it.
 * logits_out and w_out still receive fp32 arrays, holding the bf16 values.
 * At k1 = k2 this is the stock renormalising bf16 router.  It needs the
 * (BF16, BF16) dtype pair (MOE_ENOTSUP otherwise) and combines with
 * MOE_FLAG_FORCE_GROUPED or MOE_FLAG_FORCE_PREFILL. */
#define MOE_FLAG_ROUTER_BF16 8u

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text for a status code. */
const char *moe_status_str(int status);

/* Text of the last MOE_EHIP / argument error on the calling thread. */
const char *moe_last_error_str(void);

/*
 * moe_route -- softmax, ranking and Eq. 2 weights from given router logits
 * (the router method of "Paper of the Week #3", section "Ship It - Code of
 * the Week", from the softmax on; weights per Eq. 2 of section "The Receipt").
 *
 *   logits  [T, E] fp32, finite.                   4-byte aligned
 *   ids     [T, k1] int32 out: expert indices in rank order
 *   weights [T, k1] fp32 out: Eq. 2 weights in the same order
 *   1 <= E <= 1024;  1 <= k1 <= E;  k2 >= k1 (k2 > E behaves as k2 = E);
 *   0 <= T <= 2^18.  T = 0 returns MOE_OK and launches nothing.
 */
int moe_route(const float *logits, int64_t T, int32_t E, int32_t k1,
              int32_t k2, int32_t *ids, float *weights, void *stream);

/*
 * moe_forward_workspace -- bytes of device workspace moe_forward needs for
 * these sizes (a multiple of 256).  0 for invalid sizes.
 */
size_t moe_forward_workspace(int64_t T, int32_t H, int32_t E, int32_t I,
                             int32_t k1, int32_t act_dtype, int32_t w_dtype);

/*
 * moe_forward -- the whole routed MoE layer: router logits, route (as
 * moe_route), the activated experts and their weighted sum,
 *
 *   y[t] = sum_{r<k1} w[t,r] * Wdown[e] (silu(Wgate[e] x[t]) * (Wup[e] x[t])),
 *   e = ids[t,r],  logits[t] = Wr x[t] (+ br).
 *
 *   x      [T, H]    act_dtype (MOE_F32 or MOE_BF16)          16-byte aligned
 *   Wr     [E, H]    fp32 router weight (bf16 with MOE_FLAG_ROUTER_BF16)
 *                                                            16-byte aligned
 *   br     [E]       fp32 router bias, or NULL                 4-byte aligned
 *   Wgate  [E, I, H] w_dtype: row c of expert e = gate row of channel c
 *   Wup    [E, I, H] w_dtype: row c of expert e = up row of channel c
 *   Wdown  [E, H, I] w_dtype: column c of expert e = down column of channel c
 *                                                   (all three 16-byte aligned)
 *   y      [T, H]    act_dtype out                            16-byte aligned
 *   logits_out [T,E] fp32, ids_out [T,k1] int32, w_out [T,k1] fp32: optional
 *          copies of the route (NULL to skip), 4-byte aligned
 *   workspace: device memory of at least moe_forward_workspace(...) bytes,
 *          256-byte aligned, ZERO-FILLED before its first use.  It carries
 *          state from call to call, so one zero fill at allocation lasts for
 *          its lifetime, whatever the shapes of later calls: an epoch word
 *          that advances on every call that hands values over as tagged
 *          words (one-token calls and the 2-64-token router + route; the
 *          epoch is the source of the tags, and the words sit at fixed
 *          places of regions of their own, so a stale word cannot carry the
 *          current tag until 2^31 calls have passed), the error word read by
 *          moe_workspace_status, and counters that return to zero after
 *          every call.  Calls that run concurrently need separate
 *          workspaces.
 *   flags: 0 or one MOE_FLAG_FORCE_* value, optionally with
 *          MOE_FLAG_ROUTER_BF16.
 *
 *   Supported dtype pairs (act, w): (F32, F32) and (BF16, BF16); accumulation
 *   is fp32.  1 <= E <= 1024; H and I multiples of 8; 1 <= k1 <= E;
 *   k2 >= k1; 0 <= T <= 2^18; E*H and E*I at most 2^25; T*H and T*E at most
 *   2^28 (and T*k1 small enough for the prefill GEMM grids; MOE_EINVAL
 *   otherwise).  T = 0 returns MOE_OK and launches nothing.
 *   Identical inputs give bitwise identical logits, ids, weights and y.
 */
int moe_forward(const void *x, int32_t act_dtype, int64_t T, int32_t H,
                const void *Wr, const float *br, int32_t E,
                const void *Wgate, const void *Wup, const void *Wdown,
                int32_t w_dtype, int32_t I, int32_t k1, int32_t k2, void *y,
                float *logits_out, int32_t *ids_out, float *w_out,
                uint32_t flags, void *workspace, size_t workspace_bytes,
                void *stream);

/*
 * moe_forward_noalloc -- moe_forward without a workspace, for callers that
 * cannot allocate device memory (code under HIP graph capture, serving loops
 * that forbid allocation, harnesses without an allocator).  It computes
 * exactly what moe_forward computes, with the same kernels and paths, using
 * a fixed device array of moe_noalloc_scratch_bytes() bytes (32 MiB) in
 * place of the workspace; it calls no hipMalloc, hipFree or other
 * allocating routine.  Sizes whose moe_forward_workspace exceeds the array
 * return MOE_EWORKSPACE before anything is launched (the array holds the
 * decode shapes: e.g. up to 256 tokens of an H=2048, E=128, I=768, k1=8
 * layer, or 64 tokens of an H=4096, E=512, I=1024, k1=10 one).
 *
 * The array is shared by every call on a device and keeps the last call's
 * contents; the first call on a device clears the part that must start at
 * zero (a fill kernel on that call's stream).  Calls that overlap on one
 * device (several streams or threads) race on it and must be serialised by
 * the caller.  Arguments, outputs and errors as for moe_forward.
 */
int moe_forward_noalloc(const void *x, int32_t act_dtype, int64_t T, int32_t H,
                        const void *Wr, const float *br, int32_t E,
                        const void *Wgate, const void *Wup, const void *Wdown,
                        int32_t w_dtype, int32_t I, int32_t k1, int32_t k2, void *y,
                        float *logits_out, int32_t *ids_out, float *w_out,
                        uint32_t flags, void *stream);

/* moe_noalloc_scratch_bytes -- size of moe_forward_noalloc's device array. */
size_t moe_noalloc_scratch_bytes(void);

/*
 * moe_forward_shared -- moe_forward plus a shared expert, which runs on every
 * token beside the routed ones ("Channel Selection for Mixture-of-Experts
 * Decoding Needs No Calibration Data", appendix B "Experimental setup":
 * shared experts always run in full).  The pages do not give its gating; the
 * layer computed here is
 *
 *   y[t] = sum_{r<k1} w[t,r] * E_{ids[t,r]}(x[t])  +  g[t] * S(x[t]),
 *   S(x) = Sdown (silu(Sgate x) * (Sup x)),
 *   g[t] = sigmoid(x[t] . sgate) with a gate vector, 1 with sgate = NULL.
 *
 *   Sgate  [Is, H]   w_dtype: row c = gate row of shared channel c  16-byte aligned
 *   Sup    [Is, H]   w_dtype: row c = up row of shared channel c    16-byte aligned
 *   Sdown  [H, Is]   w_dtype: column c = down column of channel c   16-byte aligned
 *   Is     shared channels: a positive multiple of 8, H * Is <= 2^31
 *   sgate  [H] fp32 gate vector, or NULL                            4-byte aligned
 * Every other argument, and the route outputs, as for moe_forward (the
 * route is unchanged by the shared expert; T*Is at most 2^28).  The
 * workspace size comes from moe_forward_shared_workspace.
 * MOE_FLAG_FORCE_PREFILL also needs Is % 64 == 0.  For one token with
 * Is % I == 0 the shared expert runs inside the single launch of the layer,
 * streaming while the token is routed.
 */
int moe_forward_shared(const void *x, int32_t act_dtype, int64_t T, int32_t H,
                       const void *Wr, const float *br, int32_t E,
                       const void *Wgate, const void *Wup, const void *Wdown,
                       int32_t w_dtype, int32_t I, int32_t k1, int32_t k2,
                       const void *Sgate, const void *Sup, const void *Sdown,
                       int32_t Is, const float *sgate, void *y,
                       float *logits_out, int32_t *ids_out, float *w_out,
                       uint32_t flags, void *workspace, size_t workspace_bytes,
                       void *stream);

/* moe_forward_shared_workspace -- bytes of workspace moe_forward_shared needs
 * (a multiple of 256); 0 for invalid sizes.  Is = 0 gives
 * moe_forward_workspace's size. */
size_t moe_forward_shared_workspace(int64_t T, int32_t H, int32_t E, int32_t I,
                                    int32_t k1, int32_t Is, int32_t act_dtype,
                                    int32_t w_dtype);

/*
 * moe_down_column_norms -- dnorm[e, c] = ||Wdown[e, :, c]||_2, the norm of
 * each channel's down column ("Channel Selection for Mixture-of-Experts
 * Decoding Needs No Calibration Data", section 5.2 scales channel scores by
 * it), accumulated in fp32.  Computed once per weight set; an input of
 * moe_forward_channel_topk.
 *
 *   Wdown  [E, H, I] w_dtype (MOE_F32 or MOE_BF16)               16-byte aligned
 *   dnorm  [E, I] fp32 out                                         4-byte aligned
 *          (moe_forward_channel_topk reads it with 16-byte alignment)
 */
int moe_down_column_norms(const void *Wdown, int32_t w_dtype, int32_t E,
                          int32_t H, int32_t I, float *dnorm, void *stream);

/*
 * moe_down_columns -- the column copy of the down weights,
 * Wdown_cols[e, c, :] = Wdown[e, :, c]: each channel's down column as one
 * contiguous row ("Channel Selection for Mixture-of-Experts Decoding Needs No
 * Calibration Data", section 2: a channel owns one down column; section 5.2
 * reads only the selected channels' weights).  Made once per weight set, like
 * moe_down_column_norms; an input of moe_forward_channel_topk.
 *
 *   Wdown       [E, H, I] w_dtype (MOE_F32 or MOE_BF16)          16-byte aligned
 *   Wdown_cols  [E, I, H] w_dtype out                            16-byte aligned
 */
int moe_down_columns(const void *Wdown, int32_t w_dtype, int32_t E, int32_t H, int32_t I,
                     void *Wdown_cols, void *stream);

/*
 * moe_forward_channel_topk -- moe_forward with channel selection inside the
 * activated experts ("Channel Selection ...", section 5.2; section 2: a
 * channel owns one gate row, one up row and one down column).  After the
 * route and the gate/up projections, each channel (r, c) of a token's k1
 * activated experts is scored
 *
 *   score = w_r * dnorm[e_r, c] * |silu(g) * u|     (output units),
 *
 * the `keep` highest scores over the token's k1*I channels are kept (exact
 * top-k; equal scores keep the lower flat index j = r*I + c), and
 *
 *   y[t] = sum over the kept channels of w_r * a[r, c] * Wdown[e_r, :, c].
 *
 * keep = k1*I is the full layer (up to rounding), keep = 0 gives y = 0.
 * Arguments as moe_forward, plus:
 *   dnorm      [E, I] fp32 from moe_down_column_norms          16-byte aligned
 *   keep       0 <= keep <= k1*I; k1*I <= 8192 (MOE_ENOTSUP beyond)
 *   Wdown_cols [E, I, H] from moe_down_columns, or NULL        16-byte aligned
 *              With it the down projection reads only the kept channels'
 *              columns (keep rows of H values per token, summed in a fixed
 *              order: flat-channel order within fixed groups, then the
 *              groups' sums in a fixed tree); without it, every down row is
 *              read with the unkept activations set to zero.
 *   scores_out [T, k1*I] fp32, or NULL: the scores the selection used
 *                                                              16-byte aligned
 *   kept_out   [T, k1*I] uint8, or NULL: 1 for a kept channel, else 0
 *                                                               8-byte aligned
 * It runs on the grouped path: MOE_FLAG_FORCE_PREFILL returns MOE_ENOTSUP;
 * MOE_FLAG_ROUTER_BF16 applies.  The workspace size comes from
 * moe_forward_channel_topk_workspace.
 */
int moe_forward_channel_topk(const void *x, int32_t act_dtype, int64_t T,
                             int32_t H, const void *Wr, const float *br,
                             int32_t E, const void *Wgate, const void *Wup,
                             const void *Wdown, int32_t w_dtype, int32_t I,
                             int32_t k1, int32_t k2, const float *dnorm,
                             int32_t keep, const void *Wdown_cols, void *y,
                             float *logits_out, int32_t *ids_out, float *w_out,
                             float *scores_out, uint8_t *kept_out, uint32_t flags,
                             void *workspace, size_t workspace_bytes, void *stream);

/* moe_forward_channel_topk_workspace -- bytes of workspace
 * moe_forward_channel_topk needs (a multiple of 256); 0 for invalid sizes. */
size_t moe_forward_channel_topk_workspace(int64_t T, int32_t H, int32_t E, int32_t I,
                                          int32_t k1, int32_t act_dtype, int32_t w_dtype);

/*
 * moe_profile_launch -- profiling aid; changes no output.  Arms the NEXT
 * moe_forward call on the calling thread: it records the hipEvent_t `start`
 * on its stream immediately before its kernel launch number `launch` (0 =
 * the call's first launch) and `stop` immediately after it, then disarms.
 * A call with fewer launches records nothing.  start and stop are created and
 * owned by the caller (NULL disarms).  Returns MOE_EINVAL for launch < 0.
 *
 * moe_profile_launch_name -- the kernel name of the launch bracketed by the
 * last armed call on this thread ("" if none was), e.g. "b1_layer".
 */
int moe_profile_launch(int32_t launch, void *start, void *stop);
const char *moe_profile_launch_name(void);

/*
 * moe_workspace_status -- the device status of a workspace.  The one-token
 * kernel's workgroups hand the route and the activations to one another
 * through tagged words of the workspace, and the router + route launch of
 * 2..64 tokens makes its route blocks wait for every token's logits; every
 * such wait is bounded, and one that gives up (a precondition broken, or a
 * fault elsewhere on the device) lets its kernel run to the end with
 * unspecified outputs and sets an error word in the workspace.  The pages do
 * not cover this (their router runs in the framework's own kernels); it is
 * this library's contract.
 *
 * Waits for `stream`, reads the error word and resets it: MOE_EDEVICE if a
 * wait gave up in any call on this workspace since the last check, else
 * MOE_OK.  With MOE_EDEVICE it also clears the workspace's other
 * synchronisation counts, which a wait that gave up may have left set.  A
 * synchronous host call: not for use under graph capture.
 *   workspace  the moe_forward* workspace (256-byte aligned)
 */
int moe_workspace_status(void *workspace, void *stream);

/*
 * moe_debug_withhold_route -- test hook for the status above.  The next
 * `calls` calls on the calling thread that run a launch with such a wait
 * (the one-token kernel, or the router + route launch of 2..64 tokens) withhold
 * their hand-over: the one-token kernel does not publish its route, and the
 * route blocks of the router + route launch wait for a tag that no logit
 * carries.  Every such wait gives up
 * after `spin_limit` re-reads (>= 1); the kernels still run to the end,
 * reading only in-range expert rows, and the outputs are unspecified.
 * calls = 0 disarms.
 */
int moe_debug_withhold_route(int32_t calls, uint32_t spin_limit);

/*
 * moe_hbm_read_probe -- measurement aid: the read-only streaming ceiling.
 * Loads every 16-byte chunk of buf once with the streaming loads the expert
 * kernels use and writes one word per workgroup to out (an xor of what it
 * read, so the loads are live).  Timing a launch over a buffer much larger
 * than the device's last-level cache gives the read bandwidth a kernel can
 * reach, the ceiling for the decode kernels beside the HBM peak.
 *   buf     device buffer, 16-byte aligned; bytes a positive multiple of 16
 *   out     [blocks] uint32 device buffer, 4-byte aligned
 *   blocks  workgroups of 256 threads, 1..65536
 * Returns MOE_EINVAL / MOE_EALIGN on bad arguments, MOE_EHIP on a failed
 * launch.
 */
int moe_hbm_read_probe(const void *buf, size_t bytes, uint32_t *out, int32_t blocks,
                       void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
