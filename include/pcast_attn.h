/*
 * pcast_attn.h -- C ABI of the FP8 "P-cast" attention forward for AMD MI355X (gfx950).
 *
 * The operation (FlashAttention blog by marketmaker.cc, sections "Perché
 * l'attenzione è legata alla memoria", "L'algoritmo Flash Attention" and
 * "La ricorrenza softmax online"; P-cast summaries on gist.science, sections
 * 1 and 2):
 *
 *   O = softmax(Q K^T / sqrt(d) + bias) V
 *
 * computed tile by tile with online softmax over key blocks of
 * PCAST_KV_BLOCK keys.  For each query row, a running max m (including the
 * current block) and a running sum l of the un-cast probabilities are kept;
 * the probability tile P is multiplied by the static scale S, rounded to FP8
 * E4M3 (OCP e4m3fn, round to nearest even, saturating at 448) and multiplied
 * with V rounded to E4M3 on the FP8 matrix cores; the accumulator is divided
 * by S*l at the end.  Key blocks are visited 0 -> last (forward) or last -> 0
 * (reverse), the two iteration orders the P-cast summary compares
 * ("Ottimizzazione 1").  S = 0 selects the reference path with P and V in
 * bf16 instead of E4M3 (no P-cast).
 *
 * All entry points are plain C, take device pointers, never allocate memory
 * that outlives the call, never fall back to another implementation, and
 * report errors through their return code.
 */
#ifndef PCAST_ATTN_H
#define PCAST_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PCAST_ABI_VERSION 10

/* Keys per KV block.  The block size is part of the numerics (the running
 * max is updated once per block), so it is fixed. */
#define PCAST_KV_BLOCK 64

#define PCAST_ORDER_FORWARD 0
#define PCAST_ORDER_REVERSE 1

/* Return codes. */
#define PCAST_OK 0
#define PCAST_EINVAL 1  /* bad pointer, shape, scalar or alignment; nothing was enqueued */
#define PCAST_ENOTSUP 2 /* device is not gfx950, or d / N outside the supported set    */
#define PCAST_EHIP 3    /* HIP runtime or launch error; see pcast_strerror(code)        */

/*
 * attn_fwd_pcast -- enqueue one attention forward on `stream`.
 *
 * Q      device, bf16 bits, [B][Hq][N][d] row-major, contiguous, 16-byte aligned.
 * K, V   device, bf16 bits, [B][Hkv][N][d] row-major, contiguous, 16-byte aligned.
 * bias   device, float32 [N], additive logit bias per key (natural-log units),
 *        or NULL for none.  Keys with bias != 0 are "sink" keys; every other
 *        key is "non-sink" (all keys when bias is NULL).
 * B, Hq, Hkv  batch and head counts, Hq % Hkv == 0; query head h reads key/value
 *        head h / (Hq / Hkv).
 * N      sequence length (queries and keys), N >= 1.  For S > 0 any N: when
 *        N % 64 != 0 the last key block is partial and its keys past N are
 *        masked (they take no probability), query rows past N are neither
 *        stored nor counted.
 * d      head size, 64 or 128.
 * causal 0 = every key visible; 1 = key j visible to query i iff j <= i.
 * S      > 0 and finite: P-cast scale (powers of two are exact in fp32; values
 *        above 448 saturate the largest probabilities).  0: bf16 reference path.
 * order  PCAST_ORDER_FORWARD or PCAST_ORDER_REVERSE.
 * out    device, float32 [B][Hq][N][d], written completely.
 * stats  device, uint64 [pcast_stats_words(B, Hq, N)], or NULL for no
 *        counting.  For query rows [64r, 64r + 64) of (batch b, head h), word
 *        2*((b*Hq + h)*ceil(N/64) + r) receives the number of unmasked non-sink
 *        (query, key) pairs evaluated, and the next word the number of those
 *        whose E4M3 code of P*S is zero (underflow).  Words are overwritten,
 *        not accumulated.  In the bf16 path the second word counts P values
 *        that round to zero in bf16.
 * stream hipStream_t, or NULL for the default stream.
 *
 * Non-finite inputs: Q, K, V and bias must be finite.  The device code has no
 * NaN semantics for max and min, so no NaN is guaranteed to propagate: a NaN
 * or infinity in row i of Q leaves row i of out, and the two counters of its
 * 64-row block, undefined (possibly finite and wrong), and every other row and
 * block exactly as without it; a non-finite value in row j of K or V, or in
 * bias[j], leaves undefined every row that sees key j.
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer after
 * returning.  The call takes pcast_workspace_bytes() of temporary device
 * memory from HIP's stream-ordered allocator on `stream` and releases it on
 * the same stream; pcast_prepare_v + attn_fwd_pcast_prepared do the same work
 * without allocating.
 * Synchronisation: the call returns once the work is enqueued; results are
 * valid after `stream` completes.  Calls on different streams may overlap.
 * Errors: returns PCAST_OK or one of the codes above; argument errors are
 * detected before anything is enqueued; no C++ exception crosses this
 * boundary.
 */
int attn_fwd_pcast(const void* Q, const void* K, const void* V, const float* bias, int B, int Hq,
                   int Hkv, int N, int d, int causal, float S, int order, float* out,
                   unsigned long long* stats, void* stream);

/*
 * attn_fwd_pcast_noalloc -- attn_fwd_pcast for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments, kernels and results (bit for
 * bit), with the V operand copy in a scratch array of
 * PCAST_NOALLOC_SCRATCH_BYTES that the library holds on each device it runs on
 * until the process ends.  Calls no allocator.
 * Limit: pcast_workspace_bytes(B, Hkv, N, d, S) must not exceed
 * PCAST_NOALLOC_SCRATCH_BYTES (64 MiB: B * Hkv * N * d <= 2^26 for S > 0, half
 * that for S = 0), else PCAST_ENOTSUP before anything is enqueued.
 * Every call on one device shares that device's scratch: calls that overlap on
 * one device (different streams or threads without ordering between them)
 * race and give undefined results.  Calls ordered on one stream are safe.
 */
#define PCAST_NOALLOC_SCRATCH_BYTES (64u << 20)

int attn_fwd_pcast_noalloc(const void* Q, const void* K, const void* V, const float* bias, int B, int Hq,
                           int Hkv, int N, int d, int causal, float S, int order, float* out,
                           unsigned long long* stats, void* stream);

/*
 * The same forward in two stages, for callers that bring their own temporary
 * memory (and for timing the attention kernel on its own).
 *
 * pcast_prepare_v -- enqueue the copy of V that the matrix cores read: for
 * each (b, kv head, key block) a [d][64] tile of E4M3(V) (S > 0: round to
 * nearest even, saturating at +/-448) or of V itself (S = 0, bf16), with the
 * 64 keys in the order in which the attention kernel holds its probabilities
 * (a partial last block, N % 64 != 0, is padded with zeros).
 *   V          device, bf16 [B][Hkv][N][d], 16-byte aligned.
 *   workspace  device, pcast_workspace_bytes(B, Hkv, N, d, S) bytes, 16-byte
 *              aligned, owned by the caller; overwritten.
 *   B, Hkv, N, d, S as for attn_fwd_pcast (only S == 0 versus S > 0 matters).
 * Returns as attn_fwd_pcast.
 *
 * attn_fwd_pcast_prepared -- enqueue the attention kernel reading V from a
 * workspace filled by pcast_prepare_v with the same V, B, Hkv, N, d and the
 * same choice of S == 0 or S > 0 (stream order, or any other synchronisation,
 * must make the pre-pass complete first).  Other arguments, results and errors
 * as for attn_fwd_pcast.  Allocates nothing.
 */
int pcast_prepare_v(const void* V, int B, int Hkv, int N, int d, float S, void* workspace,
                    void* stream);

int attn_fwd_pcast_prepared(const void* Q, const void* K, const void* workspace, const float* bias,
                            int B, int Hq, int Hkv, int N, int d, int causal, float S, int order,
                            float* out, unsigned long long* stats, void* stream);

/*
 * attn_fwd_pcast_multi -- several configurations of the prepared forward on the same
 * Q, K and V in one grid: configuration i has its own bias[i], S[i], order[i], out[i]
 * and stats[i], and its results equal those of attn_fwd_pcast_prepared with these
 * arguments, bit for bit.  This is the shape of the P-cast summary's experiment
 * (section "Risultati Sperimentali": the same inputs under a sweep of sink
 * strengths, scales and key-block orders); one launch lets the row blocks of all
 * configurations share the chip, longest first, instead of each configuration
 * waiting for its own longest rows.
 *
 * Q, K       device, bf16, as for attn_fwd_pcast.
 * workspace  the V operand copy that pcast_prepare_v(V, B, Hkv, N, d, S > 0, ...)
 *            wrote (every S[i] must be > 0: the FP8 P.V path; S[i] = 0 gives
 *            PCAST_ENOTSUP).
 * B, Hq, Hkv, N, d, causal  as for attn_fwd_pcast, shared by all configurations.
 * n_cfg      number of configurations, >= 1.
 * bias       host array of n_cfg device pointers (float32 [N], or NULL for no bias),
 *            or NULL for no bias in any configuration.
 * S, order   host arrays of n_cfg values (S finite and > 0; order 0 or 1).
 * out        host array of n_cfg device pointers, float32 [B][Hq][N][d], 16-byte aligned.
 * stats      host array of n_cfg device pointers (uint64 [pcast_stats_words(B, Hq, N)],
 *            8-byte aligned, all non-null), or NULL for no counting.
 * The out and stats buffers of different configurations must not overlap (their
 * writes are unordered).  The host arrays are read during the call only.
 * Configurations are grouped by how
 * P is converted (S a power of two or not, S above 448 or not), at most 112 per launch.
 * Allocates nothing; errors as for attn_fwd_pcast_prepared.
 */
int attn_fwd_pcast_multi(const void* Q, const void* K, const void* workspace, int B, int Hq, int Hkv, int N, int d,
                         int causal, int n_cfg, const float* const* bias, const float* S, const int* order,
                         float* const* out, unsigned long long* const* stats, void* stream);

/*
 * attn_fwd_pcast_rows -- attn_fwd_pcast_prepared (same arguments, same out and
 * stats, bit for bit) that also writes two per-row diagnostics of the P-cast
 * (P-cast summary on gist.science, sections 1 and 2: probability mass of the
 * non-sink keys silently zeroed by the cast, and the running statistics m, l
 * of the online softmax, FlashAttention blog section "La ricorrenza softmax
 * online"):
 *   lse   device, float32 [B][Hq][N], or NULL: ln sum_j exp(s_ij) over the
 *         row's visible keys, s_ij = q.k / sqrt(d) + bias_j (natural units).
 *   lost  device, float32 [B][Hq][N], or NULL: the fraction of the row's
 *         non-sink probability mass whose E4M3 code is 0,
 *         sum_{j non-sink, code 0} p_j / sum_{j non-sink} p_j with p_j the
 *         un-cast probability (0 for a row with no non-sink key).
 * Requires S > 0 (PCAST_ENOTSUP for S = 0).  With lost requested every key
 * block takes the kernel's sequential step, so the call is slower than the
 * plain one; with lost NULL the plain pipelined kernel runs and also writes
 * lse (the same values bit for bit), at the plain call's speed.
 * Allocates nothing.
 */
int attn_fwd_pcast_rows(const void* Q, const void* K, const void* workspace, const float* bias, int B,
                        int Hq, int Hkv, int N, int d, int causal, float S, int order, float* out,
                        unsigned long long* stats, float* lse, float* lost, void* stream);

/*
 * Closed forms of the collapse model (P-cast summary on gist.science, section
 * "Metodologia e Analisi" and "Contributi Chiave" point 1), for predicting
 * from Delta, S and k whether a configuration zeroes the non-sink
 * probabilities.  Model: non-sink logits i.i.d. N(0,1), k sink keys at
 * z + Delta, forward order, so every later non-sink probability is taken
 * relative to Delta + M_k, M_k the max of k standard normals; its code is 0
 * when S * p <= 2^-10.  Host functions; NaN for S <= 0, non-finite arguments
 * or k outside 1..1024.
 *   pcast_sink_max_mean(k)             E[M_k] (1.0294 for k = 4)
 *   pcast_delta_critical(S, k)         Delta_c = 10 ln 2 + ln S - E[M_k], where the
 *                                      summary's plug-in underflow fraction is 1/2
 *   pcast_underflow_model(Delta, S, k) E[Phi(Delta + M_k - 10 ln 2 - ln S)], the
 *                                      expected fraction of non-sink codes at 0
 *   pcast_lost_mass_model(Delta, S, k) E[Phi(Delta + M_k - 10 ln 2 - ln S - 1)],
 *                                      the expected lost non-sink mass fraction
 */
double pcast_sink_max_mean(int k);
double pcast_delta_critical(double S, int k);
double pcast_underflow_model(double delta, double S, int k);
double pcast_lost_mass_model(double delta, double S, int k);

/*
 * pcast_collapse_check -- the run-time warning of the collapse model: reads a
 * host copy of an attention call's bias and reports whether forward order at
 * scale S is predicted to zero most non-sink probabilities (P-cast summary on
 * gist.science, "Contributi Chiave" point 1: collapse once the sink strength
 * exceeds Delta_c(S); "Ottimizzazione 1": reverse order defers the sink block
 * to the last step, so only the non-sink keys of that block can be zeroed).
 *   bias       host, float32 [N] (the bias passed to the attention call), or NULL.
 *   N          number of keys, >= 1.
 *   S, order   as for attn_fwd_pcast (S > 0 and finite).
 * Outputs (each may be NULL):
 *   delta      the sink strength: the largest bias value (0 if none is positive);
 *   k          the number of keys carrying it (0 without a positive bias);
 *   delta_c    pcast_delta_critical(S, k), NaN when k is 0 or above 1024;
 *   underflow  pcast_underflow_model(delta, S, k), the forward-order fraction of
 *              non-sink codes expected at zero (0 when k is 0);
 *   collapse   1 when order is forward and delta > delta_c, else 0.
 * Returns PCAST_OK, or PCAST_EINVAL for N <= 0, a bad S or order, or a
 * non-finite bias value.  Host code only; touches no device.
 */
int pcast_collapse_check(const float* bias, int N, double S, int order, double* delta, int* k,
                         double* delta_c, double* underflow, int* collapse);

/*
 * attn_bwd_pcast -- gradients of the forward by recomputation from its
 * log-sum-exp (FlashAttention blog, section "Passaggio all'indietro: ricalcolo
 * anziché archiviazione": only O and the softmax statistics are kept, the
 * probability tiles are recomputed).  The P-cast is passed straight through
 * (its derivative taken as 1): with s_ij = q_i.k_j/sqrt(d) + bias_j over the
 * visible keys, P = exp(s - lse), dP = dO V^T, D_i = dO_i . O_i,
 * dS = P (dP - D), dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d), dV = P^T dO;
 * dK and dV of a kv head sum over its Hq/Hkv query heads.
 *
 * Q, K, V  device, bf16, layouts as for attn_fwd_pcast.
 * O        device, float32 [B][Hq][N][d]: the forward's output.
 * dO       device, bf16 [B][Hq][N][d].
 * lse      device, float32 [B][Hq][N]: the forward's log-sum-exp (as written by
 *          attn_fwd_pcast_rows, natural units).
 * bias, B, Hq, Hkv, N, d, causal as for attn_fwd_pcast.
 * dQ       device, float32 [B][Hq][N][d]; dK, dV device, float32 [B][Hkv][N][d];
 *          written completely.
 * workspace  device, pcast_bwd_workspace_bytes(B, Hq, Hkv, N, d) bytes, 16-byte
 *          aligned, owned by the caller (per row, fp32 [B][Hq][N] each: -D with the row dot
 *          D = dO . O, then -lse * sqrt(d)).  Any N >= 1: with N % 64 != 0 the
 *          workspace also holds copies of Q, K, V, O, dO, lse, the bias and the
 *          gradients padded to whole 64-key blocks (zero rows; the bias of the
 *          keys past N is -inf, so they take no probability), the kernels run on
 *          those, and the gradients of the first N rows are copied out.
 * All products run on bf16 matrix cores with fp32 accumulation; P and dS are
 * rounded to bf16 where they are operands.  Allocates nothing; errors as for
 * attn_fwd_pcast, plus PCAST_ENOTSUP when one head's rows (N * d * 2 bytes,
 * N rounded up to a multiple of 64) reach 2 GiB.
 */
size_t pcast_bwd_workspace_bytes(int B, int Hq, int Hkv, int N, int d);

int attn_bwd_pcast(const void* Q, const void* K, const void* V, const float* O, const void* dO,
                   const float* lse, const float* bias, int B, int Hq, int Hkv, int N, int d, int causal,
                   float* dQ, float* dK, float* dV, void* workspace, void* stream);

/*
 * attn_decode_pcast -- decode with split KV: Nq query rows at the end of a
 * sequence of Nk keys, the keys cut into ranges of split_keys keys that each
 * run the P-cast pipeline from their own running max, merged by rescaling the
 * ranges' (m, l, A) to their common max (FlashAttention blog, section "La
 * ricorrenza softmax online"; the P-cast summary, section 1, ties the cast to
 * the running max the pipeline holds, so the split is part of the numerics:
 * a sink only raises the max of its own range).
 *
 * Q      device, bf16 [B][Hq][Nq][d]; row i is at position Nk - Nq + i and sees
 *        keys j <= Nk - Nq + i (every key when Nq = 1).
 * K      device, bf16 [B][Hkv][Nk][d].
 * vop    device, the V operand copy written by pcast_prepare_v(V, B, Hkv, Nk,
 *        d, S > 0, ...): E4M3 V, reusable across calls while V is unchanged.
 * bias   device, float32 [Nk] per-key logit bias, or NULL (sinks: bias != 0).
 * Nq     1 <= Nq <= Nk (PCAST_EINVAL otherwise) and (Hq / Hkv) * Nq <= 32
 *        (the query heads of one kv head and their rows share one 32-column
 *        MFMA tile), else PCAST_ENOTSUP.
 * Nk     any length >= Nq: with Nk % 64 != 0 the last key block is partial
 *        (its keys past Nk do not exist; the V copy and, with FP8 logits, the K
 *        codes are zero-padded).
 * split_keys  keys per range, a positive multiple of 64 (PCAST_EINVAL
 *        otherwise); the last range may be shorter.  split_keys >= Nk gives
 *        the P-cast path itself.
 * S, order, d as for attn_fwd_pcast; S must be > 0 (PCAST_ENOTSUP for 0).
 * out    device, float32 [B][Hq][Nq][d].
 * stats  device, uint64 [pcast_stats_words(B, Hq, Nq)] or NULL: per (b, h)
 *        the non-sink (query, key) pairs of its Nq rows and those with code 0.
 * workspace  device, pcast_decode_workspace_bytes(B, Hkv, Nk, d, split_keys)
 *        bytes, 16-byte aligned, owned by the caller: the ranges' partial
 *        results.  Allocates nothing.
 * Two kernels run on `stream`: one wave per (b, kv head, range), then one
 * workgroup per (b, kv head) for the merge.
 */
size_t pcast_decode_workspace_bytes(int B, int Hkv, int Nk, int d, int split_keys);

int attn_decode_pcast(const void* Q, const void* K, const void* vop, const float* bias, int B, int Hq,
                      int Hkv, int Nq, int Nk, int d, float S, int order, int split_keys, float* out,
                      unsigned long long* stats, void* workspace, void* stream);

/*
 * The forward with FP8 logits: Q and K rounded to E4M3 as well, so that Q K^T
 * runs on the FP8 matrix cores too (FlashAttention blog by marketmaker.cc,
 * section "FA3: Meccanica della tramoggia", item 3: FP8 attention inputs
 * quantised block by block, one scale per block; the P-cast summary on
 * gist.science, closing remarks, names Q/K/V quantisation as the noise that
 * may outweigh the P-cast gain).  This path has no random rotation.
 *
 * Blocks: each query row of Q, and each 64-key block of each head of K.  The
 * scale of a block is the smallest power of two 2^e with max|x| <= 448 * 2^e
 * over the block; the codes are E4M3(x * 2^-e) (round to nearest even; the
 * choice of e keeps them in range, so none saturates).  The logit of (i, j)
 * is the fp32 accumulation of the code products times 2^(e_i + e_block(j)) /
 * sqrt(d), which is exact, so the logits are those of the rounded Q and K up
 * to the matrix cores' accumulation.  Softmax, P-cast, V and the epilogue are
 * as in attn_fwd_pcast.  Inputs must be finite.
 *
 * pcast_workspace_bytes_qk8 -- bytes of the workspace: the V operand copy, the
 * codes of K and the exponents of the key blocks, 256-byte aligned each.
 *
 * pcast_prepare_qk8 -- enqueue the pre-pass that fills that workspace from K
 * and V (bf16 [B][Hkv][N][d], 16-byte aligned), one key block per workgroup.
 * The workspace (16-byte aligned, owned by the caller) is overwritten.  Q
 * needs no pre-pass: the attention kernel rounds each row as it loads it.
 *
 * attn_fwd_pcast_qk8_prepared -- enqueue the attention kernel reading Q (bf16,
 * as for attn_fwd_pcast) and a workspace that pcast_prepare_qk8 filled with
 * the same B, Hkv, N, d (stream order, or other synchronisation, must
 * complete the pre-pass first).  Allocates nothing.
 *
 * attn_fwd_pcast_qk8 -- both, with a workspace from HIP's stream-ordered
 * allocator on `stream`, released on the same stream.
 *
 * Arguments, results and errors as for attn_fwd_pcast, and further: S must be
 * > 0 (PCAST_ENOTSUP for S = 0, which has no FP8 P.V).
 */
size_t pcast_workspace_bytes_qk8(int B, int Hkv, int N, int d);

int pcast_prepare_qk8(const void* K, const void* V, int B, int Hkv, int N, int d, void* workspace,
                      void* stream);

int attn_fwd_pcast_qk8_prepared(const void* Q, const void* workspace, const float* bias, int B, int Hq,
                                int Hkv, int N, int d, int causal, float S, int order, float* out,
                                unsigned long long* stats, void* stream);

int attn_fwd_pcast_qk8(const void* Q, const void* K, const void* V, const float* bias, int B, int Hq,
                       int Hkv, int N, int d, int causal, float S, int order, float* out,
                       unsigned long long* stats, void* stream);

/*
 * attn_decode_pcast_qk8 -- the split-KV decode of attn_decode_pcast with FP8
 * logits, as the forward above: each query row of Q rounded to E4M3 with its
 * own power-of-two scale inside the kernel, K read as the E4M3 codes and
 * per-64-key-block exponents of a workspace that pcast_prepare_qk8(K, V, B,
 * Hkv, Nk, d, ...) filled (its V operand copy serves the P.V product), so a
 * decode step reads one byte per element of K instead of two.
 *
 * qk8_workspace  device, pcast_workspace_bytes_qk8(B, Hkv, Nk, d) bytes,
 *        16-byte aligned, filled by pcast_prepare_qk8 with the same B, Hkv,
 *        Nk, d (stream order, or other synchronisation, must complete it first).
 * Every other argument, the results and the errors as for attn_decode_pcast.
 * Allocates nothing.
 */
int attn_decode_pcast_qk8(const void* Q, const void* qk8_workspace, const float* bias, int B, int Hq, int Hkv,
                          int Nq, int Nk, int d, float S, int order, int split_keys, float* out,
                          unsigned long long* stats, void* workspace, void* stream);

/*
 * The FP8-logit forward with a random rotation of Q and K before the rounding
 * (FlashAttention blog, section "FA3: Meccanica della tramoggia", item 3: the
 * vectors are rotated at random before the block quantisation so that an
 * outlier's magnitude spreads over all coordinates).  Each row x of Q and K
 * becomes x diag(sigma) H, H the d x d Sylvester Hadamard matrix of +-1 and
 * sigma the caller's signs; since H H^T = d I the logits are those of the
 * unrotated inputs times d, which the kernel divides out exactly.  The rotation
 * is computed in fp64 (exact for bf16 inputs) and rounded to E4M3 with one
 * power-of-two scale per query row and per 64-key block, as in
 * attn_fwd_pcast_qk8.
 *
 * pcast_workspace_bytes_qk8_rot -- bytes of the workspace: that of the
 * unrotated variant plus the codes of Q and one exponent per query row.  Any N:
 * K's codes take whole 64-key blocks (a zero row for each key past N, so a
 * partial block's exponent is that of the keys that exist), Q's take N rows.
 * pcast_prepare_qk8_rot -- enqueue the V copy and the rotation pre-passes of K
 * and Q.  signs: device, int8 [d], 16-byte aligned, the signs sigma (a negative
 * entry is -1, any other +1; the caller draws them).  Other arguments as for
 * pcast_prepare_qk8, plus Q and Hq.
 * attn_fwd_pcast_qk8_rot_prepared -- the attention kernel on that workspace;
 * arguments and errors as for attn_fwd_pcast_qk8_prepared (no Q: its codes are
 * in the workspace).  Allocates nothing.
 */
size_t pcast_workspace_bytes_qk8_rot(int B, int Hq, int Hkv, int N, int d);

int pcast_prepare_qk8_rot(const void* Q, const void* K, const void* V, const signed char* signs, int B, int Hq,
                          int Hkv, int N, int d, void* workspace, void* stream);

int attn_fwd_pcast_qk8_rot_prepared(const void* workspace, const float* bias, int B, int Hq, int Hkv, int N, int d,
                                    int causal, float S, int order, float* out, unsigned long long* stats,
                                    void* stream);

/*
 * pcast_cast_e4m3 -- enqueue the P-cast conversion alone: codes[i] = the E4M3
 * code (OCP e4m3fn) of S * P[i], computed by the same device code that every
 * attention kernel above applies to its probability tile (P-cast summary on
 * gist.science, section "Ottimizzazione 2": for S = 2^k the product is formed
 * inside the conversion and is exact, so the code is that of the exact S*P
 * rounded to nearest even; for any other S the product is rounded to fp32
 * first and then converted; above 448 every code saturates at 448, 0x7E).  It
 * lets a caller check the kernels' rounding bit for bit.
 *
 * P      device, float32 [n], 16-byte aligned: probabilities in [0, 1] (the
 *        kernels convert nothing else; codes of other values are unspecified).
 * codes  device, uint8 [n], 4-byte aligned, overwritten.
 * n      a non-negative multiple of 4 (PCAST_EINVAL otherwise).
 * S      finite and > 0 (PCAST_EINVAL otherwise).
 * Allocates nothing; errors as for attn_fwd_pcast.
 */
int pcast_cast_e4m3(const float* P, unsigned char* codes, long long n, float S, void* stream);

/* Number of uint64 words the stats buffer needs: B * Hq * ceil(N / 64) * 2. */
size_t pcast_stats_words(int B, int Hq, int N);

/* Bytes of the V operand copy: B * Hkv * (N rounded up to a multiple of 64) * d
 * for S > 0, twice that for S = 0. */
size_t pcast_workspace_bytes(int B, int Hkv, int N, int d, float S);

/* Human-readable text for a return code, with the detail of the last error
 * raised on the calling thread when there is one. */
const char* pcast_strerror(int code);

/* PCAST_ABI_VERSION of the built library. */
int pcast_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PCAST_ATTN_H */
