/*
 * spec_verify.h -- C ABI of the speculative-decoding verify library (HIP, gfx950).
 *
 * The library implements the verify step of speculative decoding:
 *   - spec_verify_sample: rejection-sampling verify of K draft tokens per row.
 *     p_i = softmax(target_i / T), q_i = softmax(draft_i / T), both computed in
 *     fp32; draft token x_i is accepted iff r_i < min(1, p_i(x_i) / q_i(x_i));
 *     the walk stops at the first rejection n, where a replacement token is
 *     drawn from norm(max(0, p_n - q_n)); if all K are accepted, a bonus token
 *     is drawn from p_K (target row K).
 *     Sources: "Speculative Decoding —— LLM推理优化技术（一）", §2.1 (acceptance
 *     probability, residual law), §2.3 (multi-token rule, bonus token), §4 (the
 *     temperature divides the logits; zero residual mass falls back to p);
 *     kwkr.cn/news/620797 engineering notes, §3.1 (accept iff r < alpha, reject
 *     iff r >= alpha; bonus from the target's last position), §3.2 (fp32
 *     probabilities; truncate alpha to 1 when p >= q), §3.4 (the same
 *     temperature on both sides).
 *   - spec_verify_greedy: greedy (temperature 0) verify of G disjoint candidate
 *     n-grams: the longest prefix matching the target's per-position argmax
 *     wins and is followed by the argmax after it.
 *     Source: "Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池,不靠草稿模型的
 *     投机解码", section "验证分支:输出分布不变性", and eq. (1) (greedy decoding is
 *     the per-position argmax).
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, row-major and
 *     contiguous, aligned to their element size. The library never allocates
 *     device memory and keeps no state between calls.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and never synchronise the host.
 *   - Every argument error is detected on the host and returned as a negative
 *     status BEFORE any HIP call; outputs are then untouched. A launch failure
 *     returns SPEC_ERR_HIP.
 *   - Data faults found on the device are reported per row in the outputs
 *     (see each function), never by the status.
 *   - Outputs must not overlap inputs or each other.
 *   - The workspace carries partial results from one launch of a call to the
 *     next launch of the same call. It needs no initialisation and keeps
 *     nothing between calls. Calls that run at the same time must use
 *     different workspaces; calls in one stream may share one.
 *   - Logits are finite or -inf. A +inf or NaN logit gives unspecified values
 *     for its row (never an out-of-bounds access).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPEC_ABI_VERSION 1
#define SPEC_MAX_K 64        /* draft positions per row; the first-reject scan is one 64-lane ballot */
#define SPEC_MAX_V (1 << 30) /* vocabulary entries per row */
#define SPEC_MAX_ROWS (1 << 24) /* logit rows per call */

typedef enum { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

typedef enum {
  SPEC_OK = 0,
  SPEC_ERR_NULL = -1,        /* a required pointer is NULL */
  SPEC_ERR_SHAPE = -2,       /* a size is out of range */
  SPEC_ERR_TEMPERATURE = -3, /* temperature not finite or not > 0 */
  SPEC_ERR_DTYPE = -4,       /* unknown spec_dtype */
  SPEC_ERR_WORKSPACE = -5,   /* workspace smaller than the *_workspace_size query */
  SPEC_ERR_HIP = -6,         /* a HIP launch failed */
  SPEC_ERR_ALIGN = -7,       /* a pointer is not aligned to its element size */
  SPEC_ERR_PHASE = -8,       /* phase mask outside 1..15 (spec_verify_sample_phases) */
  SPEC_ERR_FILTER_V = -9,    /* V > SPEC_MAX_FILTER_V (spec_verify_sample_filtered) */
  SPEC_ERR_STAGES = -10,     /* invalid stage schedule (spec_verify_sample_staged) */
  SPEC_ERR_POOL = -11        /* pool buffer smaller than spec_ngram_pool_bytes / spec_ngram_cache_bytes */
} spec_status;

#define SPEC_MAX_FILTER_V (1 << 24) /* vocabulary entries per row of the filtered verify */
#define SPEC_MAX_STAGES 8           /* pass-1 stages of spec_verify_sample_staged */
#define SPEC_MAX_POOL_G 64          /* continuations a pool key holds */
#define SPEC_MAX_POOL_N 17          /* n-gram length: a continuation holds at most 16 tokens */
#define SPEC_MAX_POOL_W 64          /* n-grams per sequence in one insert call */
#define SPEC_MAX_CACHE_SETS (1 << 24) /* sets per sequence of the hashed pool (a power of two) */
#define SPEC_MAX_CACHE_WAYS 64        /* keys a set of the hashed pool holds */
#define SPEC_MAX_NGRAM_SAMPLE_V (1 << 20) /* vocabulary entries of spec_verify_ngram_sample */
#define SPEC_MAX_NGRAM_SAMPLE_GN 1024    /* G*N of spec_verify_ngram_sample: one sequence's inputs staged on chip */

/* Bytes of workspace spec_verify_sample needs for these sizes (0 for invalid sizes). */
size_t spec_verify_sample_workspace_size(int32_t B, int32_t K, int32_t V);

/*
 * Rejection-sampling verify of B independent rows.
 *
 * target_logits    [B, K+1, V] dtype. Row i (< K) is the target distribution for
 *                  draft token i (already aligned by the caller: the logits
 *                  that PREDICT x_i); row K is the bonus row.
 * draft_logits     [B, K, V] dtype. Row i is the draft distribution x_i was drawn from.
 * dtype            SPEC_F32 or SPEC_BF16, shared by both logits tensors.
 * draft_tokens     [B, K] int32.
 * uniforms         [B, K+1, 2] float, each in [0, 1): [b,i,0] = accept uniform
 *                  r_i (read for i < K); [b,i,1] = draw uniform u_i (the
 *                  resample at i < K, the bonus draw at i = K).
 * B, K, V          0 <= B, 0 <= K <= SPEC_MAX_K, 1 <= V <= SPEC_MAX_V,
 *                  B*(2K+1) <= SPEC_MAX_ROWS. B = 0 is a no-op. K = 0 draws one
 *                  token from the bonus row.
 * temperature      finite, > 0; logits are divided by it on both sides.
 * out_tokens       [B, K+1] int32: x_0..x_{n-1}, then the drawn token at n, then -1.
 * out_num_accepted [B] int32: n in [0, K], or -1 for a data fault.
 * out_probs        NULL or [B, K, 2] float: p_i(x_i), q_i(x_i) in fp32 for every
 *                  i < K (NaN where x_i is out of range; p_i (q_i) is NaN when target
 *                  (draft) row i has no finite logit).
 * workspace        device memory of at least spec_verify_sample_workspace_size bytes.
 *
 * Draw rule: token = the smallest k with sum_{v<=k} w_v > u * sum_v w_v, where w
 * is max(0, p_n - q_n) (or p_K for the bonus draw); if the residual mass is 0,
 * w = p_n.
 * Data faults (reported as out_num_accepted[b] = -1 and out_tokens[b,:] = -1):
 * walking i = 0, 1, ...: x_i outside [0, V), or target row i or draft row i with
 * no finite logit, at a position the walk reaches; or all K accepted and the
 * bonus row has no finite logit.
 */
spec_status spec_verify_sample(const void* target_logits, const void* draft_logits, int32_t dtype,
                               const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                               int32_t V, float temperature, int32_t* out_tokens,
                               int32_t* out_num_accepted, float* out_probs, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Bytes of workspace spec_row_stats needs for these sizes (0 for invalid sizes). */
size_t spec_row_stats_workspace_size(int32_t rows, int32_t V);

/*
 * Softmax statistics of logit rows, as the verify computes them for p and q
 * ("Speculative Decoding —— LLM推理优化技术（一）" §2.1: p and q are softmaxes of
 * whole rows; §4: the temperature divides the logits; kwkr.cn notes §3.2: fp32
 * probabilities). With c = fl32(log2(e) / temperature) and R = fl32(m * c):
 *   out_max[r] = m, the row's largest logit (-inf when none is finite);
 *   out_sum[r] = S = sum_v 2^(fl32(x_v * c - R)), accumulated as the verify does
 *                (fp32 per thread, fp64 across threads and segments);
 * so the row's law is p_v = 2^(x_v * c - R) / S. The same streaming reduction as
 * the verify's pass 1; a caller (or a test) can rebuild every probability of a
 * row from these two numbers.
 *
 * logits     [rows, V] dtype (device), row-major, aligned to its element size.
 * rows, V    0 <= rows <= SPEC_MAX_ROWS, 1 <= V <= SPEC_MAX_V; rows = 0 is a no-op.
 * out_max    [rows] float (device); out_sum [rows] double (device, 8-byte aligned).
 * workspace  at least spec_row_stats_workspace_size(rows, V) bytes; needs no
 *            initialisation.
 * Errors as spec_verify_sample (shape, dtype, temperature, NULL, alignment,
 * workspace), all before any HIP call.
 */
spec_status spec_row_stats(const void* logits, int32_t dtype, int32_t rows, int32_t V, float temperature,
                           float* out_max, double* out_sum, void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_sample for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 *
 * Arguments and outputs as spec_verify_sample, without the workspace: the call
 * uses a fixed device array of SPEC_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends, and allocates nothing (no
 * hipMalloc, no allocating library routine). The array's device address is
 * looked up once per device, on the first call with that device current.
 * Sizes whose spec_verify_sample_workspace_size exceeds
 * SPEC_NOALLOC_SCRATCH_BYTES return SPEC_ERR_WORKSPACE (before any HIP call);
 * every argument error is found before any HIP call as well. A failed lookup of
 * the array returns SPEC_ERR_HIP. Every call on one GPU shares that GPU's array:
 * calls that may overlap on one GPU (different streams without ordering between
 * them) race and give unspecified outputs. The array needs no clearing between
 * calls (the kernels keep nothing in it from one call to the next).
 */
#define SPEC_NOALLOC_SCRATCH_BYTES (4u << 20)
size_t spec_verify_sample_noalloc_max_bytes(void); /* SPEC_NOALLOC_SCRATCH_BYTES */
spec_status spec_verify_sample_noalloc(const void* target_logits, const void* draft_logits, int32_t dtype,
                                       const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                                       int32_t V, float temperature, int32_t* out_tokens,
                                       int32_t* out_num_accepted, float* out_probs, void* stream);

/*
 * spec_verify_sample as its four launches, for callers that schedule or time
 * them apart. Same arguments as spec_verify_sample plus a mask of phases,
 * which run in this order on `stream` (a call with every bit set is
 * spec_verify_sample):
 *   SPEC_PHASE_ROW_STATS  pass 1: reads target rows 0..K-1 and draft rows 0..K-1
 *                         once; leaves per-segment max / sum-exp in the workspace.
 *   SPEC_PHASE_ACCEPT     accept tests and the first rejection: writes
 *                         out_num_accepted, out_probs and every out_tokens entry
 *                         except the drawn one.
 *   SPEC_PHASE_MASS       pass 2: reads only the row(s) the draw needs (target and
 *                         draft row n after a rejection, or the bonus row).
 *   SPEC_PHASE_DRAW       the inverse-CDF search; writes the drawn token (and the
 *                         fault outputs of a bonus row with no finite logit).
 * A phase reads what the earlier phases of the same arguments left in the
 * workspace; running it without them gives unspecified outputs but never an
 * access outside the arguments' buffers. SPEC_ERR_PHASE for a mask outside 1..15.
 */
#define SPEC_PHASE_ROW_STATS 1
#define SPEC_PHASE_ACCEPT 2
#define SPEC_PHASE_MASS 4
#define SPEC_PHASE_DRAW 8
spec_status spec_verify_sample_phases(const void* target_logits, const void* draft_logits, int32_t dtype,
                                      const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                                      int32_t V, float temperature, int32_t* out_tokens,
                                      int32_t* out_num_accepted, float* out_probs, void* workspace,
                                      size_t workspace_bytes, void* stream, int32_t phases);

/*
 * spec_verify_sample with early exit: the draft positions are read in stages, and
 * a stage reads the rows of a batch row only if every earlier position was
 * accepted. The walk stops at the first rejection, so the rows past it are never
 * needed ("Speculative Decoding —— LLM推理优化技术（一）" §2.3: the first rejected
 * draft ends the round). The stages cost one launch each; a workload whose drafts
 * are often rejected early reads fewer bytes, one that accepts most drafts pays
 * the extra launches.
 *
 * Arguments, workspace (spec_verify_sample_workspace_size) and outputs as
 * spec_verify_sample, plus:
 * stage_ends   HOST array of num_stages draft positions, strictly increasing, in
 *              [1, K], the last equal to K: stage s reads positions
 *              [stage_ends[s-1], stage_ends[s]) (from 0 for s = 0). With K = 0,
 *              num_stages is 0 and stage_ends may be NULL. Otherwise
 *              1 <= num_stages <= SPEC_MAX_STAGES. SPEC_ERR_STAGES for any other schedule.
 * Every output equals spec_verify_sample's, except that with more than one stage
 * out_probs[b, i] is NaN for positions i past the first rejection n (not every
 * such row is read).
 */
spec_status spec_verify_sample_staged(const void* target_logits, const void* draft_logits, int32_t dtype,
                                      const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                                      int32_t V, float temperature, int32_t* out_tokens,
                                      int32_t* out_num_accepted, float* out_probs, void* workspace,
                                      size_t workspace_bytes, void* stream, const int32_t* stage_ends,
                                      int32_t num_stages);

/* Bytes of workspace spec_verify_sample_filtered needs for these sizes (0 for invalid sizes). */
size_t spec_verify_sample_filtered_workspace_size(int32_t B, int32_t K, int32_t V);

/*
 * Rejection-sampling verify on top-k / top-p filtered laws.
 * Source: kwkr.cn/news/620797 engineering notes, §3.4: the temperature is
 * applied to both sides before p and q are formed; a top-k or top-p truncation
 * must use the same parameter on the draft and the target side, and the
 * correction is drawn only inside the truncated set.
 *
 * Arguments as spec_verify_sample, plus:
 * top_k     NULL or [B] int32 device array: the k of batch row b, applied to its
 *           target rows 0..K and draft rows 0..K-1 alike. A row keeps every
 *           entry that has fewer than k entries with a strictly larger logit (all
 *           ties of the k-th largest logit stay). k <= 0 or k >= V: no top-k.
 * top_p     NULL or [B] float device array: then, on the law left by top-k and
 *           renormalised, a row keeps an entry when the kept entries with a
 *           strictly larger logit hold mass < p, and always keeps the entries of
 *           its largest logit (so p <= 0 keeps only those). p >= 1 or NaN: no top-p.
 * out_kept  NULL or [B, 2K+1] int32: the number of entries each row keeps, target
 *           rows 0..K first, then draft rows 0..K-1 (0 for a row with no finite logit).
 * V         at most SPEC_MAX_FILTER_V (SPEC_ERR_FILTER_V otherwise): kept masses
 *           are summed exactly in 64-bit fixed point, 2^-40 per unit of mass.
 * The verify then runs on p' and q', the kept probabilities renormalised: a draft
 * token outside its draft row's kept set has q' = 0 (accepted when p' > 0); the
 * residual max(0, p'_n - q'_n), its zero-mass fallback p'_n and the bonus law p'_K
 * all lie inside the target row's kept set. out_probs holds p'_i(x_i), q'_i(x_i).
 * Unlike spec_verify_sample, every row is read, the bonus row too, and normally
 * once. With 0 < k <= 64 the entries above a running bound are collected on chip
 * and both cuts are taken from them. With top-p alone or k > 64 the first step of
 * the read sets a bound meant to lie below the cut; the entries above it are kept
 * on chip (long bf16 rows with top-p alone: a count per bf16 value instead) and the
 * mass below it is summed, and the cut is taken there when they provably hold it.
 * A long fp32 row with top-p alone whose kept set outgrows the on-chip buffer (a flat
 * row) is read twice: counts in bins of mass bound the cut to a band of values, then
 * the second read sums every entry's exact mass and keeps the band's entries.
 * A row none of these finishes (the kept entries overflow, or do not hold the
 * cut) takes an exact radix select, which reads the row once for its maximum and
 * once per radix digit of each active filter (bf16: 2 digits, fp32: 3). Results
 * do not depend on which path a row took.
 */
spec_status spec_verify_sample_filtered(const void* target_logits, const void* draft_logits, int32_t dtype,
                                        const int32_t* draft_tokens, const float* uniforms, int32_t B, int32_t K,
                                        int32_t V, float temperature, int32_t* out_tokens,
                                        int32_t* out_num_accepted, float* out_probs, void* workspace,
                                        size_t workspace_bytes, void* stream, const int32_t* top_k,
                                        const float* top_p, int32_t* out_kept);

/*
 * spec_verify_sample_filtered as its phases (the bits of spec_verify_sample_phases,
 * run in order); SPEC_PHASE_ROW_STATS is the filter pass over all 2K+1 rows of
 * every batch row.
 */
spec_status spec_verify_sample_filtered_phases(const void* target_logits, const void* draft_logits, int32_t dtype,
                                               const int32_t* draft_tokens, const float* uniforms, int32_t B,
                                               int32_t K, int32_t V, float temperature, int32_t* out_tokens,
                                               int32_t* out_num_accepted, float* out_probs, void* workspace,
                                               size_t workspace_bytes, void* stream, const int32_t* top_k,
                                               const float* top_p, int32_t* out_kept, int32_t phases);

/* Bytes of workspace spec_verify_greedy needs for these sizes (0 for invalid sizes). */
size_t spec_verify_greedy_workspace_size(int32_t B, int32_t G, int32_t N, int32_t V);

/*
 * Greedy verify of G disjoint candidates per row (temperature 0 only: argmax
 * matching under sampling would change the output law, kwkr.cn notes §2).
 *
 * target_logits  [B, G, N, V] dtype. Row i of candidate g holds the target's
 *                logits after the prefix cand[b,g,0..i-1]; row N-1 is the bonus row.
 * cand_tokens    [B, G, N-1] int32: the candidate n-gram's tokens after the
 *                (already matched) first token.
 * B, G, N, V     0 <= B, 1 <= G, 2 <= N <= SPEC_MAX_K + 1, G*N <= 8192,
 *                1 <= V <= SPEC_MAX_V, B*G*N <= SPEC_MAX_ROWS.
 * out_tokens     [B, N] int32: cand[b,best,0..L-1], then argmax of row L of
 *                candidate best, then -1.
 * out_accept_len [B] int32: L in [0, N-1], or -1 for a data fault.
 * out_best_cand  [B] int32: the winning candidate, or -1 for a data fault.
 * Argmax ties go to the lowest vocabulary index; prefix-length ties to the
 * lowest candidate index. Data faults: a candidate token outside [0, V), or a
 * row with no finite logit (out_tokens[b,:] = -1).
 */
spec_status spec_verify_greedy(const void* target_logits, int32_t dtype, const int32_t* cand_tokens,
                               int32_t B, int32_t G, int32_t N, int32_t V, int32_t* out_tokens,
                               int32_t* out_accept_len, int32_t* out_best_cand, void* workspace,
                               size_t workspace_bytes, void* stream);

/* Bytes of workspace spec_verify_ngram_sample needs for these sizes (0 for invalid sizes). */
size_t spec_verify_ngram_sample_workspace_size(int32_t B, int32_t G, int32_t N, int32_t V);

/*
 * Sampling verify (temperature > 0) of G greedy-drafted candidate n-grams.
 * Source: "Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池,不靠草稿模型的投机解码",
 * section "采样模式的验证" (the lookahead branch drafts greedily, so a candidate
 * token's draft law is one-hot; the verify still samples in full), and
 * "Speculative Decoding —— LLM推理优化技术（一）" §2.1 (with q = delta_x a token is
 * accepted with probability p(x) and a rejection removes it from the law).
 *
 * target_logits  [B, G, N, V] dtype: row i of candidate g is the target's law
 *                after the candidate's first i tokens; row N-1 the bonus row.
 * cand_tokens    [B, G, N-1] int32.
 * uniforms       [B, N, G+1] float in [0, 1): [b,i,h] accepts candidate h at
 *                position i; [b,i,G] is the draw uniform of position i.
 * B, G, N, V     0 <= B, 1 <= G <= 64, 2 <= N <= SPEC_MAX_K + 1,
 *                G*N <= SPEC_MAX_NGRAM_SAMPLE_GN, 1 <= V <= SPEC_MAX_NGRAM_SAMPLE_V,
 *                B*G*N <= SPEC_MAX_ROWS.
 * temperature    finite, > 0; p = softmax(logits / T) in fp32.
 * out_tokens     [B, N] int32: the accepted tokens, then the drawn token, then -1.
 * out_accept_len [B] int32: L in [0, N-1], or -1 for a data fault.
 * out_rows       [B] int32: the candidate whose rows the final draw read (-1 on a fault).
 *
 * The walk: at position i the active candidates (those whose first i tokens are
 * the tokens accepted so far; all of them at i = 0) are tried in index order on
 * p_cur, the law of the lowest active candidate's row i with the tokens rejected
 * so far at i removed and renormalised: candidate h's token x is accepted iff
 * uniforms[b,i,h] < p_cur(x). An acceptance keeps the candidates whose token at i
 * is x and moves to i + 1; after N-1 acceptances a bonus token is drawn from row
 * N-1 of the lowest active candidate. When every try at i fails, the token is
 * drawn from p_cur (the rule of spec_verify_sample; zero remaining mass falls
 * back to p). Data faults: a candidate token outside [0, V), or a consulted row
 * with no finite logit.
 */
spec_status spec_verify_ngram_sample(const void* target_logits, int32_t dtype, const int32_t* cand_tokens,
                                     const float* uniforms, int32_t B, int32_t G, int32_t N, int32_t V,
                                     float temperature, int32_t* out_tokens, int32_t* out_accept_len,
                                     int32_t* out_rows, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The n-gram pool that supplies spec_verify_greedy's candidates.
 * Source: "Lookahead Decoding 完全拆解:Jacobi 迭代与 N-gram 池,不靠草稿模型的投机解码",
 * sections "Lookahead 分支" (each step yields W n-grams of length N for the pool),
 * "N-gram 池与身份判定" (only n-grams whose first token equals the last generated
 * token are verified) and "验证分支" (n-grams not adopted stay in the pool).
 *
 * One pool per sequence (batch row), keyed by an n-gram's first token. A key
 * holds its G most recently inserted distinct continuations (the N-1 tokens after
 * the first), newest first; inserting a continuation the key holds makes it the
 * newest; when a key is full its oldest continuation is dropped.
 *
 * pool         DEVICE memory of at least spec_ngram_pool_bytes(B, V, G, N) bytes,
 *              16-byte aligned, owned by the caller: [B][V][G][N-1] int32, a
 *              key's slots newest first, an empty slot -1 in every token.
 *              spec_ngram_pool_init must run on it once before any other use.
 * B, V, G, N   0 <= B, 1 <= V <= SPEC_MAX_V, 1 <= G <= SPEC_MAX_POOL_G,
 *              2 <= N <= SPEC_MAX_POOL_N; the pool size must fit in size_t.
 * SPEC_ERR_POOL when pool_bytes is smaller than spec_ngram_pool_bytes.
 */
size_t spec_ngram_pool_bytes(int32_t B, int32_t V, int32_t G, int32_t N);  /* 0 for invalid sizes */
spec_status spec_ngram_pool_init(void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G, int32_t N,
                                 void* stream);
/*
 * Insert W n-grams per sequence: ngrams [B, W, N] int32 (device), sequence b's
 * n-grams in window order (index 0 first), 0 <= W <= SPEC_MAX_POOL_W. An n-gram
 * with any token outside [0, V) is skipped; out_skipped (NULL or [B] int32)
 * receives the number skipped per sequence.
 */
spec_status spec_ngram_pool_insert(void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G, int32_t N,
                                   const int32_t* ngrams, int32_t W, int32_t* out_skipped, void* stream);
/*
 * The candidates for each sequence's last generated token: last_tokens [B]
 * int32; out_cand [B, G, N-1] int32 receives the key's continuations newest
 * first and -1 in the slots past out_count [B] (0 for a token outside [0, V)).
 * The pool is read only. The first out_count[b] rows of out_cand[b] are the
 * candidate tokens spec_verify_greedy takes after the matched first token.
 */
spec_status spec_ngram_pool_lookup(const void* pool, size_t pool_bytes, int32_t B, int32_t V, int32_t G, int32_t N,
                                   const int32_t* last_tokens, int32_t* out_cand, int32_t* out_count, void* stream);

/*
 * The hashed n-gram pool: the same pool as spec_ngram_pool_*, held in a bounded
 * table whose size follows its capacity instead of B*V. Source: as above (the
 * Lookahead Decoding page, sections "Lookahead 分支", "N-gram 池与身份判定" and
 * "验证分支"); the page leaves the pool's capacity open, so this bound is a reading.
 *
 * Per sequence, `sets` sets of `ways` keys. A key's home set is the top log2(sets)
 * bits of (key * 2654435769) mod 2^32 (Knuth's multiplicative hashing with
 * floor(2^32 / golden ratio)). Every inserted n-gram takes the next value of its
 * sequence's 32-bit clock (skipped ones take none) and a key's stamp is its newest
 * n-gram's value. A new key in a full set evicts the key with the oldest stamp,
 * continuations and all (ages modulo 2^32: exact while every held key was inserted
 * within the sequence's last 2^32 insertions); a key that comes back starts empty.
 * Within a key the direct pool's rule holds: its G most recently inserted distinct
 * continuations, newest first. While no set overflows, inserts and lookups give
 * exactly what the direct pool gives. Lookups change nothing.
 *
 * cache        DEVICE memory of at least spec_ngram_cache_bytes(B, sets, ways, G, N)
 *              bytes, 16-byte aligned, owned by the caller. Per sequence:
 *              seq = 4 + sets * (2*ways + ways*G*(N-1)) int32 rounded up to a
 *              multiple of 4; word 0 the clock, words 1..3 zero; then set s at word
 *              4 + s*(2*ways + ways*G*(N-1)): keys[ways] int32 (-1: empty),
 *              stamps[ways] uint32, slots[ways][G][N-1] int32 (newest first, an
 *              empty slot -1 throughout). spec_ngram_cache_init must run on it once
 *              before any other use, and every call passes the same sizes.
 * B, sets, ways, G, N   0 <= B, 1 <= sets <= SPEC_MAX_CACHE_SETS (a power of two),
 *              1 <= ways <= SPEC_MAX_CACHE_WAYS, 1 <= G <= SPEC_MAX_POOL_G,
 *              2 <= N <= SPEC_MAX_POOL_N; the table must fit in size_t.
 * V            1 <= V <= SPEC_MAX_V: tokens outside [0, V) are skipped (insert) or
 *              have no continuation (lookup).
 * SPEC_ERR_POOL when cache_bytes is smaller than spec_ngram_cache_bytes.
 */
size_t spec_ngram_cache_bytes(int32_t B, int32_t sets, int32_t ways, int32_t G, int32_t N); /* 0: invalid sizes */
spec_status spec_ngram_cache_init(void* cache, size_t cache_bytes, int32_t B, int32_t sets, int32_t ways, int32_t G,
                                  int32_t N, void* stream);
/* As spec_ngram_pool_insert: ngrams [B, W, N] int32 (device) in window order,
 * 0 <= W <= SPEC_MAX_POOL_W; out_skipped NULL or [B] int32. */
spec_status spec_ngram_cache_insert(void* cache, size_t cache_bytes, int32_t B, int32_t V, int32_t sets, int32_t ways,
                                    int32_t G, int32_t N, const int32_t* ngrams, int32_t W, int32_t* out_skipped,
                                    void* stream);
/* As spec_ngram_pool_lookup: last_tokens [B] int32; out_cand [B, G, N-1] int32 (newest
 * first, -1 past out_count [B]). The table is read only. */
spec_status spec_ngram_cache_lookup(const void* cache, size_t cache_bytes, int32_t B, int32_t V, int32_t sets,
                                    int32_t ways, int32_t G, int32_t N, const int32_t* last_tokens, int32_t* out_cand,
                                    int32_t* out_count, void* stream);

/*
 * Fill out [B, K+1, 2] with the verify uniforms of one round from
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
 * as 1, 2, 3", SC'11). Counter for (b, i) = (i, b, round lo32, round hi32);
 * key = (seed lo32, seed hi32); output word 0 -> [b,i,0], word 1 -> [b,i,1],
 * each mapped as (w >> 8) * 2^-24.
 * 0 <= B, 0 <= K <= SPEC_MAX_K, B*(K+1) <= SPEC_MAX_ROWS.
 */
spec_status spec_fill_uniforms(uint64_t seed, uint64_t round, int32_t B, int32_t K, float* out, void* stream);

/* Static description of a status code; never NULL. */
const char* spec_status_string(int32_t status);

/* SPEC_ABI_VERSION of the built library. */
int32_t spec_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
