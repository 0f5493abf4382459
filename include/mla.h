/*
 * mla.h — C ABI of the MLA (multi-head latent attention) decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * What one decode step computes, for every sequence b and query head i, over
 * the L_b cached tokens of b (no mask: every cached token is attended):
 *
 *     o[b,i] = W_UV[i] · softmax_t( scale · ( q̃[b,i]·c_t + q_R[b,i]·k_R,t ) ) · c_t
 *     q̃[b,i] = W_UK[i]ᵀ · q_C[b,i]
 *
 * where c_t (d_latent wide) is the cached joint KV latent of token t and k_R,t
 * (d_rope wide) is its decoupled RoPE key, shared by all heads.  Sources:
 *  - "DeepSeek V2的MLA注意力机制…低秩压缩技术…" (snabindia.com):
 *    §2.1 the keys and values are rebuilt from one latent, K = W_U^K·KV_comp
 *    and V = W_U^V·KV_comp; §2.2 the decoupled query (content part q_C,
 *    position part q_R) and the single position key shared by all heads;
 *    §2.3 only KV_comp and k_R are cached, the score is the dot product of
 *    the concatenated query and key over sqrt(d), and W_U^K can be absorbed
 *    into the query and W_U^V applied after the weighted sum (§4.1
 *    optimize_for_inference);  §3.1 the DeepSeek-V2 geometry (128 heads,
 *    head dim 128, d_c = 512, RoPE dim 64).
 *  - "Multi-Head Latent Attention（MLA）：大模型KV Cache显存优化原理与实操"
 *    (CSDN): §2.1 textbook attention softmax(QKᵀ/sqrt(d_k))·V; §3.2 the
 *    latent cache is a [seq, latent] array per sequence.
 *  - "engineering DeepSeek sparse attention long context inference"
 *    (hotdry.top): FP8 KV cache for 128K contexts; the nn.Linear weight
 *    layout [h·d, d_c] of the up-projections.
 *
 * The step is four calls, each only enqueued on the caller's HIP stream:
 *     mla_absorb_q  ->  mla_decode  ->  mla_combine  ->  mla_up_proj
 * (mla_combine_up_proj does the last two in one launch for bf16 W_UV).
 * Around the step: mla_cache_append writes each sequence's new token into the
 * cache before it; mla_absorb_q_rope is mla_absorb_q with the decoupled RoPE
 * of q_R applied; mla_decode_multi takes several query tokens per sequence
 * (causal among them); mla_mha_decode is the multi-head attention baseline
 * over a full per-head K/V cache, the cache MLA replaces.
 * mla_decode splits every sequence into num_splits token ranges and writes one
 * normalised partial result per range; mla_combine merges them exactly with
 * log-sum-exp weights; with num_splits == 1 the partial already is the final
 * u and mla_combine may be skipped.
 *
 * Conventions for every call
 *  - Pointers named as tensors are DEVICE pointers, owned by the caller,
 *    row-major and contiguous, with the shapes given at each argument.  The
 *    library never allocates, frees, retains or synchronises: each call
 *    validates its arguments on the host, enqueues kernels on `stream`
 *    (a hipStream_t; NULL = the default stream) and returns.
 *  - Errors: argument problems are reported synchronously, before any launch,
 *    as a status code (nothing is printed, no exception crosses the ABI).
 *    A failed launch returns MLA_E_HIP.  Faults inside a kernel surface at the
 *    caller's next synchronisation, as with any asynchronous HIP work.
 *  - Thread safety: no mutable global state; calls on different streams are
 *    independent.
 *  - dtype codes: MLA_F32 (IEEE binary32), MLA_BF16 (upper half of binary32),
 *    MLA_FP8_E4M3 (OCP 8-bit E4M3, bias 7, no infinities, max 448).
 *  - Compiled geometry: d_latent = 512 and d_rope = 64 (the DeepSeek-V2
 *    values); d_nope and d_v may be 1..256 in mla_absorb_q / mla_up_proj.
 *  - Data: a sequence of length 0 yields u = 0, lse = -inf and o = 0.
 *    Cache slots that hold no token of the sequence being read (past its
 *    length, the tail of its last page) are never read and may hold anything,
 *    including NaN.  NaN or Inf in read inputs propagate.
 */
#ifndef MLA_H
#define MLA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MLA_OK = 0,
  MLA_E_ARG = 1,         /* null pointer, negative size, bad enum value */
  MLA_E_DTYPE = 2,       /* dtype combination not provided */
  MLA_E_SHAPE = 3,       /* dimension outside the compiled geometry */
  MLA_E_ALIGN = 4,       /* a pointer or stride violates the stated alignment */
  MLA_E_HIP = 5,         /* the HIP runtime reported an error at launch */
  MLA_E_UNSUPPORTED = 6, /* valid request the library does not provide */
  MLA_E_SCRATCH = 7      /* request larger than the library's static scratch */
} mla_status_t;

typedef enum { MLA_F32 = 0, MLA_BF16 = 1, MLA_FP8_E4M3 = 2 } mla_dtype_t;

/* Model geometry of one attention layer.
 * softmax_scale <= 0 selects 1/sqrt(d_nope + d_rope): the scale belongs to the
 * per-head query/key width of the non-absorbed form (DeepSeek V2 page §2.3),
 * not to the 576-wide absorbed dot product. */
typedef struct {
  int32_t heads;     /* h >= 1 */
  int32_t d_nope;    /* content (non-RoPE) query/key width per head */
  int32_t d_rope;    /* decoupled RoPE width (64) */
  int32_t d_latent;  /* latent width d_c (512) */
  int32_t d_v;       /* value width per head */
  float softmax_scale;
} mla_dims_t;

/* The latent KV cache of one layer.  Every cached token is one row of
 * d_latent + d_rope elements, [c_KV | k_R] (DeepSeek V2 page §2.3: only the
 * latent and the RoPE key are cached).
 *
 * Contiguous (page_size == 0): token t of sequence b is row b*seq_stride + t.
 * Paged (page_size == 64): token t of sequence b is row
 *   block_table[b*max_pages + t/64]*64 + t%64  (pages of 64 rows; the DeepSeek
 * V2 page §1.2 / §3.3 lists paged KV memory as the companion optimisation).
 *
 * Ring (ring == 1, contiguous only; [V2] §4.1 keeps the KV cache in a ring
 * buffer so that it can grow): the seq_stride rows of sequence b are a ring of
 * capacity C = seq_stride and token t sits in row b*seq_stride + t % C, so
 * the ring holds the last min(L_b, C) tokens; those are the ones attended
 * (a window of the last C tokens once L_b > C; seq_lens and max_seq_len may
 * then exceed seq_stride).  Attention does not depend on the order of the
 * tokens, so the decode reads the ring's first min(L_b, C) rows.
 * mla_cache_ring_grow moves a ring into a larger one.
 *
 * rows must be 16-byte aligned.  An FP8_E4M3 cache carries one fp32 factor per
 * row in row_scale (same row index): value = decode(code) * row_scale[row]. */
typedef struct {
  int32_t dtype;               /* mla_dtype_t of rows */
  const void* rows;            /* device, [n_rows][d_latent + d_rope] */
  const float* row_scale;      /* device, [n_rows]; FP8 only, else NULL */
  int32_t page_size;           /* 0 or 64 */
  int64_t seq_stride;          /* contiguous: rows between sequences (>= max length) */
  const int32_t* block_table;  /* device, [B][max_pages]; paged only */
  int32_t max_pages;
  const int32_t* seq_lens;     /* device, [B], each in [0, max_seq_len] */
  int32_t max_seq_len;         /* host-side bound on every seq_lens[b] */
  int32_t ring;                /* 0, or 1: contiguous rows used as a ring (above) */
} mla_cache_t;

/* Absorb W_UK into the query (DeepSeek V2 page §2.3 and §4.1):
 *   q_abs[b][i][0:d_latent]        = sum_n q_nope[b][i][n] * W_UK[i][n][:]
 *   q_abs[b][i][d_latent:+d_rope]  = q_rope[b][i][:]
 * q_nope [B][h][d_nope], q_rope [B][h][d_rope] (dtype q_dt, F32 or BF16);
 * w_uk [h][d_nope][d_latent] (w_dt, F32 or BF16); fp32 accumulation.
 * q_abs [B][h][d_latent+d_rope] in q_abs_dt: F32 or BF16 (round to nearest
 * even), or FP8_E4M3 for the fp8-cache decode (the FP8 KV cache of the
 * "engineering DeepSeek sparse attention long context inference" page, with
 * the query in the same format): then q_abs_scale is device fp32 [B][h] and
 * each row, the 576 values of one (b, i) computed in fp32, is stored by the
 * fp8 cache rows' rule: q_abs_scale[b][i] = max(amax, 2^-126) / 448 with amax
 * the row's largest magnitude, code = the E4M3 value nearest to the binary32
 * quotient value / q_abs_scale[b][i] (ties to even, clamped to +-448).  The
 * FP8 output needs BF16 inputs, d_nope a multiple of 16 and at most 128, and
 * 16-byte aligned q_nope, q_rope and w_uk (else MLA_E_UNSUPPORTED).
 * q_abs_scale must be NULL for the other output dtypes (MLA_E_ARG). */
mla_status_t mla_absorb_q(const mla_dims_t* dims, int32_t B, const void* q_nope,
                          const void* q_rope, int32_t q_dt, const void* w_uk,
                          int32_t w_dt, void* q_abs, int32_t q_abs_dt,
                          float* q_abs_scale, void* stream);

/* mla_absorb_q with the decoupled RoPE of the positional query ([V2] §2.2:
 * q_R and k_R carry the position, q_C does not; frequencies 1/base^(2i/d_r)
 * as in the rotary listings of [V2] and [LAT], whose cat(freqs, freqs) form
 * pairs element i with element i + d_r/2):
 *   q_abs[b][i][d_latent + j] = rotation of q_rope[b][i][:] by positions[b]:
 *     x[j] cos t_j - x[j + d_r/2] sin t_j          (j < d_r/2)
 *     x[j] cos t_j + x[j - d_r/2] sin t_(j-d_r/2)  (j >= d_r/2)
 *   t_j = positions[b] * inv_freq[j] in binary32, inv_freq[j] = base^(-2j/d_r)
 *   rounded once to binary32; every head of a sequence shares its position.
 * The latent part is mla_absorb_q's.  positions: device int32 [B] (any value);
 * rope_base > 1 and finite (10000 in the listings), else MLA_E_ARG.  k_R in
 * the cache is expected already rotated by its own token's position.  Other
 * arguments and errors as mla_absorb_q; q_abs_dt FP8_E4M3 (which would need a
 * scale) returns MLA_E_ARG. */
mla_status_t mla_absorb_q_rope(const mla_dims_t* dims, int32_t B, const void* q_nope,
                               const void* q_rope, int32_t q_dt, const void* w_uk,
                               int32_t w_dt, const int32_t* positions, float rope_base,
                               void* q_abs, int32_t q_abs_dt, void* stream);

/* Attention of every head over the latent cache, split into num_splits token
 * ranges per sequence.  Split p of sequence b covers tokens
 *   [p*C, min((p+1)*C, L_b)),  C = 32 * ceil(max_seq_len / (32*num_splits)),
 * so every range is a whole number of 32-token tiles; an empty range writes
 * u = 0 and lse = -inf.  When one workgroup takes R > 1 consecutive ranges
 * it merges them (one softmax over their tokens, the same log-sum-exp merge
 * mla_combine does): split g then covers ranges gR .. gR + R - 1, i.e.
 * tokens [gRC, min((g+1)RC, L_b)), and the splits from ceil(num_splits / R)
 * on hold lse = -inf with their u_part not written.  That happens with an FP8 query, and
 * with a BF16 cache when num_splits >= 32, for
 *   R = min(num_splits, max(1, floor(B * q_len * num_splits * ceil(h/64) / 256)))
 * (enough workgroups to fill the 256 CUs once); otherwise R = 1.  For each
 * (b, p, i) over split p's token set T:
 *   s_t  = scale * (q_abs[b][i][0:d_latent]·c_t + q_abs[b][i][d_latent:]·k_R,t)
 *   u_part[b][p][i][:] = sum_{t in T} e^{s_t} c_t / sum_{t in T} e^{s_t}
 *   lse_part[b][p][i]  = ln sum_{t in T} e^{s_t}      (natural log)
 * q_abs [B][h][d_latent+d_rope] (q_abs_dt); q_abs_scale: device fp32 [B][h]
 * for an FP8 query (value = code * q_abs_scale[b][i]), else NULL.  u_part
 * [B][num_splits][h][d_latent] in part_dt (F32 or BF16); lse_part
 * [B][num_splits][h] fp32.  1 <= num_splits <= 1024.
 * Provided dtype pairs (cache / q_abs): F32/F32, BF16/BF16, FP8/BF16 and
 * FP8/FP8; other pairs return MLA_E_DTYPE.  An FP8 cache is read as
 * code * row_scale.  With a BF16 query every code is widened exactly to bf16,
 * the row scale multiplies the score and the bf16-rounded probability in the
 * PV product.  With an FP8 query both products run on the fp8 matrix cores
 * over the raw codes, in ranges of whole 64-token tiles
 * (C = 64 * ceil(max_seq_len / (64*num_splits))): the scores are the exact
 * code products times both factors, and the PV product takes p * row_scale
 * rounded to E4M3 with one power-of-two factor per (head, 32 tokens) that
 * puts the largest of them in [128, 256); l sums the unrounded p.  The BF16
 * and FP8 paths need h to be a multiple of 32. */
mla_status_t mla_decode(const mla_dims_t* dims, int32_t B, const void* q_abs,
                        int32_t q_abs_dt, const float* q_abs_scale,
                        const mla_cache_t* cache, int32_t num_splits, void* u_part,
                        int32_t part_dt, float* lse_part, void* stream);

/* mla_decode for q_len query tokens per sequence (a multi-token step, e.g. a
 * speculative draft): the last q_len cached rows of sequence b are its new
 * tokens, and query token j (0-based) attends causally ([LAT]'s varlen
 * attention call with causal=True) to the cached rows
 *   t < L_b - (q_len - 1 - j),   L_b = min(seq_lens[b], max_seq_len),
 * i.e. its own row and the rows before it (none if that bound is <= 0: u = 0,
 * lse = -inf).  q_abs [B][q_len][h][576] (mla_absorb_q over B*q_len
 * sequences); u_part [B][q_len][num_splits][h][d_latent] and lse_part
 * [B][q_len][num_splits][h] are laid out as mla_decode's for B*q_len
 * sequences, so mla_combine / mla_combine_up_proj over B*q_len finish the
 * step.  Split ranges as mla_decode's (from max_seq_len).  1 <= q_len <= 16
 * (else MLA_E_ARG); BF16 and FP8 caches (an F32 cache with q_len > 1 returns
 * MLA_E_UNSUPPORTED, and so does a ring cache with q_len > 1: the windows of
 * the earlier query tokens reach tokens the ring has overwritten).  Other arguments and errors as mla_decode (no
 * q_abs_scale). */
mla_status_t mla_decode_multi(const mla_dims_t* dims, int32_t B, int32_t q_len,
                              const void* q_abs, int32_t q_abs_dt, const mla_cache_t* cache,
                              int32_t num_splits, void* u_part, int32_t part_dt,
                              float* lse_part, void* stream);

/* Decode kernels (the work decomposition of the BF16-cache decode; the result
 * is the same up to rounding order):
 *   MLA_KERNEL_H64  -- one workgroup per (sequence, split range, 64 heads);
 *                      two workgroups share each cached tile through L2.
 *                      Every cache dtype.
 *   MLA_KERNEL_H64_BALANCED -- the 64-head kernel over a balanced partition
 *                      of the batch instead of the fixed split ranges, for
 *                      ragged batches (split-KV sized to the chip rather than
 *                      to the longest sequence).  Rows v = b * q_len + j lie
 *                      end to end, row v weighing 5 + n_v when it attends
 *                      A_v > 0 tokens (n_v = ceil(A_v / 32) tiles, placed after
 *                      its 5 units of start weight) and 0 when it attends none,
 *                      N = the total weight; the line is cut into G spans
 *                      [floor(w N / G), floor((w+1) N / G)),
 *                        G = min(256 / ceil(h / 64),
 *                                max(1, floor(N / ceil(n_max / (S - 1)))))
 *                      with n_max the largest row weight (G = 1 if N = 0), so
 *                      no row meets more than S = num_splits spans.  Split p of
 *                      row v is the part of v's tiles in span w_v + p, w_v = the
 *                      span holding v's first tile;
 *                      splits past v's last span, and all splits of an
 *                      empty row, are empty (lse = -inf, u not written).  mla_combine
 *                      and mla_combine_up_proj merge them as any other
 *                      splits.  BF16 cache and query, 2 <= num_splits, B *
 *                      q_len <= 512 and B * q_len * (ceil(max_seq_len / 32) + 5)
 *                      < 2^31; else MLA_E_UNSUPPORTED.
 *   (an FP8 query always runs its own 64-head kernel: AUTO or H64.)
 *   MLA_KERNEL_AUTO -- what mla_decode and mla_decode_multi use: H64.
 * Values 2 and 3 named workgroups of 128 heads (each tile entering one CU
 * once for all heads); they measured slower than H64 on every full-size bf16
 * workload (with one 36 KB tile in flight per CU their stream is
 * latency-bound under full load) and are retired: MLA_E_UNSUPPORTED. */
typedef enum {
  MLA_KERNEL_AUTO = 0,
  MLA_KERNEL_H64 = 1,
  MLA_KERNEL_H64_BALANCED = 4
} mla_decode_kernel_t;

/* mla_decode_multi with the decode kernel chosen by the caller (`kernel`, an
 * mla_decode_kernel_t).  q_len = 1 is mla_decode.  A kernel for a cache or
 * shape it does not cover returns MLA_E_UNSUPPORTED, as do the retired values
 * 2 and 3; an unknown value MLA_E_ARG.  Other arguments, layouts and errors as mla_decode_multi. */
mla_status_t mla_decode_ex(const mla_dims_t* dims, int32_t B, int32_t q_len, const void* q_abs,
                           int32_t q_abs_dt, const mla_cache_t* cache, int32_t num_splits,
                           void* u_part, int32_t part_dt, float* lse_part, int32_t kernel,
                           void* stream);

/* Measurement: the decode's tile stream without its arithmetic, the ceiling its
 * HBM fraction is read against ([REV]'s KV-bottleneck introduction: the cache
 * stream's bandwidth is the quantity).  `workgroups` workgroups of 512 threads
 * each stream `tiles` consecutive 36,864-byte tiles (32 rows of 1152 bytes) of
 * `src` (device, 16-byte aligned, src_bytes long) into LDS with the decode's
 * DMA and waits, 2 tiles in flight, and discard them; with `paired` (an even
 * number of workgroups) workgroups 2k and 2k+1 of the XCD-aware order read the
 * same tiles, as the decode's two head groups do; else each its own.  Reads
 * (paired ? workgroups/2 : workgroups) * tiles * 36864 bytes (more than
 * src_bytes: MLA_E_SHAPE).  sink: device int32 [workgroups], overwritten.
 * MLA_E_ARG for a NULL pointer, workgroups or tiles < 1, or an odd paired
 * count; MLA_E_ALIGN for a misaligned src. */
mla_status_t mla_stream_probe(const void* src, int64_t src_bytes, int32_t workgroups,
                              int32_t tiles, int32_t paired, int32_t* sink, void* stream);

/* Merge the split partials of mla_decode with log-sum-exp weights:
 *   lse[b][i] = ln sum_p e^{lse_part[b][p][i]}
 *   u[b][i][:] = sum_p e^{lse_part[b][p][i] - lse[b][i]} * u_part[b][p][i][:]
 * Parts with lse = -inf carry no weight and their u_part is not read; if
 * every part is empty, u = 0 and
 * lse = -inf.  u_part/lse_part as written by mla_decode; u [B][h][d_latent]
 * in u_dt (F32 or BF16); lse [B][h] fp32 or NULL. */
mla_status_t mla_combine(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                         const void* u_part, int32_t part_dt, const float* lse_part,
                         void* u, int32_t u_dt, float* lse, void* stream);

/* Apply W_UV after the weighted sum (DeepSeek V2 page §2.3):
 *   o[b][i][v] = sum_c W_UV[i][v][c] * u[b][i][c]
 * u [B][h][d_latent] (u_dt, F32 or BF16); w_uv [h][d_v][d_latent] (w_dt, F32
 * or BF16); o [B][h][d_v] in o_dt (F32 or BF16, round to nearest even);
 * fp32 accumulation. */
mla_status_t mla_up_proj(const mla_dims_t* dims, int32_t B, const void* u,
                         int32_t u_dt, const void* w_uv, int32_t w_dt, void* o,
                         int32_t o_dt, void* stream);

/* mla_combine followed by mla_up_proj in one launch, without the round trip
 * of u through memory:
 *   u[b][i][:]  = merge of the split partials as in mla_combine, rounded to
 *                 bf16 (the value mla_combine stores for u_dt = BF16)
 *   o[b][i][v]  = sum_c W_UV[i][v][c] * u[b][i][c]      (fp32 accumulation)
 * u_part/lse_part as written by mla_decode (part_dt F32 or BF16); w_uv
 * [h][d_v][d_latent] BF16 only, d_v a multiple of 16; o [B][h][d_v] in o_dt
 * (F32 or BF16).  u (BF16 [B][h][d_latent]) and lse (fp32 [B][h]) are
 * optional copies of the merged values: NULL skips them.  Same conventions
 * and errors as the two calls it replaces; MLA_E_DTYPE for other dtypes,
 * MLA_E_SHAPE for d_v % 16 != 0. */
mla_status_t mla_combine_up_proj(const mla_dims_t* dims, int32_t B, int32_t num_splits,
                                 const void* u_part, int32_t part_dt, const float* lse_part,
                                 const void* w_uv, int32_t w_dt, void* o, int32_t o_dt,
                                 void* u, float* lse, void* stream);

/* Append the new token of every sequence to the cache: the step before
 * mla_decode ([V2] §2.3: per token and layer only the latent c_KV and the
 * RoPE key k_R shared by all heads are cached; [DSA]: a 128K-token cache is
 * kept in FP8).  For each b with 0 <= positions[b] < capacity (contiguous:
 * seq_stride rows per sequence; paged: max_pages * 64 tokens) the row of
 * token positions[b] (the row mla_decode reads for it) becomes
 *   [c_kv[b][0:d_latent] | k_r[b][0:d_rope]]
 * in the cache dtype: F32 the input value; BF16 the input rounded to nearest
 * even; FP8_E4M3 the codes of x / s with s = fp32(max(amax, 2^-126) / 448),
 * amax the row's largest |x|, each quotient (binary32, correctly rounded)
 * clamped to +-448 and rounded to the nearest E4M3 value, ties to the even
 * mantissa; s is stored in row_scale[row].  The same bits as the input
 * quantiser of the fp8 workloads.
 * c_kv [B][d_latent] and k_r [B][d_rope] in src_dt (F32 or BF16), finite;
 * positions: device int32 [B].  A position < 0 or past the capacity, or a
 * negative page id in block_table, skips the sequence; no other row is
 * written.  A ring cache (ring == 1) has no capacity limit: token t goes to
 * row b*seq_stride + t % seq_stride, over the token C positions back.  cache->rows (and row_scale for FP8) are written through: they must
 * be writable; seq_lens and max_seq_len are neither read nor changed (the
 * caller advances its lengths).  The cache must satisfy mla_decode's layout
 * rules (16-byte aligned rows, page_size 0 or 64).  Errors: MLA_E_ARG for
 * missing pointers or a bad layout, MLA_E_SHAPE for another page size,
 * MLA_E_DTYPE for an FP8 input, MLA_E_ALIGN for misaligned rows. */
mla_status_t mla_cache_append(const mla_dims_t* dims, int32_t B, const void* c_kv,
                              const void* k_r, int32_t src_dt, const int32_t* positions,
                              const mla_cache_t* cache, void* stream);

/* Grow (or shrink) ring caches ([V2] §4.1: the ring buffer allows the cache
 * to grow): for every sequence b, the tokens its ring in `src` holds, the last
 * k = min(L_b, src.seq_stride, dst.seq_stride) of them (L_b = min(seq_lens[b],
 * max_seq_len) of src), are copied with their row factors into the ring of
 * `dst`, token t to row b*dst.seq_stride + t % dst.seq_stride.  Nothing else
 * in dst is written.  A ring grown before it wrapped (L_b <= src.seq_stride)
 * keeps every token; the caller then sets dst's lengths (the same L_b) and
 * appends into dst.  Both caches: ring == 1, contiguous, the same dtype
 * (FP8: both carry row_scale), 16-byte aligned rows, and must not overlap.
 * Errors: MLA_E_ARG (pointers, not rings, a paged cache), MLA_E_DTYPE
 * (dtypes differ), MLA_E_ALIGN. */
mla_status_t mla_cache_ring_grow(int32_t B, const mla_cache_t* src, const mla_cache_t* dst,
                                 void* stream);

/* Multi-head attention decode over a full per-head K/V cache: the baseline
 * the latent cache replaces ([LAT] §2.1 softmax(q k^T / sqrt(d_k)) v; [V2]
 * §1.1 the MHA cache holds K and V of every head, 2 x h x d elements per
 * token and layer against MLA's d_c + d_r).  For every sequence b and head i:
 *   s_t = scale * q[b][i] . k[b][i][t],  t < L_b = min(seq_lens[b], max_seq_len)
 *   o[b][i][:] = sum_t e^{s_t} v[b][i][t][:] / sum_t e^{s_t}
 *   lse[b][i]  = ln sum_t e^{s_t}  (-inf and o = 0 for an empty sequence)
 * scale = softmax_scale, or 1/sqrt(d_head) when softmax_scale <= 0.
 * q [B][heads][d_head]; k_cache, v_cache [B][heads][seq_stride][d_head]
 * (head-major), all BF16 and 16-byte aligned; d_head = 128; seq_stride >=
 * max_seq_len; o [B][heads][d_head] in o_dt (F32 or BF16); lse fp32 [B][heads]
 * or NULL.  Errors: MLA_E_ARG (pointers, lengths, NaN scale), MLA_E_SHAPE
 * (d_head), MLA_E_DTYPE (dtypes), MLA_E_ALIGN. */
mla_status_t mla_mha_decode(int32_t B, int32_t heads, int32_t d_head, const void* q,
                            const void* k_cache, const void* v_cache, int32_t dt,
                            const int32_t* seq_lens, int64_t seq_stride, int32_t max_seq_len,
                            float softmax_scale, void* o, int32_t o_dt, float* lse,
                            void* stream);

/* For callers that cannot allocate: code under HIP graph capture, serving
 * loops and harnesses that forbid hipMalloc.  mla_decode followed by
 * mla_combine_up_proj, with the split partials (bf16) and their log-sum-exps
 * in a device buffer the library owns instead of caller-given u_part /
 * lse_part.  No call here allocates or frees memory: the buffer is a static
 * device array of 64 MiB + 256 KiB, one per GPU the library runs on, held
 * until the process ends; its address on a device is looked up on the first
 * call made with that device current.
 *   Limit: B * num_splits * heads <= 65536 rows (e.g. 64 sequences x 8 splits
 *   x 128 heads); larger requests return MLA_E_SCRATCH before any launch.
 * Every call on one GPU uses that GPU's single buffer: calls that overlap on
 * one GPU (other streams, other host threads) race and must be serialised by
 * the caller; consecutive calls on one stream are ordered.  The decode writes
 * every partial row it is asked for (u = 0, lse = -inf for an empty range),
 * so nothing is cleared between calls.
 * Arguments as mla_decode (q_abs BF16 for BF16 / FP8 caches, F32 for F32;
 * no q_abs_scale) and mla_combine_up_proj (w_uv BF16, d_v % 16 == 0; o in
 * o_dt F32 or BF16; u BF16 [B][h][d_latent] and lse fp32 [B][h] optional,
 * NULL skips them); the same errors, plus MLA_E_SCRATCH, and MLA_E_HIP if
 * the buffer's address cannot be found. */
mla_status_t mla_decode_combine_up_proj_noalloc(const mla_dims_t* dims, int32_t B,
                                                const void* q_abs, int32_t q_abs_dt,
                                                const mla_cache_t* cache, int32_t num_splits,
                                                const void* w_uv, int32_t w_dt, void* o,
                                                int32_t o_dt, void* u, float* lse,
                                                void* stream);

/* Grouped-query attention decode, the other baseline ([LAT] §2.2: the query
 * heads are split into groups and each group shares one key/value head; [V2]
 * §1.2 lists MQA/GQA next to MLA).  The heads query heads form kv_heads
 * contiguous groups of G = heads / kv_heads: query head i reads key/value head
 * i / G.  As mla_mha_decode otherwise, with k_cache and v_cache
 * [B][kv_heads][seq_stride][d_head]; kv_heads == heads is mla_mha_decode and
 * kv_heads == 1 multi-query attention.  kv_heads < 1 or not dividing heads:
 * MLA_E_ARG. */
mla_status_t mla_gqa_decode(int32_t B, int32_t heads, int32_t kv_heads, int32_t d_head,
                            const void* q, const void* k_cache, const void* v_cache, int32_t dt,
                            const int32_t* seq_lens, int64_t seq_stride, int32_t max_seq_len,
                            float softmax_scale, void* o, int32_t o_dt, float* lse,
                            void* stream);

/* Chunked prefill in the naive (rebuild) form, step 1 of 2 ([V2] §2.1: keys
 * and values rebuilt from the latent; [LAT] §4.2-4.3: prefill of long inputs
 * with a causal varlen attention; [REV] "2. 分块并行计算": the prompt in
 * chunks).  For every sequence b and cached token t in [from_b, L_b)
 * (from_b = rebuild_from[b], or 0 when rebuild_from is NULL; L_b =
 * min(seq_lens[b], max_seq_len)) and every head i:
 *   k[b][i][t][0:d_nope]        = W_UK[i] c_t     (fp32 accumulation, bf16 RNE)
 *   k[b][i][t][d_nope:+d_rope]  = k_R,t           (copied)
 *   vt[b][i][v][t]              = (W_UV[i] c_t)[v]
 * k [B][h][kv_stride][d_nope + d_rope], vt [B][h][d_v][kv_stride] (values
 * stored transposed: the layout the attention step reads), BF16, 16-byte
 * aligned; kv_stride >= max_seq_len and a multiple of 32.  Rows outside
 * [from_b, L_b) are not written: with rebuild_from the caller keeps the keys
 * and values of earlier chunks and rebuilds only the new rows.  Cache: BF16,
 * contiguous or paged (not a ring); w_uk, w_uv BF16; d_nope = d_v = 128.
 * Errors: MLA_E_ARG, MLA_E_SHAPE (geometry), MLA_E_DTYPE, MLA_E_ALIGN,
 * MLA_E_UNSUPPORTED (ring cache). */
mla_status_t mla_prefill_rebuild_kv(const mla_dims_t* dims, int32_t B, const mla_cache_t* cache,
                                    const int32_t* rebuild_from, const void* w_uk,
                                    const void* w_uv, int32_t w_dt, void* k, void* vt,
                                    int64_t kv_stride, void* stream);

/* Chunked prefill, step 2 of 2: causal attention of a chunk of new tokens
 * over the rebuilt keys and values.  Sequence b has n_b = min(q_lens[b], q_len)
 * new tokens, the last n_b of its L_b = min(seq_lens[b], max_seq_len) cached
 * tokens; query token j < n_b sits at position p = L_b - n_b + j and attends
 * the tokens t <= p ([LAT] §4.2: causal=True):
 *   s_t = scale * q[b][j][i] . k[b][i][t]                 (192 wide)
 *   o[b][j][i][:] = sum_t e^{s_t} V[b][i][t][:] / sum_t e^{s_t}
 *   lse[b][j][i]  = ln sum_t e^{s_t}
 * (no token: o = 0, lse = -inf).  q [B][q_len][h][d_nope + d_rope] BF16, the
 * un-absorbed query [q_C | q_R]; q_lens device int32 [B]; k, vt as written by
 * mla_prefill_rebuild_kv; o [B][q_len][h][d_v] in o_dt (F32 or BF16); lse fp32
 * [B][q_len][h] or NULL.  Rows j >= n_b are not written.  Errors as
 * mla_prefill_rebuild_kv. */
mla_status_t mla_prefill_attn(const mla_dims_t* dims, int32_t B, int32_t q_len,
                              const int32_t* q_lens, const void* q, int32_t q_dt, const void* k,
                              const void* vt, int64_t kv_stride, const int32_t* seq_lens,
                              int32_t max_seq_len, void* o, int32_t o_dt, float* lse,
                              void* stream);

/* Static description of a status code (never NULL). */
const char* mla_status_str(mla_status_t status);

/* Library version, major*10000 + minor*100 + patch. */
int32_t mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_H */
