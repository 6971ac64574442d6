/*
 * csk.h - C ABI of the gfx950 (MI355X) hybrid compressed attention library
 * (libcsk.so): CSA and HCA compression, MXFP4 quantisation, the lightning
 * indexer with top-k selection, and sparse / dense attention over
 * compressed KV entries with a sliding window and an attention sink.
 *
 * Sources (web pages about the DeepSeek-V4 technical report):
 *   [P1] "Техотчёт DeepSeek-V4 (2026): миллион токенов контекста" (ai.flicky.cc)
 *   [P2] "Статья DeepSeek V4: Ключевые технические находки официального
 *        отчёта" (framia.pro)
 *   [P3] aixai.ru blog post on V4's million-token context,
 *        section "Гибридный attention: CSA и HCA"
 *   [P4] "Технический отчёт DeepSeek-V4 — часть 1/2" (aifinder.ae mirror)
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers: every tensor pointer is a DEVICE pointer (hipMalloc'd or a
 *   torch CUDA tensor's data_ptr) to a dense row-major array, 4-byte aligned
 *   (16-byte alignment is faster; sparse_attn and dense_compressed_attn
 *   require it of q, kv_c, kv_w, out and the workspace, CSK_EINVAL
 *   otherwise). The caller owns every buffer; the compute
 *   calls never allocate or free device memory and keep no pointer or other
 *   state between calls (the one exception is the opt-in measurement hook
 *   csk_kernel_timer_arm, which keeps the caller's event arrays until
 *   csk_kernel_timer_disarm).
 * - Device: the calling thread's current HIP device must be a gfx950
 *   (MI355X); any other device, or none, makes a call that would launch
 *   return CSK_EUNSUPPORTED (argument errors are reported first).
 * - Streams: `stream` is a hipStream_t (NULL = the default stream). Every
 *   call only enqueues kernels on it and returns without synchronising, so
 *   a non-zero return code reports argument errors and launch failures, not
 *   faults inside kernels.
 * - Scratch: calls that need scratch memory take a caller-owned device
 *   `workspace` of at least the size the matching *_workspace_size()
 *   returns. Its contents on entry do not matter. Two calls that run at the
 *   same time must not share a workspace.
 * - Dtypes: CSK_F32 = float32, CSK_BF16 = bfloat16 (uint16 bit patterns),
 *   CSK_MXFP4 = packed E2M1 codes (element 2j in the low nibble of byte j)
 *   plus one E8M0 scale byte (2^(byte-127)) per 32 consecutive elements.
 *   CSK_FP8KV = a KV entry of D values whose last d_rope (RoPE) dims stay
 *   bf16 and whose first D_nope = D - d_rope dims are OCP E4M3 codes with
 *   one power-of-two scale byte (2^(byte-127)) per 32 dims ([P2]: FP8 KV
 *   storage; [P1] «Почему это так сильно экономит», item 1: FP8 KV with
 *   BF16 RoPE dims). Entry bytes: [D_nope codes][d_rope bf16][D_nope/32
 *   scales], padded with zeros to csk_fp8kv_entry_bytes(D, d_rope), a
 *   multiple of 16 (656 for 512 + 64, against 1152 in bf16). The scale of a
 *   block puts its largest magnitude in [128, 256) (s = floor(log2 amax) -
 *   7, clamped to [-126, 127]; an all-zero block has byte 127); codes are
 *   the nearest E4M3 value of x / 2^s, ties to the even mantissa, zero as
 *   the +0 code.
 * - Errors: every call returns CSK_OK (0) or a negative code and leaves a
 *   message for csk_last_error() (thread-local). Nothing aborts or prints.
 * - Determinism: results are bitwise reproducible run to run for the same
 *   arguments (no floating-point atomics on any result path). The attention
 *   calls' max_workgroups argument decides how a row is split, so results
 *   are reproducible for a fixed value of it.
 * - Rounding: compression and MXFP4 encoding compute in fp32 and round once
 *   to the output dtype (round to nearest even). Attention computes logits,
 *   softmax sums and outputs in fp32; with bf16 data its intermediates are
 *   bf16 where the matrix cores take them: the rotated query, the
 *   probabilities entering the P.V product, and (rows split over several
 *   workgroups) the partial outputs, which the merge combines in fp32 before
 *   the final rounding.
 */
#ifndef CSK_H
#define CSK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSK_OK 0
#define CSK_EINVAL (-1)       /* null pointer, bad size or combination of arguments */
#define CSK_EUNSUPPORTED (-2) /* dtype/shape combination not built, or no gfx950 device */
#define CSK_EWORKSPACE (-3)   /* workspace smaller than *_workspace_size() */
#define CSK_EHIP (-4)         /* HIP runtime error while launching */

#define CSK_F32 0
#define CSK_BF16 1
#define CSK_MXFP4 2
#define CSK_FP8KV 3

/* Bytes of one CSK_FP8KV entry of D values with d_rope RoPE dims (0 for a
 * shape that has none: D - d_rope not a multiple of 32, or d_rope odd). */
int csk_fp8kv_entry_bytes(int D, int d_rope);

/* Message for the last failing call on this thread ("" if none). */
const char* csk_last_error(void);

/* ABI revision of this header (incremented on incompatible change). */
int csk_abi_version(void);
#define CSK_ABI_VERSION 2

/*
 * csa_compress - CSA compression ([P1] «CSA: сжать в 4 раза и выбрать
 * top-k», step 1; [P4]: every 2m tokens with stride m become one entry).
 *
 * Two KV series (C^a, C^b) and two gate series (Z^a, Z^b) of width D are
 * pooled m-fold along the sequence. Entry i (global index e = entry0 + i)
 * takes, per channel c, a softmax over the logits Z^a + bias_a of its own
 * block of m tokens together with Z^b + bias_b of the previous block, and
 * outputs the softmax-weighted sum of the matching C values. Global entry 0
 * has no previous block (its softmax spans its m a-slots only). After
 * pooling, the last d_rope channels are rotated by partial RoPE at the
 * entry's position (interleaved channel pairs; pair j turns by
 * pos * rope_base^(-2j/d_rope), angle formed in fp64).
 *
 *   ca, za, cb, zb : source rows, in_dtype (CSK_F32 | CSK_BF16). Row r of
 *                    batch b is at element offset (b*src_bstride + r)*D, for
 *                    r in [0, S). When entry0 > 0, rows r in [-m, 0) of cb
 *                    and zb must also be readable: they form the previous
 *                    block of the first produced entry.
 *   bias_a, bias_b : [m, D] fp32 learned positional biases.
 *   B, S, D, m     : batch, source rows, channels, ratio; N = S/m entries are
 *                    produced (a trailing partial block produces none).
 *   entry0         : global index of the first produced entry (>= 0).
 *   src_bstride    : rows between batches in the sources (0 means S).
 *   d_rope         : rotated channels (even, <= D; 0 = none).
 *   entry_pos      : [B, N] int32 entry positions, or NULL for m*(entry0+i).
 *   out_dtype      : CSK_F32 | CSK_BF16 | CSK_MXFP4 (MXFP4 needs D % 32 ==
 *                    0) | CSK_FP8KV (needs (D - d_rope) % 32 == 0).
 *   out            : entry i of batch b at (b*dst_bstride + i)*D elements
 *                    (MXFP4: codes at byte offset (b*dst_bstride + i)*D/2;
 *                    FP8KV: the entry at byte (b*dst_bstride + i)*ES, ES =
 *                    csk_fp8kv_entry_bytes(D, d_rope)).
 *   out_scale      : MXFP4 only: scales at byte (b*dst_bstride + i)*D/32.
 *   dst_bstride    : entries between batches in the output (0 means N).
 */
int csa_compress(const void* ca, const void* za, const void* cb, const void* zb,
                 const float* bias_a, const float* bias_b, int B, int S, int D, int m,
                 int entry0, int64_t src_bstride, int d_rope, float rope_base,
                 const int32_t* entry_pos, int in_dtype, int out_dtype, void* out,
                 uint8_t* out_scale, int64_t dst_bstride, void* stream);

/*
 * hca_compress - HCA compression ([P1] «HCA: сжать в 128 раз, но смотреть
 * на всё»: ratio m' = 128, no window overlap). As csa_compress with a single
 * series: entry i pools its own block of m rows only. entry0 only sets the
 * default positions m*(entry0+i).
 */
int hca_compress(const void* c, const void* z, const float* bias, int B, int S, int D, int m,
                 int entry0, int64_t src_bstride, int d_rope, float rope_base,
                 const int32_t* entry_pos, int in_dtype, int out_dtype, void* out,
                 uint8_t* out_scale, int64_t dst_bstride, void* stream);

/*
 * mxfp4_quantize - MXFP4 encoding of rows of `cols` values ([P1] «FP4 с
 * учётом квантования»: the indexer's Q.K path is cached and multiplied in
 * FP4; MXFP4 with E2M1 elements in 1x32 tiles). Per tile of 32: scale
 * exponent s = floor(log2 max|x|) - 2 clamped to [-127, 127] (127 stored for
 * an all-zero tile); each element is the E2M1 value nearest to x/2^s, ties
 * to the even mantissa bit, saturating at 6; zero is always the +0 code.
 *   x      : [rows, cols] in_dtype (CSK_F32 | CSK_BF16), finite values.
 *   codes  : [rows, cols/2] bytes;  scales : [rows, cols/32] bytes.
 */
int mxfp4_quantize(const void* x, int in_dtype, int64_t rows, int cols, uint8_t* codes,
                   uint8_t* scales, void* stream);

/*
 * csk_compress_batch - several csa_compress and mxfp4_quantize calls in
 * one launch ([P1] «CSA…», step 1, and «FP4 с…»: the per-token work that
 * precedes the indexer and attention at decode - the newest KV entry, its
 * indexer key and the query encode - is three launches too small to fill
 * the chip; batched, they share one kernel boundary).
 *
 * Each job computes exactly what its own call computes, bit for bit. The
 * jobs run concurrently: no job may read what another writes.
 *   jobs[q].kind == CSK_JOB_CSA  : fields ca .. dst_bstride are the
 *       csa_compress arguments of the same names (S is the source rows),
 *       with m <= 8 and B*(S/m) <= 65535 entries.
 *   jobs[q].kind == CSK_JOB_MXFP4: fields x, in_dtype, rows (<= 65535) and
 *       cols are the mxfp4_quantize arguments; codes go to out and scales
 *       to out_scale.
 *   Unused fields are ignored. The job array is host memory, read during
 *   the call; device buffers stay owned by the caller.
 *   n_jobs : 1 .. CSK_MAX_JOBS.
 *   stream : hipStream_t (NULL = default stream); asynchronous.
 * Errors: CSK_EINVAL for a bad n_jobs, an unknown kind or any argument the
 * job's own call rejects with CSK_EINVAL (the message names the job);
 * CSK_EUNSUPPORTED for m > 8, more rows than stated or what the own call
 * rejects with CSK_EUNSUPPORTED. Nothing is launched unless every job is
 * valid; jobs that produce nothing are skipped.
 */
#define CSK_MAX_JOBS 4
#define CSK_JOB_CSA 1
#define CSK_JOB_MXFP4 2
typedef struct csk_compress_job {
  int kind;
  const void* ca;
  const void* za;
  const void* cb;
  const void* zb;
  const float* bias_a;
  const float* bias_b;
  int B, S, D, m, entry0;
  int64_t src_bstride;
  int d_rope;
  float rope_base;
  const int32_t* entry_pos;
  int in_dtype, out_dtype;
  void* out;
  uint8_t* out_scale;
  int64_t dst_bstride;
  const void* x;
  int64_t rows;
  int cols;
} csk_compress_job;
int csk_compress_batch(const csk_compress_job* jobs, int n_jobs, void* stream);

/*
 * indexer_topk - lightning indexer and top-k selection ([P1] «CSA…», step
 * 2; [P3]: FP4 lightning indexer with a ReLU-scored multi-head dot product).
 *
 * For query row (b,t) at position p = q_pos[b,t], compressed entry s is a
 * candidate when s < n_entries[b] and its last source token m*(s+1)-1 <= p.
 * Score I[t,s] = sum_h w[b,t,h] * ReLU(q[b,t,h] . k[b,s]), where each q.k
 * is the exact dot product rounded once to fp32 (MXFP4) or an fp32 fused
 * multiply-add chain over channels in ascending order (CSK_F32), and the
 * head sum is an fp32 fused multiply-add chain over h = 0..HI-1 from +0.
 * With score_dtype CSK_BF16 each score is then rounded once to the nearest
 * bf16 (ties to even) before the selection ([P1] «FP4 с учётом
 * квантования»: BF16 scores for the top-k); CSK_F32 keeps the fp32 score.
 * The min(k, #candidates) highest scores are selected, ties to the lower
 * index, and returned in ascending index order, padded with -1.
 *
 *   q, q_scale : MXFP4 [B,T,HI,dI/2] codes + [B,T,HI,dI/32] scales, or
 *                CSK_F32 [B,T,HI,dI] with q_scale NULL.
 *   w          : [B,T,HI] fp32 head weights.
 *   kk, k_scale: MXFP4 [B,Nmax,dI/2] + [B,Nmax,dI/32], or CSK_F32 [B,Nmax,dI].
 *   q_pos      : [B,T] int32 absolute positions;  n_entries: [B] int32.
 *   dtype      : CSK_MXFP4 (dI % 32 == 0) or CSK_F32.
 *   score_dtype: CSK_F32 or CSK_BF16 (the scores the selection compares).
 *   idx        : [B,T,k] int32 output;  score: [B,T,k] fp32 or NULL
 *                (scores of the returned entries as selected - the bf16
 *                values with CSK_BF16 - and -inf for padding).
 *   workspace  : >= indexer_topk_workspace_size(B,T,HI,dI,Nmax,k,dtype).
 */
int indexer_topk(const void* q, const uint8_t* q_scale, const float* w, const void* kk,
                 const uint8_t* k_scale, const int32_t* q_pos, const int32_t* n_entries, int B,
                 int T, int HI, int dI, int Nmax, int m, int k, int dtype, int score_dtype,
                 int32_t* idx, float* score, void* workspace, size_t ws_bytes, void* stream);
size_t indexer_topk_workspace_size(int B, int T, int HI, int dI, int Nmax, int k, int dtype);

/*
 * indexer_topk_noalloc - indexer_topk for callers that cannot allocate:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc. Same arguments and results as indexer_topk (the same kernels,
 * bit for bit), without the workspace: the scratch lives in a static
 * device array of CSK_NOALLOC_SCRATCH_BYTES that the library holds on every
 * device it has run on until the process ends. The call allocates and
 * frees nothing and needs no zeroed memory.
 *   Limit: indexer_topk_workspace_size(B,T,HI,dI,Nmax,k,dtype) must not
 *   exceed CSK_NOALLOC_SCRATCH_BYTES (32 MiB: 1M-context decode at batch 4,
 *   128K-context decode at batch 32); larger problems return
 *   CSK_EWORKSPACE before anything is launched.
 *   Concurrency: every call on one device shares that device's scratch, so
 *   calls that overlap in time on one device (other streams, other threads)
 *   race and must be serialised by the caller; calls on one stream are
 *   ordered and safe.
 *   Set-up: the first call on a device looks up the scratch address
 *   (hipGetSymbolAddress) with that device current.
 */
#define CSK_NOALLOC_SCRATCH_BYTES (32u << 20)
int indexer_topk_noalloc(const void* q, const uint8_t* q_scale, const float* w, const void* kk,
                         const uint8_t* k_scale, const int32_t* q_pos, const int32_t* n_entries, int B,
                         int T, int HI, int dI, int Nmax, int m, int k, int dtype, int score_dtype,
                         int32_t* idx, float* score, void* stream);

/*
 * sparse_attn - CSA attention: MQA over the selected compressed entries, a
 * sliding window of uncompressed tokens and an attention sink ([P1] «CSA…»,
 * step 3: every compressed entry is both key and value for all query heads;
 * «HCA…»: 128-token window of uncompressed entries; [P4]: SWA branch,
 * attention sink, partial RoPE on the last 64 dims).
 *
 * For row (b,t,h) at position p = q_pos[b,t]: q~ = q[b,t,h] with its last
 * d_rope channels rotated at p. Candidates: kv_c[b,i] for every i in
 * idx[b,t,:] with 0 <= i < Nmax (other values are skipped; duplicates
 * count twice), and kv_w[b,r] for every window row whose position
 * w_pos0[b]+r lies in [max(0, p-W+1), p]. One softmax runs over the logits
 * scale*(q~ . K) of all candidates plus the sink logit sink[h] (which adds
 * to the denominator only). out = sum_j p_j * K_j[0:dv], lse = M + ln Z.
 * With no candidate and no sink, out = 0 and lse = -inf.
 *
 *   q       : [B,T,H,D] dtype, unrotated;  q_pos: [B,T] int32.
 *   kv_c    : [B,Nmax,D] kv_dtype (entries already rotated);  idx: [B,T,k].
 *   kv_w    : [B,S_w,D] kv_dtype (already rotated) or NULL with S_w = 0.
 *   kv_dtype: the dtype of kv_c and kv_w: dtype, or CSK_FP8KV entries
 *             ([B,Nmax,ES] bytes, ES = csk_fp8kv_entry_bytes(D, d_rope); built
 *             for dtype CSK_BF16, H = 64, D = 576, d_rope = 64, dv = 512). An
 *             FP8 entry is used as its exact value (E4M3 code times its
 *             block's scale, or the bf16 RoPE dim), so the result is that of
 *             bf16 attention over the decoded entries.
 *   w_pos0  : [B] int32 position of window row 0 (may be NULL if S_w = 0).
 *   sink    : [H] fp32 or NULL (no sink).
 *   dtype   : CSK_BF16 (fp32 accumulation) or CSK_F32.
 *   out     : [B,T,H,dv] dtype;  lse: [B,T,H] fp32 or NULL.
 *   max_workgroups: scheduling cap (>= 0). A launch over fewer query rows
 *             than the chip has CUs splits each row's candidates over
 *             several workgroups, about one per CU by default (0); a value
 *             > 0 caps that split at max_workgroups workgroups in all (a row
 *             never gets fewer than one), so that a caller running other
 *             work beside the call on another stream can leave CUs to it.
 *             Within that limit a row's 64-candidate tiles go to the fewest
 *             workgroups that keep the longest run (34 tiles over at most 8
 *             workgroups: 7 runs of at most 5).
 *             The split decides the order in which partial results are
 *             combined, so it is part of what the result bits depend on; a
 *             smaller cap never needs a larger workspace.
 *   workspace: >= sparse_attn_workspace_size(..., max_workgroups).
 */
int sparse_attn(const void* q, const int32_t* q_pos, const void* kv_c, int Nmax,
                const int32_t* idx, int k, const void* kv_w, const int32_t* w_pos0, int S_w,
                int W, const float* sink, int B, int T, int H, int D, int dv, int d_rope,
                float rope_base, float scale, int dtype, int kv_dtype, void* out, float* lse,
                int max_workgroups, void* workspace, size_t ws_bytes, void* stream);
size_t sparse_attn_workspace_size(int B, int T, int H, int D, int dv, int k, int W, int dtype,
                                  int max_workgroups);

/*
 * dense_compressed_attn - HCA attention ([P1] «HCA…»: attention over the
 * compressed entries stays dense; [P3]: every query attends to all
 * compressed blocks). As sparse_attn, but the compressed candidates are
 * every entry i < n_entries[b] whose last source token m*(i+1)-1 <= p.
 *   n_entries: [B] int32;  m: compression ratio used for visibility.
 */
int dense_compressed_attn(const void* q, const int32_t* q_pos, const void* kv_c, int Nmax,
                          const int32_t* n_entries, int m, const void* kv_w,
                          const int32_t* w_pos0, int S_w, int W, const float* sink, int B, int T,
                          int H, int D, int dv, int d_rope, float rope_base, float scale,
                          int dtype, int kv_dtype, void* out, float* lse, int max_workgroups,
                          void* workspace, size_t ws_bytes, void* stream);
size_t dense_compressed_attn_workspace_size(int B, int T, int H, int D, int dv, int Nmax, int m,
                                            int W, int dtype, int max_workgroups);

/*
 * grouped_out_proj - grouped output projection of the attention heads
 * ([P1] «CSA: сжать в 4 раза и выбрать top-k», step 4: the heads' outputs
 * are split into g groups, each group is projected to an intermediate
 * width, and the groups' intermediates together are projected to the
 * hidden size, instead of one projection of all heads at once).
 *   o   : [R,H*dv] bf16, a row's heads consecutive (head h at h*dv) - the
 *         attention output [B,T,H,dv] with R = B*T.
 *   w1  : [g,dg,(H/g)*dv] bf16: group i (heads i*H/g .. (i+1)*H/g - 1)
 *         maps its (H/g)*dv values to dg intermediate features ([out, in]).
 *   w2  : [d,g*dg] bf16: the g*dg intermediates to the d hidden features.
 *   y   : [R,d] in y_dtype (CSK_BF16 or CSK_F32).
 *   workspace: >= grouped_out_proj_workspace_size(R, g, dg) bytes; after
 *         the call it holds the intermediate u [R,g*dg] in bf16 (each value
 *         accumulated in fp32 and rounded once, as the second product takes
 *         it).
 * Both products accumulate in fp32 on the matrix cores; y is rounded once
 * to y_dtype. Built for (H/g)*dv and g*dg multiples of 64 and d a multiple
 * of 8 (else CSK_EUNSUPPORTED); o, w1, w2, y and workspace must be 16-byte
 * aligned (else CSK_EINVAL). R = 0 is a no-op.
 */
int grouped_out_proj(const void* o, const void* w1, const void* w2, int R, int H, int dv, int g,
                     int dg, int d, int y_dtype, void* y, void* workspace, size_t ws_bytes,
                     void* stream);
size_t grouped_out_proj_workspace_size(int R, int g, int dg);

/*
 * project_compress - the series projected from hidden states and compressed
 * in one pass ([P1] «CSA: сжать в 4 раза и выбрать top-k», step 1: the KV
 * series C^a, C^b and the weight series Z^a, Z^b are computed from the
 * hidden states; «HCA…»: the same pooling over blocks of m' = 128 tokens;
 * «Muon и борьба с нестабильностью»: KV entries normalised directly by
 * RMSNorm). The series are products X W^T accumulated in fp32 on the matrix
 * cores and pooled in registers; they are never written to memory.
 *   csa     : 1 = CSA (m must be 4; w = [4,D,hidden]: W_ca, W_za, W_cb,
 *             W_zb), 0 = HCA (m must be 128; w = [2,D,hidden]: W_c, W_z;
 *             bias_b unused). Weights are [out, in] bf16.
 *   x       : [B,S,hidden] bf16 hidden states, token t of batch b at
 *             x + (b*src_bstride + t)*hidden (src_bstride 0 = S). CSA with
 *             entry0 > 0: the 4 tokens before each batch's first token are
 *             the previous block (the first entry's b slots) and are read.
 *   bias_a, bias_b: [m,D] fp32 positional biases of the a / b slots.
 *   gamma   : [D] fp32 RMSNorm scale, or NULL for no norm. With gamma each
 *             pooled entry e becomes e * gamma / sqrt(mean(e^2) + eps) over
 *             all D dims, before its RoPE rotation.
 *   entry0, d_rope, rope_base, entry_pos, out_dtype, out, out_scale,
 *   dst_bstride: as csa_compress.
 *   workspace: >= project_compress_workspace_size(csa, B, S, D, m) bytes
 *             (the pooled fp32 entries and per-block sums of squares).
 * Built for hidden % 64 == 0 and D % 32 == 0 (else CSK_EUNSUPPORTED); x, w
 * and workspace must be 16-byte aligned.
 */
int project_compress(int csa, const void* x, const void* w, const float* bias_a, const float* bias_b,
                     const float* gamma, float eps, int B, int S, int hidden, int D, int m, int entry0,
                     int64_t src_bstride, int d_rope, float rope_base, const int32_t* entry_pos,
                     int out_dtype, void* out, uint8_t* out_scale, int64_t dst_bstride, void* workspace,
                     size_t ws_bytes, void* stream);
size_t project_compress_workspace_size(int csa, int B, int S, int D, int m);

/*
 * rmsnorm - RMSNorm of rows of D values (the queries' per-head norm: rows =
 * B*T*H; [P1] «Muon и борьба с нестабильностью»; [P4]: QK norms):
 * y = x * gamma / sqrt(mean(x^2) + eps), the sum of squares in fp32.
 *   x: [rows,D] in in_dtype; gamma: [D] fp32; y: [rows,D] in out_dtype
 *   (CSK_F32 or CSK_BF16, rounded once). y may equal x (in place, same
 *   dtype).
 */
int rmsnorm(const void* x, const float* gamma, int64_t rows, int D, float eps, int in_dtype,
            int out_dtype, void* y, void* stream);

/*
 * csk_kernel_timer_arm - opt-in measurement hook (process-wide, one armed
 * timer at a time). The next n launches of the library kernel named
 * `kernel` ("indexer_scores_fp4", "attn_bf16_sparse", ...) are each
 * bracketed by hipEventRecord(ev_start[j]) / hipEventRecord(ev_stop[j]) on
 * the launch stream. The events are caller-created hipEvent_t handles; the
 * library keeps the two arrays (not copies) until csk_kernel_timer_disarm(),
 * so they must stay valid until then. csk_kernel_timer_count() returns how
 * many launches were recorded. While no timer is armed a launch reads one
 * atomic flag and nothing else.
 */
int csk_kernel_timer_arm(const char* kernel, void** ev_start, void** ev_stop, int n);
int csk_kernel_timer_count(void);
void csk_kernel_timer_disarm(void);

#ifdef __cplusplus
}
#endif
#endif
