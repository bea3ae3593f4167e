/*
 * mla.h - C ABI of libmla: DeepSeek-V3 multi-head latent attention (MLA)
 * decode in the absorbed form over a paged latent KV cache, for AMD MI355X
 * (gfx950).
 *
 * One decode step of one layer is:
 *
 *   mla_get_metadata   once per step (all layers share it): split-KV work plan
 *   mla_absorb_q       q_lat = W_UK^T q_nope per head
 *   mla_decode_paged   attention of every head against the shared latent rows
 *                      -> o_lat (latent output) and lse
 *   mla_up_v           o = o_lat @ W_UV per head
 *
 * The call order follows the FlashMLA usage the pages show (FlashMLA release
 * news, usage example: plan once per step with the query rows that share one
 * KV head, then per layer a paged decode returning the output and its lse),
 * with the absorption step of "DeepSeek-V3 Multi-head Latent Attention (MLA)
 * 深度工程" section 2.4 in front and the value up-projection of section 2.2
 * behind.
 *
 * Conventions shared by every call:
 *  - bf16 tensors are passed as uint16_t bit patterns; "bf16" below.
 *  - Every pointer is a DEVICE pointer unless the comment says host.
 *  - All tensors are dense, row-major, contiguous, in the shapes given.
 *  - Sizes: b sequences, s_q query tokens per sequence, h heads,
 *    M = s_q * h query rows per sequence. Row r = j * h + i of sequence b is
 *    query token j, head i; q_lat[b, j, i, :] is row b * M + r.
 *  - The caller owns every buffer. The library never allocates device memory
 *    in these calls and keeps no state between them (apart from the device
 *    error word, see mla_take_device_error).
 *  - `stream` is a hipStream_t (NULL = the null stream). Calls are
 *    asynchronous and ordered on that stream; outputs are valid once the
 *    stream has reached the call.
 *  - Return value: MLA_OK, or a negative mla_status after which NOTHING has
 *    been launched. mla_last_error() gives a message (per host thread).
 *  - Calls on distinct buffers are thread-safe; calls that share an output
 *    or workspace buffer on different streams race.
 */
#ifndef MLA_H
#define MLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Fixed cache format: a token is one 576-wide bf16 row, 512 latent values
 * (c_KV, section 2.2) followed by 64 rotated decoupled-RoPE key values
 * (section 3.1); 64 tokens per page (FlashMLA feature list: bf16, block 64). */
#define MLA_PAGE_TOKENS 64
#define MLA_D_LATENT 512
#define MLA_D_ROPE 64
#define MLA_D_ROW 576
#define MLA_D_NOPE 128
/* Quantised cache page ("DeepSeek-V3 Multi-head Latent Attention (MLA) 深度工程",
 * section 7.2 stores the latent in 8 bits; the format below is this library's
 * reading): 64 rows of MLA_FP8_ROW_BYTES bytes - the 512 latent values as OCP
 * fp8 e4m3 codes, then the 64 positional-key values as bf16 - followed by the
 * 64 per-token scales as fp32, in token order. Row t stands for
 * c_t = e4m3(code) * scale_t and k_pe_t as stored; scale_t = 2^e_t with e_t the
 * smallest integer such that max |c_t| <= 448 * 2^e_t, but at least -126 (an
 * all-zero row has scale 1). */
#define MLA_FP8_ROW_BYTES 640
#define MLA_FP8_SCALES_OFFSET (64 * MLA_FP8_ROW_BYTES)
#define MLA_FP8_PAGE_BYTES (MLA_FP8_SCALES_OFFSET + 64 * 4)
/* int32 words per slot in tile_meta */
#define MLA_META_WORDS 8
/* Largest batch the planner accepts. */
#define MLA_MAX_BATCH 8192

typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = -1,  /* null pointer, bad size, bad combination */
  MLA_ERR_UNSUPPORTED = -2,  /* well-formed but outside what is built */
  MLA_ERR_WORKSPACE = -3,    /* workspace smaller than mla_workspace_bytes */
  MLA_ERR_HIP = -4           /* a HIP runtime call failed */
} mla_status;

/* Device error bits, set by kernels when the caller's data break the contract
 * (the kernel then reads zeros instead of the bad address). */
#define MLA_DEVERR_PAGE_ID 1       /* block_table entry outside [0, num_pages) */
#define MLA_DEVERR_SEQ_TOO_LONG 2  /* cache_seqlens[b] > max_blocks * 64 */
#define MLA_DEVERR_SHORT_SEQ 4     /* mla_append_kv: cache_seqlens[b] < s_q */

/* Message for the last non-OK return on this host thread ("" if none). Host. */
const char* mla_last_error(void);

/* Number of workgroup slots the planner should cut the work into for this
 * shape on the current device (about one per compute unit). Host query. */
int mla_num_slots(int b, int s_q, int h, int* num_slots /* host out */);

/* Bytes of workspace mla_decode_paged needs for this shape and slot count:
 * partial rows of split sequences as fp16 [b + num_slots, M, 512] (each row
 * divided by its largest magnitude), their lse and row scales, fp32
 * [b + num_slots, M] each. Returns 0 for a shape the decode does not accept.
 * Host query. */
size_t mla_workspace_bytes(int b, int s_q, int h, int num_slots);

/* mla_get_metadata - split-KV work plan (FlashMLA usage: planned once per
 * decode step from cache_seqlens and reused by every layer).
 *
 * cache_seqlens  int32 [b]         cache length L_b of each sequence, counting
 *                                  the s_q new tokens; L_b <= 0 is empty.
 * b              1..MLA_MAX_BATCH
 * num_slots      1..2^20, the grid mla_decode_paged will run (mla_num_slots)
 * split_overhead >= 0, fixed cost of one sequence piece, in pages
 * tile_meta      int32 [num_slots, 8] out
 * num_splits     int32 [b + 1] out: prefix sums of the pieces per sequence
 *
 * The plan lays sequences with pages on a cost line (split_overhead + pages
 * units each) and gives slot s the units [s q, (s+1) q), q = ceil(total /
 * num_slots). tile_meta[s] = {b_begin, page_begin, b_end, page_end,
 * split_begin, 0, 0, 0}; an empty slot is {0, 0, -1, 0, 0, 0, 0, 0}. Requires
 * sum of (split_overhead + pages) < 2^31. */
int mla_get_metadata(const int32_t* cache_seqlens, int b, int num_slots, int split_overhead,
                     int32_t* tile_meta, int32_t* num_splits, void* stream);

/* mla_absorb_q - absorb W_UK into the query (section 2.4, absorption trick):
 * q_lat[b, j, i, :] = q_nope[b, j, i, :] @ W_UK[i], fp32 accumulation,
 * rounded to bf16 (nearest even). If q_lat_lo is not NULL it receives
 * bf16(q_lat_fp32 - q_lat), the rounding residue.
 *
 * q_nope  bf16 [b, s_q, h, 128]
 * w_uk    bf16 [h, 128, 512]     (W_UK[i] maps c to k: k = W_UK[i] c)
 * q_lat   bf16 [b, s_q, h, 512] out;  q_lat_lo  same shape, nullable
 * b >= 1, 1 <= s_q <= 8, h in {16, 32, 64, 128} */
int mla_absorb_q(const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_lat, uint16_t* q_lat_lo,
                 int b, int s_q, int h, void* stream);

/* mla_absorb_q_with_plan - mla_get_metadata and mla_absorb_q in one launch.
 * The plan reads only cache_seqlens and the absorption only the queries and
 * W_UK, so one workgroup plans while the others multiply; the launch that
 * would run the plan alone is saved. That pays only while every workgroup of
 * the GEMM is resident at once: when its tiles already fill the CUs (128
 * heads at b = 128, or more rows), the call runs the two kernels back to back
 * instead. Meant for the first layer of a decode step; later layers reuse
 * the plan and call mla_absorb_q.
 *
 * Arguments, outputs and error behaviour are those of the two calls:
 * q_nope, w_uk, q_lat, q_lat_lo, b, s_q, h as for mla_absorb_q;
 * cache_seqlens, num_slots, split_overhead, tile_meta, num_splits as for
 * mla_get_metadata (b <= MLA_MAX_BATCH). Both outputs are bit-identical to
 * those of the separate calls. Every check runs before the launch. */
int mla_absorb_q_with_plan(const uint16_t* q_nope, const uint16_t* w_uk, uint16_t* q_lat, uint16_t* q_lat_lo,
                           int b, int s_q, int h, const int32_t* cache_seqlens, int num_slots, int split_overhead,
                           int32_t* tile_meta, int32_t* num_splits, void* stream);

/* mla_decode_paged - paged MLA decode in the absorbed form.
 *
 * For sequence b and row r = (j, i) the kernel scores every visible cached
 * token t:  s_t = softmax_scale * (q_lat[r] . c_t + q_pe[r] . kpe_t), where
 * c_t = row[0:512] and kpe_t = row[512:576] of token t (concatenated content
 * and positional parts, section 3.1), takes an exact softmax in streaming
 * form (the pages' online-softmax recurrence, section 4.1) and returns
 * o_lat[r] = sum_t p_t c_t and lse[r] = ln sum_t exp(s_t) (natural log).
 * Token t of sequence b is row t % 64 of page block_table[b, t / 64].
 * With causal != 0, query j sees the first L_b - s_q + 1 + j tokens;
 * otherwise all L_b. A row that sees no token gets o_lat = 0, lse = -inf.
 * Scores use bf16 q_lat. When q_lat_lo (the bf16 rounding residue from
 * mla_absorb_q) is given, lse also carries that residue's first-order effect,
 * softmax_scale * (q_lat_lo[r] . o_lat[r]) (d lse / d s_t = p_t): without it
 * the bf16 rounding of q_lat alone moves lse by up to ~5e-3 on short caches.
 *
 * q_lat, q_lat_lo  bf16 [b, s_q, h, 512] (lo nullable), from mla_absorb_q
 * q_pe             bf16 [b, s_q, h, 64], rotated
 * kv_cache         bf16 [num_pages, 64, 576]
 * block_table      int32 [b, max_blocks]; entries past a sequence's pages
 *                  are never read
 * cache_seqlens    int32 [b], each <= max_blocks * 64
 * tile_meta, num_splits  from mla_get_metadata with the same cache_seqlens,
 *                  b and num_slots
 * workspace        >= mla_workspace_bytes(b, s_q, h, num_slots) bytes,
 *                  256-byte aligned; contents need not be initialised
 * o_lat            bf16 [b, s_q, h, 512] out
 * lse              fp32 [b, s_q, h] out
 * softmax_scale > 0 (1/sqrt(192) for DeepSeek-V3), 1 <= b <= MLA_MAX_BATCH,
 * 1 <= s_q <= 8, h in {16, 32, 64, 128}, num_pages >= 1, num_slots 1..2^20.
 * Page ids and lengths that break the contract are read as zero rows and set
 * a device error bit (mla_take_device_error). */
int mla_decode_paged(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                     const uint16_t* kv_cache, int64_t num_pages,
                     const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                     int b, int s_q, int h, float softmax_scale, int causal,
                     const int32_t* tile_meta, const int32_t* num_splits, int num_slots,
                     void* workspace, size_t workspace_bytes,
                     uint16_t* o_lat, float* lse, void* stream);

/* Size of the device array mla_decode_paged_noalloc uses in place of a
 * workspace: 72 MiB on every GPU the library runs on, held until the process
 * ends. It covers mla_workspace_bytes(b, s_q, h, mla_num_slots(...)) for
 * b = 128 sequences at s_q * h <= 256 rows and for 32 sequences of 1024 rows. */
#define MLA_NOALLOC_SCRATCH_BYTES (72u << 20)

/* mla_decode_paged_noalloc - mla_decode_paged for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops
 * and harnesses that forbid hipMalloc. It takes no workspace: the split
 * partials go to a fixed array of MLA_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per GPU. The call itself allocates nothing; its first call on a
 * device resolves that device's array address once.
 *
 * Arguments, outputs, results and error behaviour are those of
 * mla_decode_paged (the outputs are bit-identical to that call's), without
 * workspace and workspace_bytes. A shape whose
 * mla_workspace_bytes(b, s_q, h, num_slots) exceeds MLA_NOALLOC_SCRATCH_BYTES
 * returns MLA_ERR_WORKSPACE before anything is launched.
 *
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (nothing in it needs to start at zero). Calls that overlap on one
 * GPU - on different streams, or from several host threads - race on it and
 * must be ordered by the caller. */
int mla_decode_paged_noalloc(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                             const uint16_t* kv_cache, int64_t num_pages,
                             const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                             int b, int s_q, int h, float softmax_scale, int causal,
                             const int32_t* tile_meta, const int32_t* num_splits, int num_slots,
                             uint16_t* o_lat, float* lse, void* stream);

/* mla_up_v - value up-projection per head (section 2.2: v = W_UV c, applied
 * after attention since the output is linear in c):
 * o[b, j, i, :] = o_lat[b, j, i, :] @ W_UV[i], fp32 accumulation, bf16 out.
 *
 * o_lat bf16 [b, s_q, h, 512]; w_uv bf16 [h, 512, 128]; o bf16 [b, s_q, h, 128] out.
 * b >= 1, 1 <= s_q <= 8, h in {16, 32, 64, 128}. */
int mla_up_v(const uint16_t* o_lat, const uint16_t* w_uv, uint16_t* o, int b, int s_q, int h,
             void* stream);

/* mla_gather_pages - the decode kernel's page loader on its own, for tests:
 * copies the rows of tokens 0 .. L_b - 1 of each sequence, in token order,
 * from the paged cache through LDS to out[row_offsets[b] + t, :].
 * Token t of sequence b is row t % 64 of page block_table[b, t / 64] (paged
 * KV cache, SC11 note "Page Attention" paragraph).
 *
 * kv_cache bf16 [num_pages, 64, 576]; block_table int32 [b, max_blocks];
 * cache_seqlens int32 [b]; row_offsets int64 [b]; out bf16 [sum L_b, 576]. */
int mla_gather_pages(const uint16_t* kv_cache, int64_t num_pages, const int32_t* block_table,
                     int max_blocks, const int32_t* cache_seqlens, int b,
                     const int64_t* row_offsets, uint16_t* out, void* stream);

/* mla_append_kv - write the step's new cache rows into their pages.
 * The compression stage caches only each token's latent c_KV ("DeepSeek-V3
 * Multi-head Latent Attention (MLA) 深度工程", section 2.2) with its positional
 * key k_pos (section 3.2, already rotated here); the paged module of section
 * 4.3 stores the new token's latent into the paged cache before it attends.
 * Token t of sequence b is row t % 64 of page block_table[b, t / 64].
 * cache_seqlens counts the s_q new tokens (as in mla_decode_paged), so new
 * row j of sequence b becomes token L_b - s_q + j.
 *
 * new_rows       bf16 [b, s_q, 576]: c_KV (512 values) then rotated k_pe (64)
 * kv_cache       bf16 [num_pages, 64, 576], updated in place
 * block_table    int32 [b, max_blocks]; the caller has mapped the pages the
 *                new tokens fall in
 * cache_seqlens  int32 [b]
 * b >= 1, 1 <= s_q <= 8, num_pages >= 1, max_blocks >= 1.
 * Only the destination rows change; the copy is bit-exact. A row whose token
 * index is negative (L_b < s_q: MLA_DEVERR_SHORT_SEQ) or lies past the block
 * table (MLA_DEVERR_SEQ_TOO_LONG), or whose page id lies outside
 * [0, num_pages) (MLA_DEVERR_PAGE_ID), is skipped and sets that device error
 * bit. If two new rows map to the same cache row (a block table that shares
 * pages between sequences), which one lands is unspecified. */
int mla_append_kv(const uint16_t* new_rows, uint16_t* kv_cache, int64_t num_pages,
                  const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                  int b, int s_q, void* stream);

/* mla_quantize_pages - convert a bf16 paged cache into the quantised page
 * format (MLA_FP8_PAGE_BYTES per page; see MLA_FP8_ROW_BYTES): per row, the
 * scale 2^e, the latent values divided by it (exact) and rounded to the
 * nearest e4m3 code (ties to even), the positional key copied.
 *
 * kv_cache  bf16 [num_pages, 64, 576] with finite values
 * kv_fp8    uint8 [num_pages, MLA_FP8_PAGE_BYTES] out, 16-byte aligned
 * num_pages >= 1. Every page is converted, in place of the caller's rows. */
int mla_quantize_pages(const uint16_t* kv_cache, int64_t num_pages, uint8_t* kv_fp8, void* stream);

/* mla_append_kv_fp8 - mla_append_kv into a quantised cache: each new row is
 * quantised as by mla_quantize_pages and its 640 row bytes and scale are
 * written at token L_b - s_q + j of sequence b. Arguments, checks and device
 * error bits as for mla_append_kv; kv_fp8 is uint8 [num_pages,
 * MLA_FP8_PAGE_BYTES], 16-byte aligned. Only the destination rows and scales
 * change. */
int mla_append_kv_fp8(const uint16_t* new_rows, uint8_t* kv_fp8, int64_t num_pages,
                      const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                      int b, int s_q, void* stream);

/* mla_decode_paged_fp8 - mla_decode_paged over a quantised cache. The result
 * is the decode of the cache the quantised pages stand for (latent values
 * e4m3(code) * scale, positional keys as stored): scores apply each token's
 * scale to its latent dot product, and the probabilities that weight its
 * latent row carry the scale too. Arguments, outputs, workspace and error
 * behaviour are those of mla_decode_paged, with kv_fp8 uint8 [num_pages,
 * MLA_FP8_PAGE_BYTES] (16-byte aligned) in place of kv_cache. Built for at
 * most 32 query rows per sequence (s_q * h <= 32: a tensor-parallel share of
 * the heads): larger shapes return MLA_ERR_UNSUPPORTED. */
int mla_decode_paged_fp8(const uint16_t* q_lat, const uint16_t* q_lat_lo, const uint16_t* q_pe,
                         const uint8_t* kv_fp8, int64_t num_pages,
                         const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                         int b, int s_q, int h, float softmax_scale, int causal,
                         const int32_t* tile_meta, const int32_t* num_splits, int num_slots,
                         void* workspace, size_t workspace_bytes,
                         uint16_t* o_lat, float* lse, void* stream);

/* Device error word: returns in *bits (host) the MLA_DEVERR_* bits kernels
 * set since the last call, then clears them. Synchronises the device. The
 * read and the clear are two copies: a bit set by a kernel that another host
 * thread launches between them is lost, so call it while no other thread
 * launches work on the device. */
int mla_take_device_error(int* bits /* host out */);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H */
