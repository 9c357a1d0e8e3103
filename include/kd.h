/*
 * kd.h — C ABI of the batched multi-session decode step on MI355X (gfx950).
 *
 * One decode step for B in [1, 16] concurrent sessions: every block-quantised weight
 * matrix is streamed from HBM once and applied to all B rows (mmvq at m = B), and each row
 * attends over its own ragged-length fp16 KV cache with a split-K flash-decode.  The
 * operation is the batched decode step of memra-engine 0.72.0 (src/decode_batch.rs:
 * module header "bandwidth thesis" and "exactness contract", ``decode_batch_layers``) and
 * the fused batch=N decode of hf2q ADR-040 (§0.4 corrected mental model, §0.7 F2-F5).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers named as device pointers point to GPU memory owned by the caller (for
 *    example allocated through torch); the library allocates no memory on any call.
 *    Host arrays (positions, cache base-address tables, descriptors) are read during the
 *    call only and may be freed when it returns.
 *  - ``stream`` is a ``hipStream_t`` (NULL = the null stream).  Work is enqueued
 *    asynchronously; no entry point synchronises the stream.
 *  - Arguments are validated on the host before anything is enqueued.  On any error
 *    nothing is enqueued and the status says why; ``kd_last_error()`` returns a
 *    thread-local message.  KD_ERR_HIP means a launch failed; the stream's contents for
 *    that call are then undefined.
 *  - Row invariance: for every entry point, output row b depends only on input row b (and
 *    on row b's own cache), never on B or on the other rows: the B-row result equals, bit
 *    for bit, the 1-row call on row b alone (memra-engine decode_batch.rs exactness
 *    contract; hf2q ADR-040 §0.12 execution log: the row-parity proof of the
 *    batched lm_head and the dense-matmul row-identity fix).
 *  - Calls that share a workspace must not overlap (use one workspace per stream).
 *
 * Native layouts (MI355X-first; produced by the pack / quantise entry points)
 * --------------------------------------------------------------------------
 *  A quantised matrix has n_out rows and k columns, k % 32 == 0, 32-element blocks.
 *  NR = ceil(n_out / 16) row groups, NQ = ceil(k / 128) block quads.  Tile t = r * NQ + q
 *  holds rows [16r, 16r + 16) x blocks [4q, 4q + 4); rows/blocks past the matrix are zero.
 *  Inside a tile, "lane" l = 16 g + n (g in 0..3, n in 0..15) owns row 16r + n and the
 *  eight block elements P_g = {4g..4g+3, 4g+16..4g+19} of each of the four blocks, so a
 *  64-lane wave reads a tile with fully coalesced 16-byte loads and feeds it straight to
 *  v_mfma_i32_16x16x32_i8 (K = 32 = one block).
 *   - KD_FMT_Q8_0 qs: 2048 bytes per tile.  Bytes [h*1024 + 16 l, +16) = int8 codes P_g of
 *     block 4q+2h (first 8 bytes) and of block 4q+2h+1 (last 8 bytes), h in {0,1}.
 *   - KD_FMT_Q4_0 qs: 1024 bytes per tile.  Bytes [16 l + 4 j, +4) = bytes [4g, 4g+4) of
 *     block 4q+j in GGUF order (low nibble = element i, high nibble = element i+16,
 *     value = nibble - 8).
 *   - d (both formats): fp16, 64 per tile: d[t * 64 + 4 n + j] = scale of row 16r+n,
 *     block 4q+j.
 *   - K-quant formats (KD_FMT_Q4_K, KD_FMT_Q5_K, KD_FMT_Q6_K; k % 256 == 0): the GGUF
 *     k-quant weight types the pages list among the formats a batched decode must cover
 *     (hf2q ADR-040 "Quant scope"; memra-engine decode_batch.rs exact-16 admission list).
 *     Source rows are k / 256 records of 256 values (Q4_K 144 bytes: fp16 d, fp16 dmin,
 *     12 bytes of packed 6-bit sub-block scales and mins, 128 bytes of 4-bit codes, value
 *     d sc_j q - dmin m_j in 32-value sub-block j; Q5_K 176 bytes: the same with 32 bytes
 *     of fifth bits before the codes; Q6_K 210 bytes: 128 bytes of low 4 bits, 64 bytes of
 *     upper 2 bits, 16 int8 scales, fp16 d, value d sc_(e/16) (q - 32)).  Tiles: qs bytes
 *     [16 l + 4 j, +4) = the low 4 bits of the codes P_g of block 4q+j, byte i holding
 *     element 4g+i in its low nibble and 4g+16+i in its high nibble; then (Q5_K, 1280
 *     bytes per tile) byte 1024 + 4 l + j = the fifth bits (bit i: element 4g+i, bit 4+i:
 *     4g+16+i), or (Q6_K, 1536 bytes per tile) bytes [1024 + 8 l + 2 j, +2) = the upper
 *     two bits (pair i of the first byte: element 4g+i; of the second: 4g+16+i); Q4_K tiles
 *     are 1024 bytes.  d: 192 bytes per tile: bytes [8 n + 2 j, +2) = sub-block scale and
 *     min of block 4q+j of row 16r+n (Q6_K: the int8 scales of its two 16-value halves),
 *     bytes [128 + 4 n, +4) = the row's fp16 d and dmin of that super-block (Q6_K: d, 0).
 *     A tiled K-quant matrix is 2.8-5.6 % larger than its records (d and dmin once per
 *     half record, the 12-byte scale packing unpacked to 8 bytes per quad).
 *  Quantised activations (kd_act_q8) for B rows of length k: int8 codes
 *  qs[(b * NQ + q) * 128 + 32 g + 8 j + e] = code of element P_g[e] of block 4q+j of row b,
 *  and fp32 scales d[b * 4 NQ + blk]; padded blocks have code 0 and scale 0.
 *  KV caches: per (session, layer) one K and one V array, fp16 [G][capacity][hd]
 *  (head-major: each KV head's keys are one contiguous stream).
 */
#ifndef KD_H
#define KD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KD_OK = 0,
  KD_ERR_INVALID = -1,      /* null pointer, bad shape, mismatched counts */
  KD_ERR_UNSUPPORTED = -2,  /* B outside [1,16], k % 32 != 0, head_dim not 64/128, H % G != 0, format */
  KD_ERR_CAPACITY = -3,     /* a row's pos + 1 exceeds the cache capacity */
  KD_ERR_WORKSPACE = -4,    /* workspace too small or null */
  KD_ERR_HIP = -5           /* a HIP launch failed */
} kd_status;

typedef enum {
  KD_FMT_Q8_0 = 1,
  KD_FMT_Q4_0 = 2,
  KD_FMT_F32 = 3,
  KD_FMT_Q4_K = 4,
  KD_FMT_Q5_K = 5,
  KD_FMT_Q6_K = 6
} kd_format;
/* KV cache element formats (kd_model_desc.kv_format). */
typedef enum { KD_KV_F16 = 0, KD_KV_FP8_E4M3 = 1, KD_KV_Q8_0 = 2 } kd_kv_format;

#define KD_MAX_B 16

/* A quantised matrix in the native tiled layout (device pointers, 16-byte aligned).
 * For KD_FMT_F32 (router only): qs is float [n_out][k] row-major and d is NULL. */
typedef struct {
  int32_t fmt;
  int32_t n_out;
  int32_t k;
  const void* qs;
  const void* d;
} kd_weight;

/* Quantised activations in the native layout (device pointers). */
typedef struct {
  int8_t* qs;
  float* d;
} kd_act_q8;

const char* kd_version(void);
const char* kd_last_error(void);

/* ---- layouts ------------------------------------------------------------------------ */
/* Bytes of the tiled qs and d arrays of an n_out x k matrix (0 on bad arguments). */
size_t kd_weight_qs_bytes(int32_t fmt, int32_t n_out, int32_t k);
size_t kd_weight_d_bytes(int32_t fmt, int32_t n_out, int32_t k);
/* Bytes of the qs and d arrays of B quantised activation rows of length k. */
size_t kd_act_qs_bytes(int32_t B, int32_t k);
size_t kd_act_d_bytes(int32_t B, int32_t k);

/* Repack a matrix from the row-major block layout (Q8_0: int8 [n_out][k]; Q4_0: uint8
 * [n_out][k/2], 16 bytes per block; d: fp16 [n_out][k/32]; K-quants: uint8 records
 * [n_out][k/256][144 | 176 | 210] with src_d unused and may be NULL; device pointers) into
 * the tiled layout above (dst_qs / dst_d sized by kd_weight_*_bytes).  Once per matrix, at
 * load. */
kd_status kd_pack_weight(int32_t fmt, int32_t n_out, int32_t k, const void* src_qs, const void* src_d,
                         void* dst_qs, void* dst_d, void* stream);

/* ---- activation quantiser ----------------------------------------------------------- */
/* Q(x) of fp32 rows x[B][k] (row stride ldx floats): per 32-element block a = max|x_i|,
 * d = a / 127 (IEEE fp32 division; 0 if a == 0), q_i = round-half-away(x_i / d) clamped
 * to [-127, 127].  The activation operand of every m = B product (memra-engine
 * decode_batch.rs, ``quantize_q8_1`` in ``decode_batch_layers``). */
kd_status kd_quantize_act_q8(const float* x, int32_t B, int32_t k, int32_t ldx, kd_act_q8 out, void* stream);

/* ---- mmvq at m = B -------------------------------------------------------------------- */
/* y[b][n] = sum_blk d_w[n][blk] * d_x[b][blk] * S[b][n][blk], S = exact int32 block dot of
 * the codes, for n < W->n_out, b < B; y row stride ldy floats (>= n_out).  One pass over
 * the weights serves all B rows (memra-engine decode_batch.rs ``matmul_pre`` at m = B;
 * hf2q ADR-040 §0.7 F3).  The fp32 accumulation order of each output depends only on k.
 * W->fmt must match the entry point.  Every product takes k <= 16384 and a matrix whose
 * tiled codes stay under 2 GiB (KD_ERR_UNSUPPORTED otherwise). */
kd_status kd_mmvq_q8_0(const kd_weight* W, kd_act_q8 x, int32_t B, float* y, int32_t ldy, void* stream);
kd_status kd_mmvq_q4_0(const kd_weight* W, kd_act_q8 x, int32_t B, float* y, int32_t ldy, void* stream);
/* The same product for any quantised format (Q8_0, Q4_0, Q4_K, Q5_K, Q6_K).  K-quants:
 * y[b][n] = sum_blk d_x[b][blk] (d sc_j S[b][n][blk] - dmin m_j X[b][blk]) for Q4_K / Q5_K,
 * X the sum of the activation codes of the block, and sum_blk d_x d (sc' S' + sc'' S'') for
 * Q6_K over the block's two 16-value halves; every S and X an exact integer, the fp32 terms
 * in block order (a function of k only: rows are B-invariant, as for the other formats).
 * The fused products below (SwiGLU, add + RMSNorm, RoPE) take every format as well. */
kd_status kd_mmvq(const kd_weight* W, kd_act_q8 x, int32_t B, float* y, int32_t ldy, void* stream);

/* ---- row operations (fp32, rows of length n, row stride n) ------------------------- */
/* y = x / sqrt(mean(x^2) + eps) * g  (memra-engine decode_batch.rs attn_norm / output norm). */
kd_status kd_rmsnorm_rows(const float* x, const float* g, float* y, int32_t B, int32_t n, float eps, void* stream);
/* x1 = x + r; y = rmsnorm(x1, g)  (memra-engine decode_batch.rs ``add_rms_norm``). */
kd_status kd_add_rmsnorm_rows(const float* x, const float* r, const float* g, float* x1, float* y,
                              int32_t B, int32_t n, float eps, void* stream);
/* In-place NEOX RoPE of x[B][n_heads][hd]: element i < hd/2 pairs with i + hd/2 and both
 * rotate by pos[b] * base^(-2i/hd); angles and their cos/sin are evaluated in fp64 and
 * rounded to fp32 (memra-engine decode_batch.rs ``rope_neox`` with the per-row position
 * buffer).  pos is a host array [B]. */
kd_status kd_rope_neox_rows(float* x, int32_t B, int32_t n_heads, int32_t hd, const int32_t* pos,
                            float base, void* stream);
/* a = silu(g) * u  (memra-engine decode_batch.rs ``silu_mul``). */
kd_status kd_swiglu_rows(const float* g, const float* u, float* a, int32_t B, int32_t n, void* stream);
/* z = x + y  (memra-engine decode_batch.rs residual ``add``). */
kd_status kd_add_rows(const float* x, const float* y, float* z, int32_t B, int32_t n, void* stream);

/* ---- products with fused epilogues ----------------------------------------------------- */
/* The dense FFN's first product with SwiGLU in its epilogue: W is [2F, k] with the gate and
 * up rows interleaved in blocks of 32 (the kd_layer_desc stacked layout, F % 32 == 0); the
 * output is Q(silu(gate) * up) for the B rows, in the activation layout for k = F
 * (kd_act_qs_bytes(B, F) / kd_act_d_bytes(B, F)).  silu(g) * u = g / (1 + e^-g) * u, as
 * kd_swiglu_rows (memra-engine decode_batch.rs FFN arm: gate, up, activation, quantise). */
kd_status kd_mmvq_swiglu(const kd_weight* W, kd_act_q8 x, int32_t B, kd_act_q8 out, void* stream);
/* The attention input product with NEOX RoPE and the fp16 KV append in its epilogue: W is
 * wqkv ([(H + 2G) hd, k]) with each head's rows in pair order (kd_layer_desc wqkv_pair_rows);
 * q_out fp32 [B][ldq] receives the rotated q (H hd columns); the rotated k and the v rows go
 * to position pos[b] of row b's caches as kd_kv_append stores them; angles as
 * kd_rope_neox_rows (fp64 from pos and rope_base) (memra-engine decode_batch.rs phase A). */
kd_status kd_mmvq_rope(const kd_weight* W, kd_act_q8 x, int32_t B, int32_t H, int32_t G, int32_t hd,
                       float* q_out, int32_t ldq, void* const* k_base, void* const* v_base,
                       const int32_t* pos, int32_t capacity, float rope_base, void* stream);

/* RMSNorm split across two products (the fused form of the O product + residual add +
 * post-attention norm, and of the down product + residual + next attention norm; memra-engine
 * decode_batch.rs ``decode_batch_layers``: o product, add_rms_norm, quantise before the next
 * products).  A workgroup of the producing product owns 32 output rows, one quantisation
 * block of the next product's input, but not the whole row, so it cannot know 1/rms:
 * kd_mmvq_resnorm computes x1 = res + W x (fp32 [B][n_out], x1 may not alias res), quantises
 * z = x1 * gain block by block with each block's own scale max|z|/127 into `out` (the
 * activation layout for k = n_out), and writes ss[b][blk] = the block's sum of x1^2 (fp32
 * [B][n_out / 32]).  The consumer (kd_mmvq_swiglu_normed, kd_mmvq_rope_normed, with the
 * same rows as x and norm_ss = ss) multiplies each output of row b by
 * 1 / sqrt(sum_blk ss[b][blk] / k + eps): y = x1 * that * gain has the same codes as z, and
 * the block scale times it is y's scale, so the pair computes the product of Q(RMSNorm(x1))
 * up to rounding.  n_out % 32 == 0 and n_out <= 4096; the consumers' k <= 4096. */
kd_status kd_mmvq_resnorm(const kd_weight* W, kd_act_q8 x, int32_t B, const float* res, const float* gain, float* x1,
                          kd_act_q8 out, float* ss, void* stream);
kd_status kd_mmvq_swiglu_normed(const kd_weight* W, kd_act_q8 x, int32_t B, const float* norm_ss, float eps,
                                kd_act_q8 out, void* stream);
kd_status kd_mmvq_rope_normed(const kd_weight* W, kd_act_q8 x, int32_t B, const float* norm_ss, float eps, int32_t H,
                              int32_t G, int32_t hd, float* q_out, int32_t ldq, void* const* k_base,
                              void* const* v_base, const int32_t* pos, int32_t capacity, float rope_base,
                              void* stream);

/* ---- KV append and ragged split-K decode attention --------------------------------- */
/* Store row b's k[b][G][hd] and v[b][G][hd] (fp32, rounded to fp16 nearest-even) at
 * position pos[b] of its own cache: K_b[g][pos[b]][:] (memra-engine decode_batch.rs phase A,
 * one launch for all B rows through the per-row cache pointer table).  k_base / v_base /
 * pos are host arrays [B]; several rows may share a cache only at distinct positions. */
kd_status kd_kv_append(const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                       void* const* k_base, void* const* v_base, const int32_t* pos,
                       int32_t capacity, void* stream);
/* Workspace bytes of kd_fa_decode_ragged for these per-row key counts (host t_kv[B]). */
size_t kd_fa_decode_workspace(int32_t B, int32_t H, int32_t hd, const int32_t* t_kv);
/* A sliding window is a view: pass k_base[b] + off hd, v_base[b] + off hd (fp16 elements) and
 * t_kv[b] = the window's key count, with the same capacity (the head stride).
 * out[b][h][:] = sum_j softmax_j(q[b][h] . K_b[g][j] * scale) V_b[g][j], j < t_kv[b],
 * g = h / (H/G) (memra-engine decode_batch.rs phase B, ``fa_decode_batch_seqs_v4``: one
 * launch over all rows plus one combine).  Keys are split into chunks of
 * c_b = max(128, ceil(t_b / 256)) — a function of the row's own t_kv only — and the chunk
 * partials are merged in chunk order.  q, out: fp32 [B][H][hd]; caches fp16 [G][capacity][hd];
 * H/G must be 1, 2, 4 or 8, hd 64 or 128, 1 <= t_kv[b] <= min(capacity, 131072). */
kd_status kd_fa_decode_ragged(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                              const void* const* k_base, const void* const* v_base,
                              const int32_t* t_kv, int32_t capacity, float scale, float* out,
                              void* ws, size_t ws_bytes, void* stream);

/* kd_fa_decode_ragged for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same computation and
 * output bits, with the split partials kept in a scratch array the library holds on each GPU
 * it runs on (16 MiB per GPU, until the process ends) instead of a caller's workspace.  The
 * call allocates nothing.  A call whose partials need more than the array
 * (kd_fa_decode_workspace > 16 MiB) returns KD_ERR_WORKSPACE before anything is enqueued.
 * Every call on one GPU shares its array: calls that overlap on one GPU (on different streams,
 * or from several threads) race and must be serialised by the caller. */
kd_status kd_fa_decode_ragged_noalloc(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                      const void* const* k_base, const void* const* v_base, const int32_t* t_kv,
                                      int32_t capacity, float scale, float* out, void* stream);

/* FP8 KV caches (memra-engine decode_batch.rs phase A stores quantised K/V rows, with an fp8
 * switch on the store and on ``fa_decode_kvmod``; the byte format is not given there).  Read
 * here as OCP FP8 E4M3, one byte per element, no scale: bit 7 sign, bits 6..3 exponent with
 * bias 7, bits 2..0 mantissa, no infinities, 0x7F / 0xFF NaN.  Caches are uint8
 * [G][capacity][hd]; everything else as the fp16 calls.
 * kd_kv_append_fp8 stores each fp32 value as its nearest E4M3 code (ties to the even code,
 * magnitudes past 448 saturate to +-448, NaN -> 0x7F with its sign).
 * kd_fa_decode_ragged_fp8 widens every code to its exact value (all E4M3 values are fp16
 * numbers) and computes what kd_fa_decode_ragged computes on those values; the same
 * workspace (kd_fa_decode_workspace).  NaN codes are outside its input domain. */
kd_status kd_kv_append_fp8(const float* k, const float* v, int32_t B, int32_t G, int32_t hd,
                           void* const* k_base, void* const* v_base, const int32_t* pos,
                           int32_t capacity, void* stream);
kd_status kd_fa_decode_ragged_fp8(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                  const void* const* k_base, const void* const* v_base,
                                  const int32_t* t_kv, int32_t capacity, float scale, float* out,
                                  void* ws, size_t ws_bytes, void* stream);

/* int8 KV caches (memra-engine decode_batch.rs, phase A: the append stores quantised K/V rows,
 * ``append_kv_quantized_seqs`` with per-token row bytes; Strata PR #1524 "What changes": resident
 * int8 KV; the byte format is not given there).  Read here as Q8_0 blocks along each cached
 * head row: a cache is uint8 [G][capacity][hd + 16]; row (g, j) holds hd int8 codes, then hd/32
 * fp16 scales (one per 32 consecutive elements), then zeros.  A block's value i is d * q_i.
 * kd_kv_append_q8 codes each block of the fp32 k and v rows: a = max |x_i|, d = fp16(a / 127)
 * (fp32 division, round to nearest even), q_i = round-half-away(x_i / d) clamped to
 * [-127, 127] (all 0 when d is 0); it writes the codes and scales, never the padding (a cache
 * starts zeroed).  kd_fa_decode_ragged_q8 computes what kd_fa_decode_ragged computes on those
 * values: scores on the codes with one fp32 sum per block, scaled by the block scales; values
 * d q_i formed exactly in fp32 and carried as fp16 hi + lo (values within the fp16 range, as
 * for fp16 caches); the same workspace (kd_fa_decode_workspace).  A sliding window is a view at
 * k_base[b] + off (hd + 16) bytes. */
kd_status kd_kv_append_q8(const float* k, const float* v, int32_t B, int32_t G, int32_t hd, void* const* k_base,
                          void* const* v_base, const int32_t* pos, int32_t capacity, void* stream);
kd_status kd_fa_decode_ragged_q8(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                 const void* const* k_base, const void* const* v_base, const int32_t* t_kv,
                                 int32_t capacity, float scale, float* out, void* ws, size_t ws_bytes,
                                 void* stream);

/* ---- gated delta rule (linear-attention layers) -------------------------------------- */
/* One decode step of the gated delta rule for B rows (memra-engine decode_batch.rs, the
 * Linear mixer of decode_batch_layers: one batched scan launch over every sequence's state,
 * through a per-row pointer table, with scale 1/sqrt(d_state); the update read as the
 * published gated delta rule).  Per row b and value head h, with state S [d_v][d_k] fp32:
 *   S' = exp(g) S;  S_new = S' + beta (v - S' k) k^T;  o = scale S_new q.
 * q, k, v, o: fp32 [B][n_heads][d_state] (q and k as the prep step leaves them, e.g.
 * L2-normalised); g (log decay) and beta: fp32 [B][n_heads].  state_in[b] / state_out[b]:
 * host arrays of device pointers to fp32 [n_heads][d_state][d_state] (row-major [v][k]);
 * state_out[b] may equal state_in[b] (in place) but no row may write a state another row
 * reads or writes.  d_state must be 128; 1 <= B <= 16. */
kd_status kd_gdn_step(const float* q, const float* k, const float* v, const float* g, const float* beta,
                      int32_t B, int32_t n_heads, int32_t d_state, const void* const* state_in,
                      void* const* state_out, float scale, float* o, void* stream);

/* ---- whole step ---------------------------------------------------------------------- */
typedef struct {
  const float* attn_norm;   /* [d] */
  kd_weight wqkv;           /* [(H + 2G) hd, d]: rows q (H hd), then k (G hd), then v (G hd) */
  int32_t wqkv_pair_rows;   /* 1: within each head the packed rows are in RoPE pair order --
                               packed row 2i is row i, packed row 2i + 1 is row i + hd/2
                               (i < hd/2) -- so every 16-row tile holds 8 whole pairs and the
                               product itself rotates q and k and stores k and v in the caches;
                               0: canonical order (a separate RoPE + append launch) */
  kd_weight wo;             /* [d, H hd] */
  const float* ffn_norm;    /* [d]; NULL for an attention-only layer */
  kd_weight w_gate, w_up;   /* dense SwiGLU [F, d] (qs NULL if MoE or attention-only); or w_gate
                               holding [2F, d] with w_up.qs NULL, rows interleaved in blocks of
                               32 -- packed rows 64m .. 64m+31 are gate rows 32m .. 32m+31 and
                               packed rows 64m+32 .. 64m+63 the same up rows (F % 32 == 0) --
                               so one product streams both and applies SwiGLU and the
                               activation quantiser to its own output */
  kd_weight w_down;         /* [d, F] */
  const float* router;      /* MoE: fp32 [E][d] */
  kd_weight e_gate, e_up;   /* MoE: experts stacked by rows, expert e = rows [e Fe, (e+1) Fe) of [E Fe, d];
                               or e_gate alone holding [E 2Fe, d] with e_up.qs NULL: expert e =
                               rows [e 2Fe, (e+1) 2Fe), its gate and up interleaved in blocks of
                               32 rows as w_gate above (Fe % 32 == 0), so one grouped product
                               per layer applies SwiGLU and quantises for e_down */
  kd_weight e_down;         /* MoE: expert e = rows [e d, (e+1) d) of [E d, Fe] */
  kd_weight s_gate, s_up;   /* MoE shared expert [Fs, d]; or s_gate alone holding [2Fs, d]
                               interleaved as w_gate, with s_up.qs NULL */
  kd_weight s_down;         /* [d, Fs] */
  int32_t swa_window;       /* sliding-window attention (memra-engine decode_batch.rs, the SWA
                               view of the Full-attention walk): 0 = every key; W > 0: a row
                               whose cache holds len = pos + 1 > W keys after its append attends
                               keys [len - W, len) only, as a view of its cache at that offset
                               (keys keep their absolute rotation) */
  const float* q_norm;      /* QK-norm (memra-engine decode_batch.rs, the QK-norm arm of the
                               Full-attention walk): NULL, or per-head gains [hd] -- each query
                               head is RMS-normalised over its hd values (with rms_eps) and
                               scaled by the gains before RoPE; needs wqkv_pair_rows == 0 */
  const float* k_norm;      /* the same for every key head (NULL when q_norm is NULL) */
  int32_t attn_gate;        /* attention output gate (memra-engine decode_batch.rs, the gated
                               Full-attention arm): 1 = wqkv holds H hd more rows after v, the
                               gate (in RoPE pair order too when wqkv_pair_rows = 1), and every
                               attention output element is multiplied by sigmoid(gate) before
                               wo; 0 = no gate */
  /* Linear-attention layers (memra-engine decode_batch.rs, the Linear mixer of
   * decode_batch_layers: batched projections, the fused conv ring, the prep, one batched scan
   * of the gated delta rule over every row's state, the gated norm, the out projection).
   * mixer = 1 replaces the attention of this layer: wqkv is the input projection
   * [C + d_v + 2 n_v, d] (canonical layout, wqkv_pair_rows = 0) whose rows are the conv
   * channels C = 2 d_state n_k + d_v (q of the n_k key heads, k of them, v of the n_v value
   * heads), then z (d_v = d_state n_v), then beta_raw (n_v), then alpha (n_v); wo is the out
   * projection [d, d_v].  Per row and value head h (key head h / (n_v / n_k)): each conv
   * channel c becomes silu(sum_j ssm_conv[c][j] w_j) over the window w of the row's last
   * d_conv inputs of that channel, oldest first; q and k are L2-normalised over the head
   * (x / sqrt(sum x^2 + rms_eps)); beta = sigmoid(beta_raw); g = ssm_a[h] softplus(alpha +
   * ssm_dt[h]); then the kd_gdn_step update with scale 1 / sqrt(d_state); the head's output o
   * becomes o / sqrt(mean(o^2) + rms_eps) ssm_norm silu(z), quantised for wo.  The attention
   * fields (q_norm, swa_window, attn_gate) must be 0 for such a layer. */
  int32_t mixer;            /* 0 attention, 1 gated delta-rule linear attention */
  const float* ssm_conv;    /* [C][d_conv] fp32 */
  const float* ssm_dt;      /* [n_v] fp32 */
  const float* ssm_a;       /* [n_v] fp32 (negative decay rates) */
  const float* ssm_norm;    /* [d_state] fp32 */
} kd_layer_desc;

typedef struct {
  int32_t n_layers, d, n_head, n_head_kv, head_dim;
  int32_t ffn;                           /* dense SwiGLU width, 0 if none */
  int32_t n_experts, n_expert_used;      /* 0 = dense */
  int32_t expert_ffn, shared_ffn;
  int32_t vocab;                         /* lm_head rows, 0 = none */
  float rope_base, rms_eps;
  const kd_layer_desc* layers;           /* host array [n_layers] (copied by kd_model_create) */
  const float* final_norm;               /* [d] or NULL */
  kd_weight lm_head;                     /* [vocab, d] or qs NULL */
  int32_t ssm_d_state, ssm_n_k, ssm_n_v, ssm_d_conv;  /* linear layers: d_state (128), key and value
                                            heads (n_v a multiple of n_k), conv width (2..8) */
  int32_t kv_format;                     /* KD_KV_F16 (fp16 caches, k_base/v_base [G][capacity][hd]
                                            fp16), KD_KV_FP8_E4M3 (uint8 codes, stored and read as
                                            kd_kv_append_fp8 / kd_fa_decode_ragged_fp8, by either
                                            wqkv layout) or KD_KV_Q8_0 (int8 rows [G][capacity][hd + 16],
                                            as kd_kv_append_q8 / kd_fa_decode_ragged_q8; a block of
                                            32 spans one head's rows across workgroups of the fused
                                            RoPE epilogue, so these models need wqkv_pair_rows = 0) */
} kd_model_desc;

typedef struct kd_model kd_model;

/* Validate a descriptor and keep a host copy of it (device pointers are borrowed, not
 * owned).  The model is immutable and may be shared across threads and streams. */
kd_status kd_model_create(const kd_model_desc* desc, kd_model** out);
void kd_model_destroy(kd_model* m);

/* Workspace bytes of kd_decode_step for B rows with these positions (host pos[B]). */
size_t kd_decode_step_workspace(const kd_model* m, int32_t B, const int32_t* pos);
/* Bytes of one row's recurrent state of one linear layer (0 if the model has none): fp32,
 * 16-byte aligned, laid out as ring 0 [d_conv - 1][C], ring 1 (the same), state 0
 * [n_v][d_state][d_state] (row-major [v][k], as kd_gdn_step), state 1 (the same).  A step at
 * position pos reads ring and state pos % 2 and writes the other ones, so the state before the
 * step stays readable (a step can be redone, or rolled back by one position).  The caller
 * places a row's state after pos = p tokens in ring/state p % 2 before its first step. */
size_t kd_recurrent_state_bytes(const kd_model* m);

/* One decode step for B rows: x_in fp32 [B][d]; row b writes K/V at pos[b] of its caches
 * and attends pos[b] + 1 keys; all appends of a layer precede its attention, so rows that
 * share a cache at consecutive positions (speculative-verify rows) attend causally.
 * k_base / v_base: host arrays [n_layers][B] of cache base addresses; for a linear layer
 * k_base[l][b] is row b's recurrent state (kd_recurrent_state_bytes; no two rows may share
 * one) and v_base[l][b] is not read.  out: fp32
 * [B][vocab] logits if the model has an lm_head, else [B][d] (output-normed if final_norm).
 * x_in and out must be 16-byte aligned (rows are read and written four floats at a time);
 * KD_ERR_INVALID otherwise.  Positions are not advanced: the caller owns session state (memra-engine
 * decode_batch.rs ``decode_batch_epilogue`` advances pos after the step). */
kd_status kd_decode_step(const kd_model* m, int32_t B, const float* x_in, const int32_t* pos,
                         void* const* k_base, void* const* v_base, int32_t capacity, float* out,
                         void* ws, size_t ws_bytes, void* stream);

/* What one step leaves behind layer by layer (tests only: teacher-forced per-layer
 * comparison, each layer checked against a reference fed this step's own layer input and,
 * where the activation quantiser rounds, its own integer decisions).  Device pointers, each
 * NULL or:
 *   resid   fp32 [n_layers + 1][B][d]: the residual rows entering layer l (l < n_layers),
 *           then the residual rows after the last layer (before the output norm);
 *   moe_ids int32 [n_layers][B][n_expert_used]: the experts each row is routed to in an MoE
 *           layer, by descending router logit (ties to the lower id);
 *   moe_p   fp32 [n_layers][B][n_expert_used]: their softmax weights, in the same order;
 *   the int8 codes of every activation quantisation, in the tiled activation layout (rows of
 *   NQ(k) * 128 bytes, NQ(k) = ceil(k / 128)), per layer:
 *   q_attn_in  [n_layers][B][NQ(d) 128]      the normed attention input (the q/k/v product's);
 *   q_attn_out [n_layers][B][NQ(max(H hd, d_v)) 128]  the attention output, or a linear layer's
 *              gated-norm output (the o / out product's input; its first NQ(k) 128 bytes);
 *   q_ffn_in   [n_layers][B][NQ(d) 128]      the normed FFN input;
 *   q_ffn_mid  [n_layers][R][NQ(F) 128]      silu(gate) up, the down product's input: dense
 *              layers R = B rows of F = ffn; MoE layers R = B n_expert_used (row, rank) rows of
 *              F = expert_ffn, row b K + rank;
 *   q_shared_mid [n_layers][B][NQ(shared_ffn) 128]  the shared expert's (MoE layers);
 *   q_head_in  [B][NQ(d) 128]                the output-normed rows entering the lm_head.
 * Entries of layers without experts are left untouched. */
typedef struct {
  float* resid;
  int32_t* moe_ids;
  float* moe_p;
  int8_t* q_attn_in;
  int8_t* q_attn_out;
  int8_t* q_ffn_in;
  int8_t* q_ffn_mid;
  int8_t* q_shared_mid;
  int8_t* q_head_in;
} kd_step_trace;

/* ---- next token: greedy argmax and embedding gather ----------------------------------- */
/* Greedy token of each row (memra-engine decode_batch.rs, ``decode_step_batch_sampled``:
 * the device argmax of each greedy row's logits, equal to the host argmax).  x: device fp32
 * [B][ldx], the first n entries of each row are its logits.  idx[b] (device int32) = the
 * lowest j < n with x[b][j] = max_j x[b][j] (ties go to the lower index); val[b] (device fp32,
 * may be NULL) = that maximum.  NaN entries never win; a row of NaN only gives index 0 and
 * value NaN.  The result is exact (comparisons only) and each row is independent of the
 * others.  1 <= B <= 65535, n >= 1, ldx >= n. */
kd_status kd_argmax_rows(const float* x, int32_t B, int32_t n, int32_t ldx, int32_t* idx, float* val,
                         void* stream);
/* The next step's input rows from tokens (memra-engine decode_batch.rs, phase 0 of
 * ``decode_step_batch``: each row starts from its token's embedding row):
 * out[b][0:d] = table[tokens[b]][0:d].  table: device fp32 [vocab][d]; tokens: device int32
 * [B] (e.g. kd_argmax_rows' idx, so the token never visits the host); out: device fp32 [B][ldo].
 * A token outside [0, vocab) gives a zero row and reads nothing.  1 <= B <= 65535, ldo >= d. */
kd_status kd_embed_rows(const float* table, int32_t vocab, int32_t d, const int32_t* tokens, int32_t B,
                        float* out, int32_t ldo, void* stream);

/* Accepted prefix of speculative-verify rows (Strata PR #1524, "What changes": target
 * verification of several streams' drafts in one step, with accepted-prefix state commits).
 * Rows are stream-major, k per stream: fed[s k + j] is the token that row j of stream s took
 * as input (j = 0: the stream's last committed token; j >= 1: its draft j), at position
 * pos_s + j, and greedy[s k + j] is that row's greedy token (kd_argmax_rows).  Writes
 * n_accept[s] = the largest a <= k - 1 with greedy[s k + j - 1] == fed[s k + j] for every
 * 1 <= j <= a, and next_token[s] = greedy[s k + a] (the target's token after the kept
 * prefix).  All arrays are device int32.  Commit: the caller sets pos_s += a + 1 and feeds
 * next_token[s]; cache slots past the new pos_s hold rejected rows' K/V and are rewritten by
 * later steps before any row attends them.  1 <= n_streams, n_streams k <= 16. */
kd_status kd_verify_accept(const int32_t* greedy, const int32_t* fed, int32_t n_streams, int32_t k,
                           int32_t* n_accept, int32_t* next_token, void* stream);

/* ---- test exports ---------------------------------------------------------------------- */
/* The exact int32 block dot products S[b][n][blk] (b < B, n < n_out, blk < k/32) that the
 * mmvq kernel computes for this matrix and activation (same kernel, epilogue replaced).
 * Q8_0 and Q4_0 only (KD_ERR_UNSUPPORTED for the K-quant formats). */
kd_status kd_debug_block_dots(const kd_weight* W, kd_act_q8 x, int32_t B, int32_t* S, void* stream);
/* kd_fa_decode_ragged with a forced chunk size (keys per split, >= 1) for split-invariance
 * tests; the workspace must hold ceil(t_b / chunk) splits per row. */
size_t kd_debug_fa_workspace(int32_t B, int32_t H, int32_t hd, const int32_t* t_kv, int32_t chunk);
kd_status kd_debug_fa_decode_chunked(const float* q, int32_t B, int32_t H, int32_t G, int32_t hd,
                                     const void* const* k_base, const void* const* v_base,
                                     const int32_t* t_kv, int32_t capacity, float scale, float* out,
                                     int32_t chunk, void* ws, size_t ws_bytes, void* stream);

/* kd_decode_step, computing exactly the same (same launches, same outputs and cache bytes),
 * that also copies the per-layer record above into *trace on the same stream (device-to-
 * device copies, plus one residual add after the last layer).  memra-engine decode_batch.rs
 * exactness contract: each layer of the batched walk must match its reference; this export
 * lets a test compare every layer against the oracle given the GPU's own layer input. */
kd_status kd_debug_decode_step_trace(const kd_model* m, int32_t B, const float* x_in, const int32_t* pos,
                                     void* const* k_base, void* const* v_base, int32_t capacity, float* out,
                                     void* ws, size_t ws_bytes, const kd_step_trace* trace, void* stream);

/* The routing of one MoE layer for B rows (tests only; the kernels kd_decode_step runs for
 * an MoE layer, hf2q ADR-040 §0.7 F4: per-token top-k routing; rows grouped by expert).
 * Device pointers: z fp32 [B][d] (the FFN-normed rows), router fp32 [E][d].  Writes
 * logits fp32 [B][E] = router z (fp32, a fixed order per d); ids int32 [B][K] = the K
 * largest logits' experts by descending logit, ties to the lower id; p fp32 [B][K] =
 * softmax over those K logits, in the same order; and the buckets: count int32 [E] = the
 * (row, rank) pairs routed to expert e, rows / pairs int32 [E][16] = their row b and pair
 * index b K + rank, in ascending row order (entries past count[e] untouched).
 * 1 <= B <= 16, 1 <= K <= min(E, 16), E <= 256, d % 4 == 0. */
kd_status kd_debug_moe_route(const float* z, const float* router, int32_t B, int32_t d, int32_t E, int32_t K,
                             int32_t* ids, float* p, float* logits, int32_t* count, int32_t* rows, int32_t* pairs,
                             void* stream);
/* The grouped product kd_decode_step runs over those buckets (tests only; hf2q ADR-040 §0.7
 * F4: each active expert's matrices read once and applied to every row routed to it).  W
 * is group 0 of n_groups stacked groups of W->n_out rows each (W->n_out % 16 == 0, tiled
 * as one [n_groups n_out, k] matrix).  For group e, its j-th row (j < count[e] <= 16)
 * multiplies activation row act_row[e][j] of x (act_rows rows) and its result goes to
 * output row out_row[e][j]; a group with count 0 reads nothing.  count [n_groups] and
 * act_row / out_row [n_groups][16] are device int32 arrays whose entries the caller keeps in
 * range (act_row < act_rows; out_row < the output's rows).  swiglu = 0: y fp32 rows (stride
 * ldy >= n_out) as kd_mmvq_q8_0 / _q4_0 give them; swiglu = 1: each group is an interleaved
 * gate/up block [2F, k] and out receives the quantised silu(gate) up rows as kd_mmvq_swiglu
 * writes them.  Each output row equals, bit for bit, the plain product of its group's rows
 * with its activation row alone. */
kd_status kd_debug_mmvq_grouped(const kd_weight* W, int32_t n_groups, kd_act_q8 x, int32_t act_rows,
                                const int32_t* count, const int32_t* act_row, const int32_t* out_row, int32_t swiglu,
                                float* y, int32_t ldy, kd_act_q8 out, void* stream);

/* A plain read of `bytes` bytes at p (device, 16-byte aligned, bytes % 16 == 0) with wide
 * non-temporal loads and no arithmetic (measurement only: the practical HBM read ceiling the
 * products and the attention are compared with).
 * sink: a device uint32 that is written only in the rare case the loaded words fold to a
 * fixed constant. */
kd_status kd_debug_read_stream(const void* p, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KD_H */
